#!/usr/bin/env python3
"""Throughput of the single-GPU MoE-layer forward pass on MI355X.

One step = the whole layer on one batch: router GEMM + top-K gating, permute
into expert segments, grouped gate/up GEMM with SwiGLU, grouped down GEMM,
unpermute + weighted combine -- the five libmoe calls moe_forward is made of,
issued separately so that every stage, and the dominant kernel (the gate/up
grouped GEMM), can be bracketed with HIP events on the stream it runs on.
Inputs are synthetic, seeded and already resident in HBM when timing starts.

Timing: W untimed warm-up steps, then K timed steps.  Before every timed step
512 MiB of scratch are written and then read back outside its events (twice
the 256 MB memory-side cache): no activation or weight of the previous step is
still cached, and the caches hold clean lines, so the step pays for no
write-back of the flush's own data.  The K cold steps run twice: first as the
five library calls issued one by one (``eager_ms_per_step``; HIP events
between the calls give the stage times), then as one HIP graph of those same
calls captured once and replayed (``graph_ms_per_step``, whose y must equal
the eager steps' bit for bit).  ``ms_per_step`` is the graph's mean (the
eager one with ``--eager``).  More steps run back to back afterwards and give
``warm_ms_per_step``.

The headline workload is the DeepSeek-V3 layer shape (N=8192, D=7168,
E=256, K=8, F=2048, sigmoid gating).  The other workloads -- the Qwen3 decode
step, the hot-expert skew (contiguous and capacity-padded) and the Mixtral
shape -- run after it in the same process and are reported under
``workloads``, each with its own roofline of its dominant kernel.
``cpu_baseline`` is the C++ oracle on a bounded sample of the headline
workload's tokens, on the host's cores.

The expert weights are the nn.Linear bf16 stacks, read in place.
``--weights packed`` times the same values packed once by moe_pack_weights
(the order the GEMMs stream them; outputs bit for bit those of the unpacked
calls), ``--weights fp8`` block-scaled FP8 copies, ``--weights fp8packed``
those with their codes packed by moe_pack_weights_fp8.  ``--config gelu_mlp``
runs the pages' other layer (MLP router, GELU experts); ``--fused`` runs the
expert FFN as one persistent launch.

Also: ``--trace-summary DIR`` and ``--pmc-summary ...`` turn rocprofv3 output
of a profiled run of this script into the tables kept under profiles/.

Prints one JSON line.  ``value`` is tokens/s of the headline layer on this GPU.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
ROOT = os.path.dirname(os.path.abspath(__file__))
GEMM_SRC = os.path.join(ROOT, "mixture_experts_layer_level_amd", "csrc", "grouped_gemm.hip")
FLUSH_BYTES = 512 << 20
DEFAULT_EXTRA = "qwen3_decode,qwen3_decode:packed,hot_skew,hot_skew:padded,mixtral"
# tokens of the CPU-oracle sample per workload (about 10-30 s of CPU work on
# 16 host cores for the C++ oracle)
CPU_TOKENS = {"deepseek_v3": 2048, "mixtral": 512, "hot_skew": 1024, "qwen3_decode": 64,
              "tiny": 64, "gelu_mlp": 256, "gelu_tiny": 64}


def source_sha() -> str:
    return hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per gate/up launch from the committed rocprofv3 --pmc summary
    of this workload, or None when there is none or the kernel source has
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    rec = None
    for line in open(path, encoding="utf-8"):
        if line.startswith("traffic: "):
            rec = json.loads(line[len("traffic: "):])
    if rec is None:
        return None
    return rec["bytes"] if rec.get("source_sha256") == source_sha() else None


def roofline(flop, nbytes, ms):
    """Bound of a kernel from its algorithmic work, and what it achieved."""
    t_mfma = flop / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBPS * 1e9)
    if t_mfma >= t_hbm:
        r = {"bound": "mfma", "achieved": flop / (ms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
             "unit": "TFLOP/s"}
    else:
        r = {"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBPS,
             "unit": "GB/s"}
    r["frac"] = r["achieved"] / r["peak"]
    return r


class Opts:
    def __init__(self, padded=False, fused=False, xperm=False, weights="bf16", graph=True):
        self.padded, self.fused, self.xperm, self.weights = padded, fused, xperm, weights
        self.graph = graph


def run_layer(cfg, o: Opts, steps: int, warmup: int, warm_steps: int, log):
    """Build the layer's inputs on the GPU, time it, return (result dict,
    inputs).  The result holds the cold step time, the warm one, the stage
    times and the roofline of the dominant kernel."""
    import numpy as np
    import torch

    import mixture_experts_layer_level_amd as moe
    import moe_synth as ms

    dev = "cuda"
    cap = cfg.capacity if o.padded else None
    if o.padded and cap is None:
        raise SystemExit(f"{cfg.name} has no capacity factor")
    gelu = cfg.expert == "gelu"
    if o.fused and (gelu or o.weights != "bf16" or o.padded):
        raise SystemExit("--fused runs the SwiGLU layer, bf16 weights, contiguous layout")
    if gelu and o.weights != "bf16":
        raise SystemExit("the GELU-expert layer runs with bf16 weights")
    t0 = time.time()
    inp = ms.make_gelu_inputs(cfg, device=dev) if gelu else ms.make_inputs(cfg, device=dev)
    torch.cuda.synchronize()
    log(f"inputs {cfg.name} generated in {time.time() - t0:.1f}s")
    p = moe.problem(cfg.N, cfg.D, cfg.F, cfg.E, cfg.K, cfg.gating, cap)
    R, capv = moe.permuted_rows(p)
    N, D, E, K, F = cfg.N, cfg.D, cfg.E, cfg.K, cfg.F
    e = lambda *s, dt=torch.float32: torch.empty(*s, dtype=dt, device=dev)
    logits, ids, w = e(N, E), e(N, K, dt=torch.int32), e(N, K)
    counts, offsets = e(E, dt=torch.int32), e(E + 1, dt=torch.int32)
    row_token, slot_row = e(R, dt=torch.int32), e(N * K, dt=torch.int32)
    h = e(R, F, dt=torch.bfloat16)
    out_perm, y = e(R, D, dt=torch.bfloat16), e(N, D, dt=torch.bfloat16)
    ws = torch.empty(moe.workspace_size(p), dtype=torch.uint8, device=dev)
    x = inp["x"]
    if gelu:
        feats = e(N, D // 4, dt=torch.bfloat16)
    else:
        wr, bias = inp["w_router"], inp["bias"]
        wg, wu, wd = inp["w_gate"], inp["w_up"], inp["w_down"]
    stream = torch.cuda.current_stream()
    fp8 = o.weights in ("fp8", "fp8packed")
    fp8p = o.weights == "fp8packed"
    if fp8:
        def quant(wt):
            rows, cols = wt.shape[-2], wt.shape[-1]
            c = torch.empty(wt.shape, dtype=torch.uint8, device=dev)
            sc = torch.empty(wt.shape[0], rows // 32, cols // 32, 32, dtype=torch.uint8,
                             device=dev)
            moe.quantize_fp8(wt.numel() // cols, cols, wt, c, sc, stream=stream)
            return c, sc
        qg, qu, qd = quant(wg), quant(wu), quant(wd)
        if fp8p:
            # the codes in the library's packed stage-image order (scales as they are)
            def pack8(kind, c0, c1=None):
                buf = torch.empty(moe.packed_weight_size(p, kind), dtype=torch.uint8, device=dev)
                moe.pack_weights_fp8(p, kind, c0, c1, buf, stream=stream)
                return buf
            pgu8 = pack8(moe.PACK_GATEUP_FP8, qg[0], qu[0])
            pdn8 = pack8(moe.PACK_DOWN_FP8, qd[0])
        torch.cuda.synchronize()
    packed = o.weights == "packed"
    if packed:
        # the same bf16 weights in the library's packed stage-image order
        def pack(kind, w0, w1=None):
            buf = torch.empty(moe.packed_weight_size(p, kind) // 2, dtype=torch.bfloat16,
                              device=dev)
            moe.pack_weights(p, kind, w0, w1, buf, stream=stream)
            return buf
        pgu, pdn = pack(moe.PACK_GATEUP, wg, wu), pack(moe.PACK_DOWN, wd)
        torch.cuda.synchronize()

    # The first expert GEMM reads its rows of x through row_token wherever the
    # library takes the shape; it refuses, before any launch, the shapes whose
    # tiles have no gathered form.  The trial call runs one whole step.
    gather = not (o.xperm or o.fused or capv)
    x_perm = None if gather else e(R, D, dt=torch.bfloat16)

    def rec(ev, i):
        if ev is not None:
            ev[i].record(torch.cuda.current_stream())

    def gateup():
        if gelu:
            if gather:
                moe.expert_up_gelu_gathered(p, x, row_token, offsets, inp["w1"], inp["b1"], h,
                                            stream=torch.cuda.current_stream())
            else:
                moe.expert_up_gelu(p, x_perm, offsets, inp["w1"], inp["b1"], h, stream=torch.cuda.current_stream())
        elif gather and fp8p:
            moe.expert_gateup_fp8_packed_gathered(p, x, row_token, offsets, pgu8, qg[1], qu[1], h,
                                                  stream=torch.cuda.current_stream())
        elif fp8p:
            moe.expert_gateup_fp8_packed(p, x_perm, offsets, pgu8, qg[1], qu[1], h,
                                         stream=torch.cuda.current_stream())
        elif gather and fp8:
            moe.expert_gateup_fp8_gathered(p, x, row_token, offsets, qg, qu, h, stream=torch.cuda.current_stream())
        elif gather and packed:
            moe.expert_gateup_packed_gathered(p, x, row_token, offsets, pgu, h,
                                              stream=torch.cuda.current_stream())
        elif packed:
            moe.expert_gateup_packed(p, x_perm, offsets, pgu, h, stream=torch.cuda.current_stream())
        elif gather:
            moe.expert_gateup_gathered(p, x, row_token, offsets, wg, wu, h, stream=torch.cuda.current_stream())
        elif fp8:
            moe.expert_gateup_fp8(p, x_perm, offsets, qg, qu, h, stream=torch.cuda.current_stream())
        else:
            moe.expert_gateup(p, x_perm, offsets, wg, wu, h, stream=torch.cuda.current_stream())

    # ev: six events per step, recorded on the launch stream before the route
    # and after the route, permute, gate/up (or fused FFN), down and combine
    def step(ev=None):
        rec(ev, 0)
        if gelu:
            moe.route_mlp(p, x, inp["w_proj"], inp["b_proj"], inp["w_out"], inp["b_out"],
                          logits, ids, w, ws, features=feats, stream=torch.cuda.current_stream())
        else:
            moe.route(p, x, wr, bias, logits, ids, w, ws, stream=torch.cuda.current_stream())
        rec(ev, 1)
        moe.permute(p, x, ids, counts, offsets, row_token, slot_row,
                    None if (gather or o.fused) else x_perm, ws, stream=torch.cuda.current_stream())
        rec(ev, 2)
        if o.fused:
            moe.fused_ffn(p, x, row_token, offsets, wg, wu, wd, out_perm, ws, stream=torch.cuda.current_stream())
            rec(ev, 3)
        else:
            gateup()
            rec(ev, 3)
            if gelu:
                moe.expert_down_bias(p, h, offsets, inp["w2"], inp["b2"], out_perm,
                                     stream=torch.cuda.current_stream())
            elif fp8p:
                moe.expert_down_fp8_packed(p, h, offsets, pdn8, qd[1], out_perm,
                                           stream=torch.cuda.current_stream())
            elif fp8:
                moe.expert_down_fp8(p, h, offsets, qd, out_perm, stream=torch.cuda.current_stream())
            elif packed:
                moe.expert_down_packed(p, h, offsets, pdn, out_perm,
                                       stream=torch.cuda.current_stream())
            else:
                moe.expert_down(p, h, offsets, wd, out_perm, stream=torch.cuda.current_stream())
        rec(ev, 4)
        moe.unpermute_combine(p, out_perm, slot_row, w, y, stream=torch.cuda.current_stream())
        rec(ev, 5)

    if gather:
        try:
            step()
        except moe.MoEError as err:
            if err.status != 2:   # MOE_ERR_UNSUPPORTED: run the permuted copy instead
                raise
            gather = False
            x_perm = e(R, D, dt=torch.bfloat16)
            step()
    else:
        step()
    torch.cuda.synchronize()
    pre_steps = 1 + warmup            # whole steps before the timed ones (for trace summaries)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # timed: every step cold, each preceded by a 512 MiB scratch write and a
    # read of it, outside its events
    scratch = torch.empty(FLUSH_BYTES // 8, dtype=torch.int64, device=dev)
    sink = torch.empty((), dtype=torch.int64, device=dev)

    def flush():
        scratch.zero_()
        torch.sum(scratch, dim=0, out=sink)

    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(6)) for _ in range(steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(steps):
        flush()
        step(evs[i])
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall

    def check_fused(when, whole_layer):
        # the error word of moe_fused_ffn (staged) or moe_forward_fused (whole
        # layer), at its offset in the workspace
        if o.fused:
            off = moe.fused_error_offset(p, whole_layer=whole_layer)
            err_word = int(ws[off:off + 4].view(torch.int32).item())
            if err_word != 0:
                raise SystemExit(f"fused FFN: a bounded wait ran out during the {when} "
                                 f"(error word {err_word}); its results are wrong")
    check_fused("timed steps", False)

    # The layer as the library's one-call forward (moe_forward, or its FP8,
    # fused or GELU form), captured once as a HIP graph (the library allocates
    # nothing and issues no memset or host synchronisation) and replayed cold
    # like the eager steps.  It computes the same sums in the same order as
    # the staged calls: y of the replays must equal y of the eager steps bit
    # for bit.  (--xperm: the staged calls themselves, since moe_forward
    # skips the permuted copy wherever it can.)
    def layer():
        s_ = torch.cuda.current_stream()
        if o.xperm:
            step()
        elif o.fused:
            moe.forward_fused(p, x, wr, bias, wg, wu, wd, y, ws, stream=s_)
        elif gelu:
            moe.forward_gelu(p, x, inp["w_proj"], inp["b_proj"], inp["w_out"], inp["b_out"],
                             inp["w1"], inp["b1"], inp["w2"], inp["b2"], y, ws, stream=s_)
        elif fp8p:
            moe.forward_fp8_packed(p, x, wr, bias, pgu8, qg[1], qu[1], pdn8, qd[1], y, ws,
                                   stream=s_)
        elif fp8:
            moe.forward_fp8(p, x, wr, bias, qg, qu, qd, y, ws, stream=s_)
        elif packed:
            moe.forward_packed(p, x, wr, bias, pgu, pdn, y, ws, stream=s_)
        else:
            moe.forward(p, x, wr, bias, wg, wu, wd, y, ws, stream=s_)

    graph_ms = None
    post_steps = 0
    if o.graph:
        y_eager = y.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer()
        torch.cuda.synchronize()
        y.zero_()
        for _ in range(2):
            g.replay()
        gevs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2))
                for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            flush()
            gevs[i][0].record(stream)
            g.replay()
            gevs[i][1].record(stream)
        torch.cuda.synchronize()
        graph_ms = sum(a_.elapsed_time(b_) for a_, b_ in gevs) / steps
        if not torch.equal(y.view(torch.int16), y_eager.view(torch.int16)):
            raise SystemExit(f"{cfg.name}: y of the graph replays differs from the eager "
                             f"staged steps")
        check_fused("graph replays", True)
        post_steps = 2 + steps
        del y_eager
    del scratch, sink

    def stage_ms(i, j):
        return sum(ev[i].elapsed_time(ev[j]) for ev in evs) / steps
    per_step = sorted(ev[0].elapsed_time(ev[5]) for ev in evs)
    ms_step = sum(per_step) / steps
    route_ms, permute_ms = stage_ms(0, 1), stage_ms(1, 2)
    gateup_ms, down_ms, combine_ms = stage_ms(2, 3), stage_ms(3, 4), stage_ms(4, 5)

    warm_ms = None
    if warm_steps > 0:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(warm_steps):
            if o.graph:
                g.replay()
            else:
                step()
        b.record(stream)
        torch.cuda.synchronize()
        warm_ms = a.elapsed_time(b) / warm_steps
        post_steps += warm_steps
        check_fused("warm steps", o.graph)
    eager_ms = ms_step
    if graph_ms is not None:
        ms_step = graph_ms

    counts_h = counts.cpu().numpy().astype(np.int64)
    kept = int(np.minimum(counts_h, capv).sum()) if capv else cfg.S
    touched = int((counts_h > 0).sum())
    wb = (1.0 + 1.0 / 32) if fp8 else 2.0          # weight bytes per element (FP8: + scales)
    nmat = 2 if gelu else 3                        # expert matrices
    if gelu:   # MLP router + Linear-GELU-Linear experts, kept slots
        flops = 2.0 * N * (D * (D // 4) + (D // 4) * E) + 4.0 * D * F * kept
    else:      # router + SwiGLU FFN, kept slots
        flops = 2.0 * N * D * E + 6.0 * D * F * kept
    tflops = flops / (ms_step * 1e-3) / 1e12
    weight_bytes = nmat * touched * F * D * wb
    # dominant kernel: the gate/up grouped GEMM (the GELU experts' up GEMM),
    # algorithmic work per launch: touched experts' weights once, the kept
    # rows of x read once, h written once
    gu_mats = nmat - 1
    gu_flops = 2.0 * gu_mats * D * F * kept
    gu_bytes = gu_mats * touched * F * D * wb + kept * D * 2 + kept * F * 2
    suffix = ("_padded" if capv else "") + ("_fp8" if fp8 else "") + \
        ("_packed" if packed or fp8p else "") + ("_xperm" if o.xperm else "")
    if o.fused:
        # the one fused launch: gate/up, SwiGLU and down of every expert
        f_flops = 6.0 * D * F * kept
        f_bytes = 3.0 * touched * F * D * 2 + kept * D * 2 * 2 + kept * F * 2 * 2
        roof = roofline(f_flops, f_bytes, gateup_ms)
        roof["traffic"] = measured_traffic(cfg.name + "_fused")
        roof["kernel"] = "fused expert FFN (gate/up + SwiGLU + down, one launch)"
        roof["algorithmic"] = {"flop": f_flops, "bytes": f_bytes}
    else:
        roof = roofline(gu_flops, gu_bytes, gateup_ms)
        roof["traffic"] = measured_traffic(cfg.name + suffix)
        roof["kernel"] = (("grouped up GEMM + bias + GELU" if gelu
                           else "grouped gate/up GEMM + SwiGLU") +
                          (", rows gathered from x through row_token" if gather else ""))
        roof["algorithmic"] = {"flop": gu_flops, "bytes": gu_bytes,
                               "per_unit": "per kept slot: %d flop, %d bytes of its row and h; "
                                           "per touched expert: %d weight bytes"
                                           % (2 * gu_mats * D * F, D * 2 + F * 2,
                                              gu_mats * F * D * wb)}
    roof["avg_ms"] = gateup_ms
    # the HBM-bound stages against 8 TB/s: permute (x read once and x_perm
    # rows written, when the copy is made; ids read, row_token and slot_row
    # written, offsets), combine (kept out_perm rows read, y written,
    # slot_row and weights read)
    S_ = N * K
    perm_bytes = (S_ * 4 * 3 + (E + 1) * 4 +
                  (0 if (o.fused or gather) else N * D * 2 + R * D * 2))
    comb_bytes = kept * D * 2 + N * D * 2 + S_ * 8
    stages = {
        "route_ms": route_ms, "permute_ms": permute_ms, "gateup_ms": gateup_ms,
        "down_ms": down_ms, "ffn_ms": gateup_ms + down_ms, "combine_ms": combine_ms,
        "permute_gbps": perm_bytes / (permute_ms * 1e-3) / 1e9,
        "permute_frac_hbm": perm_bytes / (permute_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "combine_gbps": comb_bytes / (combine_ms * 1e-3) / 1e9,
        "combine_frac_hbm": comb_bytes / (combine_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "permute_bytes": perm_bytes, "combine_bytes": comb_bytes,
        "step_ms_min": per_step[0], "step_ms_median": per_step[len(per_step) // 2],
        "step_ms_max": per_step[-1],
    }
    if capv:   # the padded layout runs every expert over cap rows
        exec_flops = flops - (4.0 if gelu else 6.0) * D * F * kept + \
            (4.0 if gelu else 6.0) * D * F * E * capv
        stages["kept_slots"] = kept
        stages["utilisation"] = kept / (E * capv)
        stages["executed_tflops"] = exec_flops / (ms_step * 1e-3) / 1e12
    res = {
        "workload": cfg.note + (" [capacity-padded]" if capv else "") +
                    (" [packed weights]" if packed or fp8p else ""),
        "config": {"workload": cfg.note + (" [capacity-padded]" if capv else ""),
                   "tokens": N, "hidden": D, "experts": E, "top_k": K, "ffn": F,
                   "gating": cfg.gating, "capacity": capv or None,
                   "expert_weights": ("fp8 e4m3, power-of-two scale per 32 values" +
                                      (", codes packed as stage images" if fp8p else "")
                                      if fp8 else "bf16, packed stage images" if packed
                                      else "bf16"),
                   "expert": ("Linear-GELU-Linear with biases, MLP router" if gelu
                              else "SwiGLU"),
                   "launch": (("the five staged library calls" if o.xperm else
                               ("moe_forward_fused" if o.fused else
                                "moe_forward_gelu" if gelu else
                                "moe_forward_fp8_packed" if fp8p else
                                "moe_forward_fp8" if fp8 else
                                "moe_forward_packed" if packed else "moe_forward") +
                               " (one call)") +
                              " captured once as a HIP graph and replayed"
                              if o.graph else "the five staged library calls, eager"),
                   "ffn_launch": ("fused (one persistent launch)" if o.fused else
                                  "two grouped GEMMs, rows of the first gathered from x"
                                  if gather else "two grouped GEMMs")},
        "value": N / (ms_step * 1e-3),
        "unit": "tokens/s",
        "ms_per_step": ms_step,
        "warm_ms_per_step": warm_ms,
        "eager_ms_per_step": eager_ms,
        "graph_ms_per_step": graph_ms,
        "tflops": tflops,
        "pct_bf16_mfma_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "weight_stream_gbps": weight_bytes / (ms_step * 1e-3) / 1e9,
        "pct_hbm_peak_weights": 100.0 * weight_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "ffn_weight_stream_gbps": weight_bytes / ((gateup_ms + down_ms) * 1e-3) / 1e9,
        "max_expert_rows": int(counts_h.max()),
        "dropped_slots": int(cfg.S - kept),
        "stages": stages,
        "roofline": roof,
        "timed_wall_s": wall_s,
        # whole steps of this run before the eager timed ones, and after them
        # (graph replays and warm steps), for kernel-trace summaries
        "trace_layout": {"pre_steps": pre_steps, "timed_steps": steps,
                         "post_steps": post_steps},
    }
    log(f"{cfg.name}{suffix}: {ms_step:.3f} ms/step cold (eager {eager_ms:.3f}, warm "
        f"{warm_ms or 0:.3f}), gate/up {gateup_ms:.3f} ms, down {down_ms:.3f} ms")
    return res, inp


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warm-steps", type=int, default=None,
                    help="back-to-back steps after the timed cold ones (default: --steps; 0 = "
                         "none)")
    ap.add_argument("--config", default="deepseek_v3",
                    help="tiny | mixtral | deepseek_v3 | qwen3_decode | hot_skew | gelu_mlp | "
                         "gelu_tiny")
    ap.add_argument("--extra", default=DEFAULT_EXTRA,
                    help="workloads run after the headline one, reported under 'workloads' "
                         "(comma-separated, name[:padded]; 'none' for none)")
    ap.add_argument("--padded", action="store_true", help="capacity-padded layout (hot_skew)")
    ap.add_argument("--fused", action="store_true",
                    help="the expert FFN as one persistent launch (moe_fused_ffn; rows gathered "
                         "from x, no permuted copy)")
    ap.add_argument("--xperm", action="store_true",
                    help="write the permuted copy of x and run the first expert GEMM on it; by "
                         "default that GEMM reads its rows of x through row_token wherever the "
                         "library takes the shape")
    ap.add_argument("--eager", action="store_true",
                    help="time the eager steps only (by default the step is also captured as "
                         "a HIP graph and ms_per_step is the graph's cold replay)")
    ap.add_argument("--weights", choices=("bf16", "fp8", "packed", "fp8packed"),
                    default="bf16",
                    help="expert weight storage: bf16 stacks read in place (default), "
                         "block-scaled FP8 (E4M3 + E8M0), the same bf16 values packed as "
                         "the GEMMs' stage images, or the FP8 codes so packed (SwiGLU layers, "
                         "not with --fused)")
    ap.add_argument("--cpu-tokens", type=int, default=-1,
                    help="tokens of the CPU-oracle sample (-1: a per-workload default of about "
                         "10-30 s of CPU work; 0: skip the CPU baseline)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB, three "
                         "times (the reference kernel for HBM byte counters), then exit")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="only summarise the rocprofv3 kernel trace under DIR: per libmoe "
                         "kernel, the launches of the timed steps (after --pre-steps whole "
                         "steps, --steps of them); prints a markdown table")
    ap.add_argument("--pre-steps", type=int, default=None,
                    help="with --trace-summary: whole steps before the timed ones "
                         "(trace_layout.pre_steps of the profiled run)")
    ap.add_argument("--post-steps", type=int, default=None,
                    help="with --trace-summary: whole steps after the timed ones "
                         "(trace_layout.post_steps of the profiled run)")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR",
                                                       "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="only summarise four rocprofv3 --pmc runs (the workload's FETCH_SIZE "
                         "and WRITE_SIZE, then those of --calib-copy-mib 1024) into HBM bytes "
                         "per launch; prints a markdown table and the traffic line")
    ap.add_argument("--label", default=None, help="kernel label for --pmc-summary's traffic line")
    ap.add_argument("--counter-summary", nargs="+", metavar="DIR",
                    help="only summarise rocprofv3 --pmc runs (one or more output folders): "
                         "per libmoe kernel, each counter's average over its dispatches, and "
                         "the derived fractions named in the table's notes; prints markdown")
    args = ap.parse_args()
    if args.trace_summary:
        if args.pre_steps is None or args.post_steps is None:
            raise SystemExit("--trace-summary needs --pre-steps and --post-steps (the "
                             "trace_layout of the profiled run's JSON line)")
        trace_summary(args.trace_summary, args.pre_steps, args.steps, args.post_steps)
        return
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, label=args.label)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.calib_copy_mib > 0:
        calib_copy(args.calib_copy_mib)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the library "
              f"runs one whole MoE layer per GPU and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    warm_steps = args.steps if args.warm_steps is None else args.warm_steps

    import torch

    import mixture_experts_layer_level_amd as moe  # noqa: F401  (fails loudly without libmoe.so)
    import moe_synth as ms

    torch.cuda.set_device(0)

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    cfg = ms.CONFIGS[args.config]
    head, inp = run_layer(cfg, Opts(args.padded, args.fused, args.xperm, args.weights,
                                    not args.eager),
                          args.steps, args.warmup, warm_steps, log)
    line = {
        "metric": "MoE-layer tokens/sec + TFLOPS (% bf16 MFMA peak) / HBM GB/s (% peak), 1 GPU",
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based draws, random-init weights)",
        "config": head["config"],
        "timing": "each timed step cold: 512 MiB scratch written then read outside its HIP "
                  "events; ms_per_step: the step as one HIP graph replay (eager_ms_per_step: "
                  "the library calls issued one by one); warm_ms_per_step: steps back to back",
        "trace_layout": head["trace_layout"],
    }
    for k in ("warm_ms_per_step", "eager_ms_per_step", "graph_ms_per_step", "tflops",
              "pct_bf16_mfma_peak", "weight_stream_gbps",
              "pct_hbm_peak_weights", "ffn_weight_stream_gbps", "max_expert_rows",
              "dropped_slots", "stages", "roofline"):
        line[k] = head[k]
    line["cpu_baseline"] = None
    ntok = CPU_TOKENS.get(cfg.name, 256) if args.cpu_tokens < 0 else args.cpu_tokens
    if ntok > 0:
        log(f"CPU oracle on {min(ntok, cfg.N)} tokens")
        line["cpu_baseline"] = (cpu_baseline_gelu(cfg, inp, min(ntok, cfg.N))
                                if cfg.expert == "gelu" else
                                cpu_baseline(cfg, inp, min(ntok, cfg.N),
                                             head["config"]["capacity"],
                                             args.weights in ("fp8", "fp8packed")))
    del inp
    torch.cuda.empty_cache()

    extras = {}
    if args.extra and args.extra != "none" and not (args.fused or
                                                    args.weights in ("fp8", "fp8packed")):
        for item in args.extra.split(","):
            # name:padded (capacity-padded layout), name:packed (packed weights),
            # name:fp8packed (FP8 weights, codes packed)
            name, _, mode = item.partition(":")
            weights = mode if mode in ("packed", "fp8packed") else args.weights
            if name == cfg.name and (mode == "padded") == args.padded and \
                    weights == args.weights:
                continue
            res, inp = run_layer(ms.CONFIGS[name],
                                 Opts(padded=mode == "padded", weights=weights,
                                      graph=not args.eager), args.steps,
                                 args.warmup, warm_steps, log)
            del inp
            torch.cuda.empty_cache()
            keep = ("workload", "value", "unit", "ms_per_step", "warm_ms_per_step",
                    "eager_ms_per_step", "graph_ms_per_step", "tflops",
                    "pct_bf16_mfma_peak", "weight_stream_gbps", "pct_hbm_peak_weights",
                    "max_expert_rows", "dropped_slots", "stages", "roofline")
            extras[name + ("_" + mode if mode else "")] = {k: res[k] for k in keep}
    line["workloads"] = extras
    print(json.dumps(line), flush=True)


def calib_copy(mib: int):
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters give the
    factor between what those counters report and the bytes actually moved."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[calib] copied {n} bytes three times", file=sys.stderr, flush=True)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo", encoding="utf-8"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, inp, n, capv, fp8=False):
    """The C++ oracle, as it stands, on the first n tokens of the same layer
    (route, permute, expert FFN, combine; the experts stream one at a time).
    FP8 weights: quantised and dequantised by the numpy oracle before the
    timed run, as the GPU's are quantised before its timed steps."""
    import numpy as np
    import torch

    from oracle import cpp as C
    from oracle import moe_oracle as O

    def b(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    x = b(inp["x"][:n])
    wr = inp["w_router"].cpu().numpy()
    bias = None if inp["bias"] is None else inp["bias"].cpu().numpy()
    wg, wu, wd = b(inp["w_gate"]), b(inp["w_up"]), b(inp["w_down"])
    if fp8:
        wg, wu, wd = (O.dequantize_fp8_bits(*O.quantize_fp8(m)) for m in (wg, wu, wd))
    cap = C.capacity(n, cfg.K, cfg.E, *cfg.capacity) if capv else None
    t0 = time.perf_counter()
    C.forward(x, wr, bias, wg, wu, wd, cfg.K, cfg.gating, cap=cap, want_h=False)
    dt = time.perf_counter() - t0
    slots = n * cfg.K if cap is None else min(n * cfg.K, cfg.E * cap)
    flop = 2.0 * n * cfg.D * cfg.E + 6.0 * cfg.D * cfg.F * slots
    return {"value": n / dt, "unit": "tokens/s", "cores": C.threads(), "kind": "oracle",
            "nproc": os.cpu_count(), "cpu_model": cpu_model(), "gflops": flop / dt / 1e9,
            "seconds": dt,
            "sample": f"first {n} of {cfg.N} tokens of the same layer (same weights), C++ "
                      f"oracle (float64 sums, OpenMP over rows and output columns)"}


def cpu_baseline_gelu(cfg, inp, n):
    """The numpy oracle of the GELU-expert layer on the first n tokens."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    from oracle import moe_oracle as O

    def h(t):
        if t.dtype == torch.bfloat16:
            return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()

    a = {k: h(v) for k, v in inp.items()}
    t0 = time.perf_counter()
    O.forward_gelu(a["x"][:n], a["w_proj"], a["b_proj"], a["w_out"], a["b_out"], a["w1"],
                   a["b1"], a["w2"], a["b2"], cfg.K)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    D4 = cfg.D // 4
    flop = 2.0 * n * (cfg.D * D4 + D4 * cfg.E) + 4.0 * cfg.D * cfg.F * n * cfg.K
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "nproc": os.cpu_count(), "gflops": flop / dt / 1e9, "cpu_model": cpu_model(),
            "seconds": dt,
            "sample": f"first {n} of {cfg.N} tokens, same weights, float64 numpy oracle"}


# ---------------------------------------------------------------- profile summaries

def _rows(path):
    with open(path, newline="", encoding="utf-8") as f:
        return list(csv.DictReader(f))


def _is_libmoe(name: str) -> bool:
    keys = ("grouped_gemm", "grouped_ffn", "router_", "topk_", "perm_", "combine_",
            "quantize_fp8", "routing_stats", "fused_reset", "write_offsets", "route_decode",
            "moe_")
    return any(k in name for k in keys)


def _short(name: str) -> str:
    """Kernel name without the namespace, return type and argument list."""
    n = name
    for pre in ("void ", "moe::(anonymous namespace)::", "(anonymous namespace)::", "moe::"):
        n = n.replace(pre, "")
    depth = 0
    for i, ch in enumerate(n):      # cut at the argument list's "(" outside any <...>
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return n[:i].strip()
    return n.strip()


def trace_summary(d: str, pre_steps, steps: int, post_steps: int):
    """Per libmoe kernel: the launches of the eager timed steps of a profiled
    run (pre_steps whole steps, then the `steps` timed ones, then post_steps
    more: graph replays and warm steps).
    A kernel launched c times per step has its first pre_steps * c launches
    skipped and the next steps * c taken; c = its launches / all steps."""
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {d}")
    launches = {}
    for f in files:
        for r in _rows(f):
            name = _short(r.get("Kernel_Name", ""))
            if not _is_libmoe(name):
                continue
            launches.setdefault(name, []).append(
                (int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    if pre_steps is None:
        raise SystemExit("--pre-steps is needed")
    counts = {k: len(v) for k, v in launches.items()}
    total_steps = pre_steps + steps + post_steps
    out = []
    layer = 0.0
    for name, v in launches.items():
        v.sort()
        c = len(v) / total_steps
        if abs(c - round(c)) > 1e-9 or round(c) == 0:
            # a kernel outside the per-step pattern (e.g. input generation)
            continue
        c = int(round(c))
        sel = v[pre_steps * c:(pre_steps + steps) * c]
        dur = [(b - a) / 1e3 for a, b in sel]
        avg = sum(dur) / len(dur)
        layer += avg * c
        out.append((name, len(dur), avg, min(dur), max(dur), c))
    out.sort(key=lambda r: -r[2] * r[5])
    print("| kernel | launches (timed) | avg µs | min µs | max µs | share of layer |")
    print("|---|---|---|---|---|---|")
    for name, n, avg, lo, hi, c in out:
        print(f"| `{name}` | {n} | {avg:.1f} | {lo:.1f} | {hi:.1f} | "
              f"{100 * avg * c / layer:.1f}% |")
    print(f"\nSum of libmoe kernel time per step: {layer:.1f} µs (timed steps only; "
          f"launches per kernel in the whole run: "
          + ", ".join(f"{k} {v}" for k, v in sorted(counts.items())) + ")")


def _pmc_avg(d: str, counter: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    acc = {}
    for f in files:
        for r in _rows(f):
            if r.get("Counter_Name") != counter:
                continue
            name = _short(r.get("Kernel_Name", ""))
            acc.setdefault(name, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def counter_summary(dirs, cus=256, xcds=8):
    """Average of every counter per libmoe kernel over the runs under dirs,
    plus derived fractions where their counters are present:
      - SQ_* / SQ_WAVE_CYCLES (shares of the cycles waves are resident);
      - TA/TD busy = xcds * *_BUSY_sum / (cus * GRBM_GUI_ACTIVE) (GRBM_GUI_ACTIVE
        reads the kernel's cycles summed over the XCDs);
      - L2 hit = TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)."""
    vals = {}
    for d in dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        for f in files:
            for r in _rows(f):
                name = _short(r.get("Kernel_Name", ""))
                if not _is_libmoe(name):
                    continue
                vals.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
    counters = sorted({c for v in vals.values() for c in v})
    derived = []
    if "SQ_WAVE_CYCLES" in counters:
        derived += [(f"{c} / SQ_WAVE_CYCLES", (lambda a, c=c: a[c] / a["SQ_WAVE_CYCLES"]))
                    for c in counters if c.startswith("SQ_") and c not in
                    ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES") and not c.startswith("SQ_INSTS")]
    if "GRBM_GUI_ACTIVE" in counters:
        for c in ("TA_TA_BUSY_sum", "TD_TD_BUSY_sum"):
            if c in counters:
                derived.append((c.split("_")[0] + " busy",
                                (lambda a, c=c: xcds * a[c] / (cus * a["GRBM_GUI_ACTIVE"]))))
    if "TCC_HIT_sum" in counters and "TCC_MISS_sum" in counters:
        derived.append(("L2 hit", lambda a: a["TCC_HIT_sum"] /
                        max(1.0, a["TCC_HIT_sum"] + a["TCC_MISS_sum"])))
    cols = counters + [n for n, _ in derived]
    print("| kernel | " + " | ".join(cols) + " |")
    print("|---|" + "---|" * len(cols))
    for name in sorted(vals, key=lambda k: -max(sum(v) / len(v) for v in vals[k].values())):
        avg = {c: sum(v) / len(v) for c, v in vals[name].items()}
        cells = [f"{avg[c]:.4g}" if c in avg else "" for c in counters]
        for _, fn in derived:
            try:
                cells.append(f"{fn(avg):.3f}")
            except (KeyError, ZeroDivisionError):
                cells.append("")
        print(f"| `{name}` | " + " | ".join(cells) + " |")


def pmc_summary(fetch_dir, write_dir, cfetch_dir, cwrite_dir, label=None):
    """HBM bytes per launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for a copy of known size."""
    fetch, write = _pmc_avg(fetch_dir, "FETCH_SIZE"), _pmc_avg(write_dir, "WRITE_SIZE")
    cf, cw = _pmc_avg(cfetch_dir, "FETCH_SIZE"), _pmc_avg(cwrite_dir, "WRITE_SIZE")
    copy_f = max(cf.values())   # the copy kernel is the largest dispatch of that run
    copy_w = max(cw.values())
    n = 1024 * 1024             # KiB copied by --calib-copy-mib 1024
    kf, kw = n / copy_f, n / copy_w
    print(f"Calibration: a 1 GiB device-to-device copy reads FETCH_SIZE = {copy_f:.0f} KiB and "
          f"WRITE_SIZE = {copy_w:.0f} KiB, so bytes = FETCH_SIZE x 1024 x {kf:.4f} and "
          f"WRITE_SIZE x 1024 x {kw:.4f}. Values are averages over the dispatches of each "
          f"kernel.\n")
    print("| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read GB | HBM write GB | total GB |")
    print("|---|---|---|---|---|---|")
    best = None
    for name in sorted(fetch, key=lambda k: -fetch[k]):
        if not _is_libmoe(name):
            continue
        f, w = fetch[name], write.get(name, 0.0)
        rd, wr = f * 1024 * kf / 1e9, w * 1024 * kw / 1e9
        print(f"| `{name}` | {f:.0f} | {w:.0f} | {rd:.3f} | {wr:.3f} | {rd + wr:.3f} |")
        if label and label in name and best is None:
            best = (name, int((rd + wr) * 1e9))
    if best:
        print("\nMachine-readable line for the benchmark (bytes per launch of the dominant "
              "kernel; valid only while the kernel source has this SHA-256):\n")
        print("traffic: " + json.dumps({"kernel": best[0], "bytes": best[1],
                                        "source_sha256": source_sha()}))


if __name__ == "__main__":
    main()
