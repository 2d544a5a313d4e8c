#!/usr/bin/env python3
"""Throughput of the single-GPU MoE-layer forward pass on MI355X.

One step = the whole layer on one batch: router GEMM + top-K gating, permute
into expert segments, grouped gate/up GEMM with SwiGLU, grouped down GEMM,
unpermute + weighted combine -- the five libmoe calls moe_forward is made of,
issued separately so the dominant kernel (the gate/up grouped GEMM) can be
bracketed with HIP events on the stream it runs on.  Inputs are synthetic,
seeded and already resident in HBM when timing starts.

``--config gelu_mlp`` runs the pages' other layer: an MLP router
(Linear(D, D/4) + GELU, then the gate Linear) and experts
Linear(D, 4D) - GELU - Linear(4D, D) with biases; its dominant kernel is the
up GEMM with the bias + GELU epilogue.

With ``--weights fp8`` the expert weights are stored as block-scaled FP8
(E4M3 codes, one power-of-two scale per 32 values; quantised once before
timing) and the two grouped GEMMs read them through the FP8 entry points.

Prints one JSON line.  ``value`` is tokens/s of the layer on this GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
ROOT = os.path.dirname(os.path.abspath(__file__))
GEMM_SRC = os.path.join(ROOT, "mixture_experts_layer_level_amd", "csrc", "grouped_gemm.hip")


def measured_traffic(workload: str):
    """HBM bytes per gate/up launch from the committed rocprofv3 --pmc summary of
    this workload, or None when there is none or the kernel source has changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    rec = None
    for line in open(path, encoding="utf-8"):
        if line.startswith("traffic: "):
            rec = json.loads(line[len("traffic: "):])
    if rec is None:
        return None
    sha = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()
    return rec["bytes"] if rec.get("source_sha256") == sha else None


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mixtral",
                    help="tiny | mixtral | deepseek_v3 | qwen3_decode | hot_skew | gelu_mlp | "
                         "gelu_tiny")
    ap.add_argument("--padded", action="store_true", help="capacity-padded layout (hot_skew)")
    ap.add_argument("--fused", action="store_true",
                    help="the expert FFN as one persistent launch (moe_fused_ffn; rows gathered "
                         "from x, no permuted copy)")
    ap.add_argument("--xperm", action="store_true",
                    help="write the permuted copy of x and run the first expert GEMM on it; by "
                         "default that GEMM reads its rows of x through row_token "
                         "(moe_expert_gateup_gathered, moe_expert_gateup_fp8_gathered, "
                         "moe_expert_up_gelu_gathered) wherever the library takes the shape")
    ap.add_argument("--weights", choices=("bf16", "fp8"), default="bf16",
                    help="expert weight storage: bf16, or block-scaled FP8 (E4M3 + E8M0)")
    ap.add_argument("--cpu-tokens", type=int, default=4096,
                    help="tokens of the CPU-oracle sample, at most the workload's N (0 = skip "
                         "the CPU baseline); the oracle's fixed cost (weights to float64) "
                         "dominates small samples")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB, three "
                         "times (the reference kernel for HBM byte counters), then exit")
    args = ap.parse_args()
    if args.calib_copy_mib > 0:
        calib_copy(args.calib_copy_mib)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              f"(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mixture_experts_layer_level_amd as moe
    import moe_synth as ms

    cfg = ms.CONFIGS[args.config]
    dev = "cuda"
    torch.cuda.set_device(0)
    cap = cfg.capacity if args.padded else None
    if args.padded and cap is None:
        raise SystemExit(f"{cfg.name} has no capacity factor")
    gelu = cfg.expert == "gelu"
    if args.fused and (gelu or args.weights != "bf16" or args.padded):
        raise SystemExit("--fused runs the SwiGLU layer, bf16 weights, contiguous layout")
    if gelu and args.weights != "bf16":
        raise SystemExit("the GELU-expert layer runs with bf16 weights")
    t0 = time.time()
    inp = ms.make_gelu_inputs(cfg, device=dev) if gelu else ms.make_inputs(cfg, device=dev)
    torch.cuda.synchronize()
    print(f"[bench] inputs {cfg.name} generated in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)
    p = moe.problem(cfg.N, cfg.D, cfg.F, cfg.E, cfg.K, cfg.gating, cap)
    R, capv = moe.permuted_rows(p)
    N, D, E, K, F = cfg.N, cfg.D, cfg.E, cfg.K, cfg.F
    e = lambda *s, dt=torch.float32: torch.empty(*s, dtype=dt, device=dev)
    logits, ids, w = e(N, E), e(N, K, dt=torch.int32), e(N, K)
    counts, offsets = e(E, dt=torch.int32), e(E + 1, dt=torch.int32)
    row_token, slot_row = e(R, dt=torch.int32), e(N * K, dt=torch.int32)
    x_perm, h = e(R, D, dt=torch.bfloat16), e(R, F, dt=torch.bfloat16)
    out_perm, y = e(R, D, dt=torch.bfloat16), e(N, D, dt=torch.bfloat16)
    ws = torch.empty(moe.workspace_size(p), dtype=torch.uint8, device=dev)
    x = inp["x"]
    if gelu:
        feats = e(N, D // 4, dt=torch.bfloat16)
    else:
        wr, bias = inp["w_router"], inp["bias"]
        wg, wu, wd = inp["w_gate"], inp["w_up"], inp["w_down"]
    stream = torch.cuda.current_stream()
    fp8 = args.weights == "fp8"
    if fp8:
        def quant(wt):
            rows, cols = wt.shape[-2], wt.shape[-1]
            c = torch.empty(wt.shape, dtype=torch.uint8, device=dev)
            sc = torch.empty(wt.shape[0], rows // 32, cols // 32, 32, dtype=torch.uint8,
                             device=dev)
            moe.quantize_fp8(wt.numel() // cols, cols, wt, c, sc, stream=stream)
            return c, sc
        qg, qu, qd = quant(wg), quant(wu), quant(wd)
        torch.cuda.synchronize()

    # The first expert GEMM (gate/up, or the GELU layer's up GEMM) reads its rows of x through row_token
    # wherever the library takes the shape; it refuses, before any launch, the
    # shapes whose tiles have no gathered form.  One route + permute first, so
    # that the trial call runs on real routing tables.
    gather = not (args.xperm or args.fused or capv)
    if gather:
        if gelu:
            moe.route_mlp(p, x, inp["w_proj"], inp["b_proj"], inp["w_out"], inp["b_out"], logits,
                          ids, w, ws, features=feats, stream=stream)
        else:
            moe.route(p, x, wr, bias, logits, ids, w, stream=stream)
        moe.permute(p, x, ids, counts, offsets, row_token, slot_row, None, ws, stream=stream)
        try:
            if gelu:
                moe.expert_up_gelu_gathered(p, x, row_token, offsets, inp["w1"], inp["b1"], h,
                                            stream=stream)
            elif fp8:
                moe.expert_gateup_fp8_gathered(p, x, row_token, offsets, qg, qu, h, stream=stream)
            else:
                moe.expert_gateup_gathered(p, x, row_token, offsets, wg, wu, h, stream=stream)
        except moe.MoEError as err:
            if err.status != 2:   # MOE_ERR_UNSUPPORTED: run the permuted copy instead
                raise
            gather = False
        torch.cuda.synchronize()

    # ev: six events per step, recorded on the launch stream before the route
    # and after the route, permute, gate/up (or up, or fused FFN), down and
    # combine calls
    def rec(ev, i):
        if ev is not None:
            ev[i].record(stream)

    def step_gelu(ev=None):
        i = inp
        rec(ev, 0)
        moe.route_mlp(p, x, i["w_proj"], i["b_proj"], i["w_out"], i["b_out"], logits, ids, w, ws,
                      features=feats, stream=stream)
        rec(ev, 1)
        moe.permute(p, x, ids, counts, offsets, row_token, slot_row,
                    None if gather else x_perm, ws, stream=stream)
        rec(ev, 2)
        if gather:
            moe.expert_up_gelu_gathered(p, x, row_token, offsets, i["w1"], i["b1"], h,
                                        stream=stream)
        else:
            moe.expert_up_gelu(p, x_perm, offsets, i["w1"], i["b1"], h, stream=stream)
        rec(ev, 3)
        moe.expert_down_bias(p, h, offsets, i["w2"], i["b2"], out_perm, stream=stream)
        rec(ev, 4)
        moe.unpermute_combine(p, out_perm, slot_row, w, y, stream=stream)
        rec(ev, 5)

    def step_fused(ev=None):
        rec(ev, 0)
        moe.route(p, x, wr, bias, logits, ids, w, stream=stream)
        rec(ev, 1)
        moe.permute(p, x, ids, counts, offsets, row_token, slot_row, None, ws, stream=stream)
        rec(ev, 2)
        moe.fused_ffn(p, x, row_token, offsets, wg, wu, wd, out_perm, ws, stream=stream)
        rec(ev, 3)
        rec(ev, 4)
        moe.unpermute_combine(p, out_perm, slot_row, w, y, stream=stream)
        rec(ev, 5)

    def step(ev=None):
        if gelu:
            return step_gelu(ev)
        if args.fused:
            return step_fused(ev)
        rec(ev, 0)
        moe.route(p, x, wr, bias, logits, ids, w, stream=stream)
        rec(ev, 1)
        moe.permute(p, x, ids, counts, offsets, row_token, slot_row,
                    None if gather else x_perm, ws, stream=stream)
        rec(ev, 2)
        if gather and fp8:
            moe.expert_gateup_fp8_gathered(p, x, row_token, offsets, qg, qu, h, stream=stream)
        elif gather:
            moe.expert_gateup_gathered(p, x, row_token, offsets, wg, wu, h, stream=stream)
        elif fp8:
            moe.expert_gateup_fp8(p, x_perm, offsets, qg, qu, h, stream=stream)
        else:
            moe.expert_gateup(p, x_perm, offsets, wg, wu, h, stream=stream)
        rec(ev, 3)
        if fp8:
            moe.expert_down_fp8(p, h, offsets, qd, out_perm, stream=stream)
        else:
            moe.expert_down(p, h, offsets, wd, out_perm, stream=stream)
        rec(ev, 4)
        moe.unpermute_combine(p, out_perm, slot_row, w, y, stream=stream)
        rec(ev, 5)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(6))
           for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps

    def stage_ms(i, j):
        return sum(ev[i].elapsed_time(ev[j]) for ev in evs) / args.steps
    route_ms, permute_ms = stage_ms(0, 1), stage_ms(1, 2)
    gateup_ms, down_ms, combine_ms = stage_ms(2, 3), stage_ms(3, 4), stage_ms(4, 5)
    per_step = sorted(ev[0].elapsed_time(ev[5]) for ev in evs)

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
    # the dominant kernel (gate/up grouped GEMM; up GEMM of the GELU experts):
    # algorithmic work per launch
    gu_mats = nmat - 1
    gu_flops = 2.0 * gu_mats * D * F * kept
    gu_bytes = gu_mats * touched * F * D * wb + kept * D * 2 + kept * F * 2   # weights, x_perm, h
    t_mfma = gu_flops / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = gu_bytes / (PEAK_HBM_GBPS * 1e9)
    if t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": gu_flops / (gateup_ms * 1e-3) / 1e12,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": gu_bytes / (gateup_ms * 1e-3) / 1e9,
                "peak": PEAK_HBM_GBPS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(args.config + ("_padded" if capv else "") +
                                       ("_fp8" if fp8 else "") + ("_xperm" if args.xperm else ""))
    roof["kernel"] = (("grouped up GEMM + bias + GELU" if gelu
                       else "grouped gate/up GEMM + SwiGLU") +
                      (", rows gathered from x through row_token" if gather else ""))
    if args.fused:
        # the one fused launch: gate/up, SwiGLU and down of every expert
        f_flops = 6.0 * D * F * kept
        f_bytes = 3.0 * touched * F * D * 2 + kept * D * 2 * 2 + kept * F * 2 * 2
        t_m, t_h = f_flops / (PEAK_BF16_TFLOPS * 1e12), f_bytes / (PEAK_HBM_GBPS * 1e9)
        if t_m >= t_h:
            roof = {"bound": "mfma", "achieved": f_flops / (gateup_ms * 1e-3) / 1e12,
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
        else:
            roof = {"bound": "hbm", "achieved": f_bytes / (gateup_ms * 1e-3) / 1e9,
                    "peak": PEAK_HBM_GBPS, "unit": "GB/s"}
        roof["frac"] = roof["achieved"] / roof["peak"]
        roof["traffic"] = measured_traffic(args.config + "_fused")
        roof["kernel"] = "fused expert FFN (gate/up + SwiGLU + down, one launch)"
        roof["algorithmic"] = {"flop": f_flops, "bytes": f_bytes}
    roof["avg_ms"] = gateup_ms
    roof.setdefault("algorithmic", {"flop": gu_flops, "bytes": gu_bytes})
    # the HBM-bound stages against 8 TB/s: permute (x read once, x_perm rows
    # written, ids read, row_token and slot_row written, offsets), combine
    # (out_perm rows read, y written, slot_row and weights read)
    S_ = N * K
    perm_bytes = (S_ * 4 * 3 + (E + 1) * 4 +
                  (0 if args.fused or gather else N * D * 2 + R * D * 2))
    comb_bytes = kept * D * 2 + N * D * 2 + S_ * 8
    stages = {
        "route_ms": route_ms, "permute_ms": permute_ms, "ffn_ms": gateup_ms + down_ms,
        "combine_ms": combine_ms,
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
    line = {
        "metric": "MoE-layer tokens/sec + TFLOPS (% bf16 MFMA peak) / HBM GB/s (% peak), 1 GPU",
        "value": N / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based draws, random-init weights)",
        "config": {"workload": cfg.note + (" [capacity-padded]" if capv else ""),
                   "tokens": N, "hidden": D, "experts": E, "top_k": K, "ffn": F,
                   "gating": cfg.gating, "capacity": capv or None,
                   "expert_weights": ("fp8 e4m3, power-of-two scale per 32 values"
                                      if fp8 else "bf16"),
                   "expert": ("Linear-GELU-Linear with biases, MLP router" if gelu
                              else "SwiGLU"),
                   "ffn_launch": ("fused (one persistent launch)" if args.fused else
                                  "two grouped GEMMs, rows of the first gathered from x" if gather
                                  else "two grouped GEMMs")},
        "tflops": tflops,
        "pct_bf16_mfma_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "weight_stream_gbps": weight_bytes / (ms_step * 1e-3) / 1e9,
        "ffn_weight_stream_gbps": weight_bytes / ((gateup_ms + down_ms) * 1e-3) / 1e9,
        "gateup_ms": gateup_ms,
        "down_ms": down_ms,
        "max_expert_rows": int(counts_h.max()),
        "dropped_slots": int(cfg.S - kept),
        "stages": stages,
        "roofline": roof,
        "cpu_baseline": None,
    }
    print(f"[bench] {ms_step:.3f} ms/step, gate/up {gateup_ms:.3f} ms", file=sys.stderr,
          flush=True)

    # Cold-cache steps, after the timed ones and outside them: before each,
    # 512 MiB of scratch are written (twice the 256 MB memory-side cache), so
    # no activation or weight of the previous step is still cached; each step
    # is timed alone between events on the launch stream.
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(5):
        scratch.zero_()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        step()
        c1.record(stream)
        torch.cuda.synchronize()
        cold.append(c0.elapsed_time(c1))
    del scratch
    line["cold_ms_per_step"] = sorted(cold)[len(cold) // 2]

    if args.cpu_tokens > 0:
        line["cpu_baseline"] = (cpu_baseline_gelu(cfg, inp, min(args.cpu_tokens, N)) if gelu else
                                cpu_baseline(cfg, inp, min(args.cpu_tokens, N), capv, fp8))
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


def cpu_baseline(cfg, inp, n, capv, fp8=False):
    """The CPU oracle, as it stands, on the first n tokens of the same layer
    (FP8 weights: quantised by the oracle before the timed run, as the GPU's
    are before its timed steps)."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    from oracle import moe_oracle as O

    wbytes = 3 * cfg.E * cfg.F * cfg.D * 2
    if wbytes > 8e9:
        return {"value": None, "unit": "tokens/s", "cores": None, "kind": "oracle",
                "sample": f"skipped: {wbytes / 1e9:.1f} GB of expert weights do not fit "
                          f"the host-side oracle run"}

    def b(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    x = b(inp["x"][:n])
    wr = inp["w_router"].cpu().numpy()
    bias = None if inp["bias"] is None else inp["bias"].cpu().numpy()
    wg, wu, wd = b(inp["w_gate"]), b(inp["w_up"]), b(inp["w_down"])
    if fp8:
        wg, wu, wd = (O.dequantize_fp8_bits(*O.quantize_fp8(m)) for m in (wg, wu, wd))
    cap = None
    if capv:
        cap = O.capacity(n, cfg.K, cfg.E, *cfg.capacity)
    t0 = time.perf_counter()
    O.forward(x, wr, bias, wg, wu, wd, cfg.K, cfg.gating, cap=cap)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    slots = n * cfg.K if cap is None else min(n * cfg.K, cfg.E * cap)
    flop = 2.0 * n * cfg.D * cfg.E + 6.0 * cfg.D * cfg.F * slots
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "gflops": flop / dt / 1e9, "cpu_model": cpu_model(),
            "sample": f"first {n} of {cfg.N} tokens, same weights, float64 numpy oracle "
                      f"({dt:.1f} s)"}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo", encoding="utf-8"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline_gelu(cfg, inp, n):
    """The CPU oracle of the GELU-expert layer on the first n tokens."""
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
            "gflops": flop / dt / 1e9, "cpu_model": cpu_model(),
            "sample": f"first {n} of {cfg.N} tokens, same weights, float64 numpy oracle "
                      f"({dt:.1f} s)"}


if __name__ == "__main__":
    main()
