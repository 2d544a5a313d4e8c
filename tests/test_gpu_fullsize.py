"""GPU parity at the workloads' full sizes, tile by tile, against the C++ oracle.

Every tile the grouped GEMMs cut is a run of whole 32-row blocks of one
expert's segment (the 256-row tiles, the second tiles of experts that
straddle 256 rows, the extra row tiles that fill a persistent launch's last
round, the 32-row decode tiles): so the first and last row of every 32-row
block of every segment are the first and last rows of every tile of every
launch.  Those rows of h and out_perm are compared with the oracle over all
their columns, on each path the library offers at that size:

- the staged path with the permuted copy of x (moe_expert_gateup on x_perm),
- the gate/up GEMM reading its rows of x through row_token (the path the
  benchmark times; bit for bit the first),
- the fused one-launch FFN (contiguous layout; bit for bit the staged one),
- block-scaled FP8 weights (codes and scales of every expert bit-exact
  against the oracle's quantiser; h and out_perm against the oracle's FFN on
  its own dequantised weights),
- the capacity-padded layout (hot skew; padding rows exactly zero).

Routing ids and the permutation are compared over all tokens, router logits
within the fp32 summation bound on 64 tokens, and y on 64 tokens.  Bars as in
the small-shape tests: bit-exact for integer work; h, out_perm and y within
max|d| <= 1e-2 max|ref| and per-element rtol 2e-2.
"""
import numpy as np
import pytest
import torch

import moe_synth as ms
from oracle import cpp as C
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

from gpu_layer import (DEV, Layer, assert_fp_close, assert_logits_bound, bits,  # noqa: E402
                       np_, sample_tokens)
import mixture_experts_layer_level_amd as moe  # noqa: E402

UNSUPPORTED = 2


def block_rows(offsets, counts, cap):
    """(rows, experts): the first and last row of every 32-row block of every
    expert's kept rows."""
    rows, experts = [], []
    for e in range(len(counts)):
        lo = int(offsets[e])
        m = int(offsets[e + 1] - offsets[e]) if cap is None else min(int(counts[e]), cap)
        for b in range(0, m, 32):
            for r in sorted({lo + b, lo + min(b + 32, m) - 1}):
                rows.append(r)
                experts.append(e)
    return np.array(rows, dtype=np.int64), np.array(experts, dtype=np.int32)


def y_reference(tokens, ids, w, slot_row, K, x_bits, wg, wu, wd):
    """y of the given tokens from the oracle's expert FFN of their kept slots
    and its combine (k order, fp32 sum, bf16)."""
    re, rt, where = [], [], np.full(len(tokens) * K, -1, dtype=np.int32)
    for i, t in enumerate(tokens):
        for k in range(K):
            if slot_row[t * K + k] >= 0:
                where[i * K + k] = len(re)
                re.append(ids[t, k])
                rt.append(t)
    _, out = C.ffn_rows(np.array(re, np.int32), np.array(rt, np.int32), x_bits, wg, wu, wd,
                        want_h=False)
    return C.combine(out, where, w[tokens])


class Ref:
    """The oracle side of one workload: routing on the GPU's fp32 logits, the
    permutation, and the FFN of the block rows."""

    def __init__(self, L: Layer, padded: bool):
        cfg = L.cfg
        self.cfg = cfg
        self.x = bits(L.x)
        lg = np_(L.logits)
        bias = None if L.bias is None else np_(L.bias)
        assert_logits_bound(lg, self.x, np_(L.w_router), rows=sample_tokens(cfg.N, 64))
        self.ids, self.w = C.route_from_logits(lg, bias, cfg.K, cfg.gating)
        self.cap = L.cap if padded else None
        (self.counts, self.offsets, self.row_token,
         self.slot_row) = C.permute(self.ids, cfg.E, self.cap)
        self.rows, self.experts = block_rows(self.offsets, self.counts, self.cap)
        self.tokens = sample_tokens(cfg.N, 64)

    def ffn(self, wg, wu, wd):
        return C.ffn_rows(self.experts, self.row_token[self.rows], self.x, wg, wu, wd)

    def y(self, wg, wu, wd):
        return y_reference(self.tokens, self.ids, self.w, self.slot_row, self.cfg.K, self.x,
                           wg, wu, wd)


def check_rows(ref: Ref, h, out_perm, h_ref, out_ref, what):
    if h is not None:
        assert_fp_close(O.bf16_to_f64(bits(h)[ref.rows]), h_ref, f"h ({what})")
    assert_fp_close(O.bf16_to_f64(bits(out_perm)[ref.rows]), out_ref, f"out_perm ({what})")


def check_y(ref: Ref, y, y_ref, what):
    assert_fp_close(O.bf16_to_f64(bits(y)[ref.tokens]), y_ref, f"y[64 tokens] ({what})")


def covered_mask(ref: Ref, R):
    m = np.zeros(R, dtype=bool)
    for e in range(ref.cfg.E):
        lo = ref.offsets[e]
        n = ref.offsets[e + 1] - lo if ref.cap is None else min(ref.counts[e], ref.cap)
        m[lo:lo + n] = True
    return m


def fused_error_word(L, whole_layer):
    off = moe.fused_error_offset(L.p, whole_layer)
    return int(L.ws[off:off + 4].view(torch.int32).item())


def quantize_on_gpu(w: torch.Tensor):
    rows, cols = w.shape[-2], w.shape[-1]
    codes = torch.empty(w.shape, dtype=torch.uint8, device=DEV)
    scales = torch.empty(w.shape[0], rows // 32, cols // 32, 32, dtype=torch.uint8, device=DEV)
    moe.quantize_fp8(w.numel() // cols, cols, w, codes, scales)
    return codes, scales


def blocked(scales: np.ndarray) -> np.ndarray:
    """Oracle scales [E, rows, cols/32] -> the ABI layout [E, rows/32, cols/32, 32]."""
    E, rows, nb = scales.shape
    return np.swapaxes(scales.reshape(E, rows // 32, 32, nb), -1, -2)


FULL = [("mixtral", False), ("deepseek_v3", False), ("qwen3_decode", False),
        ("hot_skew", False), ("hot_skew", True)]


@pytest.mark.parametrize("name,padded", FULL,
                         ids=[f"{n}{'_padded' if p else ''}" for n, p in FULL])
def test_full_size_per_tile(name, padded):
    cfg = ms.CONFIGS[name]
    print(f"[full-size per tile] {name} padded={padded}: staged", flush=True)
    L = Layer(cfg, padded=padded)
    L.staged()
    ref = Ref(L, padded)
    assert np.array_equal(np_(L.ids), ref.ids), "top-K ids"
    assert np.abs(np_(L.w).astype(np.float64) - ref.w).max() <= 1e-6
    for got, exp, nm in ((L.counts, ref.counts, "counts"), (L.offsets, ref.offsets, "offsets"),
                         (L.row_token, ref.row_token, "row_token"),
                         (L.slot_row, ref.slot_row, "slot_row")):
        assert np.array_equal(np_(got), exp), nm
    if name == "hot_skew":
        assert 0.2 <= ref.counts.max() / cfg.S <= 0.3
    cov = covered_mask(ref, L.R)
    wg, wu, wd = bits(L.w_gate), bits(L.w_up), bits(L.w_down)
    h_ref, out_ref = ref.ffn(wg, wu, wd)
    y_ref = ref.y(wg, wu, wd)
    check_rows(ref, L.h, L.out_perm, h_ref, out_ref, "staged, x_perm")
    check_y(ref, L.y, y_ref, "staged")
    if padded:
        pad = ref.row_token < 0
        assert np.all(bits(L.out_perm)[pad] == 0) and np.all(bits(L.x_perm)[pad] == 0)
    y2 = torch.empty_like(L.y)
    L.forward(y2)
    assert torch.equal(y2.view(torch.int16), L.y.view(torch.int16)), "moe_forward vs staged"

    if not padded:
        # gate/up rows read from x through row_token: bit for bit the staged h
        print(f"[full-size per tile] {name}: gathered", flush=True)
        hg = torch.full_like(L.h, float("nan"))
        try:
            moe.expert_gateup_gathered(L.p, L.x, L.row_token, L.offsets, L.w_gate, L.w_up, hg)
            torch.cuda.synchronize()
            assert np.array_equal(bits(hg)[cov], bits(L.h)[cov]), "gathered h vs staged"
        except moe.MoEError as err:
            assert err.status == UNSUPPORTED and cfg.D < 1024
        del hg

        # the fused one-launch FFN
        print(f"[full-size per tile] {name}: fused", flush=True)
        outf = torch.empty_like(L.out_perm)
        moe.fused_ffn(L.p, L.x, L.row_token, L.offsets, L.w_gate, L.w_up, L.w_down, outf, L.ws)
        torch.cuda.synchronize()
        assert fused_error_word(L, False) == 0
        check_rows(ref, None, outf, None, out_ref, "fused")
        assert np.array_equal(bits(outf)[cov], bits(L.out_perm)[cov]), "fused vs staged"
        yf = torch.empty_like(L.y)
        moe.forward_fused(L.p, L.x, L.w_router, L.bias, L.w_gate, L.w_up, L.w_down, yf, L.ws)
        torch.cuda.synchronize()
        assert fused_error_word(L, True) == 0
        assert torch.equal(yf.view(torch.int16), L.y.view(torch.int16)), "forward_fused"
        del outf, yf

        # block-scaled FP8 weights: every expert's codes and scales bit-exact,
        # then the FP8 FFN against the oracle on its own dequantised weights
        print(f"[full-size per tile] {name}: fp8", flush=True)
        q = [quantize_on_gpu(t) for t in (L.w_gate, L.w_up, L.w_down)]
        deq = []
        for (codes, scales), w_bits, what in zip(q, (wg, wu, wd), ("gate", "up", "down")):
            oc, osc = C.quantize_fp8(w_bits)
            assert np.array_equal(np_(codes), oc), f"fp8 codes ({what})"
            assert np.array_equal(np_(scales), blocked(osc)), f"fp8 scales ({what})"
            deq.append(C.dequantize_fp8_bits(oc, osc))
        h8 = torch.empty_like(L.h)
        out8 = torch.empty_like(L.out_perm)
        moe.expert_gateup_fp8(L.p, L.x_perm, L.offsets, q[0], q[1], h8)
        moe.expert_down_fp8(L.p, h8, L.offsets, q[2], out8)
        torch.cuda.synchronize()
        h8_ref, out8_ref = ref.ffn(*deq)
        check_rows(ref, h8, out8, h8_ref, out8_ref, "fp8")
        h8g = torch.full_like(L.h, float("nan"))
        try:
            moe.expert_gateup_fp8_gathered(L.p, L.x, L.row_token, L.offsets, q[0], q[1], h8g)
            torch.cuda.synchronize()
            assert np.array_equal(bits(h8g)[cov], bits(h8)[cov]), "fp8 gathered h vs x_perm"
        except moe.MoEError as err:
            assert err.status == UNSUPPORTED and cfg.D < 512
        y8 = torch.empty_like(L.y)
        moe.forward_fp8(L.p, L.x, L.w_router, L.bias, q[0], q[1], q[2], y8, L.ws)
        torch.cuda.synchronize()
        check_y(ref, y8, ref.y(*deq), "fp8")
        del q, deq, h8, out8, h8g, y8
    del L
    torch.cuda.empty_cache()
