"""GPU parity of the block-scaled FP8 expert-weight path against the oracle.

Bars: quantised codes and scale bytes bit-exact (integer work on the bf16
bits); h, out_perm and y within the FFN bar of the bf16 path (max|d| <= 1e-2
max|ref|, per-element rtol 2e-2) against the oracle's FFN on the oracle's own
quantisation of the same bf16 weights.  Because every dequantised weight is an
exact bf16 number, the FP8 kernels must also agree bit for bit with the bf16
kernels run on the dequantised weights; that is checked as a property of the
kernels on the small cases.
"""
import numpy as np
import pytest
import torch

import moe_synth as ms
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

from gpu_layer import (DEV, SMALL, Layer, assert_fp_close, bits,  # noqa: E402
                       check_permutation, check_routing, np_, sample_tokens)
import mixture_experts_layer_level_amd as moe  # noqa: E402


def blocked(scales: np.ndarray) -> np.ndarray:
    """Oracle scales [..., rows, cols/32] -> the ABI layout [..., rows/32, cols/32, 32]."""
    *lead, rows, nb = scales.shape
    return np.swapaxes(scales.reshape(*lead, rows // 32, 32, nb), -1, -2)


def quantize_on_gpu(w: torch.Tensor):
    """moe_quantize_fp8 of a bf16 stack [..., rows, cols]."""
    rows, cols = w.shape[-2], w.shape[-1]
    lead = tuple(w.shape[:-2])
    codes = torch.empty(w.shape, dtype=torch.uint8, device=DEV)
    scales = torch.empty(lead + (rows // 32, cols // 32, 32), dtype=torch.uint8, device=DEV)
    moe.quantize_fp8(w.numel() // cols, cols, w, codes, scales)
    return codes, scales


def check_quantized(q, w_bits: np.ndarray, what: str):
    """GPU (codes, scales) bit-exact against the oracle; returns the oracle's pair."""
    oc, os_ = O.quantize_fp8(w_bits)
    assert np.array_equal(np_(q[0]), oc), f"{what}: codes"
    assert np.array_equal(np_(q[1]), blocked(os_)), f"{what}: scales"
    return oc, os_


def _bits_tensor(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


@pytest.mark.parametrize("shape,kind", [
    ((32, 32), "normal"), ((64, 320), "normal"), ((3, 96, 128), "normal"),
    ((256, 2048), "normal"), ((64, 256), "all_bits"), ((96, 4096), "all_bits"),
    ((32, 192), "specials"),
])
def test_quantize_matches_oracle(shape, kind):
    """Codes and scales bit-exact: normal weights, uniformly random bit
    patterns (every bf16 value: subnormals, huge values, infinities, NaNs,
    both zeros) and blocks built around the clamps and saturation."""
    print(f"[quantize] {shape} {kind}", flush=True)
    rng = np.random.default_rng(sum(shape) + len(kind))
    if kind == "normal":
        w = O.f64_to_bf16_bits(rng.standard_normal(shape) * 0.02)
    elif kind == "all_bits":
        w = rng.integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)
    else:
        w = O.f64_to_bf16_bits(rng.standard_normal(shape))
        w[0, :32] = 0                                     # all-zero block
        w[1, :32] = 0x8000                                # all negative zeros
        w[2, :32] = rng.integers(1, 128, 32)              # bf16 subnormals only
        w[3, :32] = 0x7F7F                                # largest bf16
        w[4, :32] = O.f64_to_bf16_bits(np.full(32, 1.9921875))   # saturates to 448
        w[5, :4] = [0x7F80, 0xFF80, 0x7FC0, 0xFFC1]       # infinities and NaNs
        w[6, 32:64] = O.f64_to_bf16_bits(np.ldexp(1.0, np.arange(32) - 20))  # 2^-20 .. 2^11
        w[7, :32] = O.f64_to_bf16_bits(np.linspace(-464, 464, 32))
    wt = _bits_tensor(w)
    q = quantize_on_gpu(wt)
    torch.cuda.synchronize()
    check_quantized(q, w, f"{shape} {kind}")


def _fp8_weights(L: Layer):
    return quantize_on_gpu(L.w_gate), quantize_on_gpu(L.w_up), quantize_on_gpu(L.w_down)


@pytest.mark.parametrize("name", list(SMALL))
def test_fp8_ffn_small(name):
    cfg = SMALL[name]
    padded = cfg.capacity is not None
    print(f"[fp8 staged] {name} N={cfg.N} D={cfg.D} E={cfg.E} K={cfg.K} F={cfg.F}", flush=True)
    L = Layer(cfg, padded=padded)
    p = L.p
    moe.route(p, L.x, L.w_router, L.bias, L.logits, L.ids, L.w)
    moe.permute(p, L.x, L.ids, L.counts, L.offsets, L.row_token, L.slot_row, L.x_perm, L.ws)
    qg, qu, qd = _fp8_weights(L)
    moe.expert_gateup_fp8(p, L.x_perm, L.offsets, qg, qu, L.h)
    moe.expert_down_fp8(p, L.h, L.offsets, qd, L.out_perm)
    moe.unpermute_combine(p, L.out_perm, L.slot_row, L.w, L.y)
    torch.cuda.synchronize()
    check_routing(L)
    offsets, row_token, slot_row = check_permutation(L)
    # the oracle quantises the same bf16 weights itself
    og = check_quantized(qg, bits(L.w_gate), "w_gate")
    ou = check_quantized(qu, bits(L.w_up), "w_up")
    od = check_quantized(qd, bits(L.w_down), "w_down")
    h_ref, out_ref = O.expert_ffn_fp8(bits(L.x_perm), offsets, og, ou, od)
    covered = np.zeros(L.R, dtype=bool)
    for e in range(cfg.E):
        covered[offsets[e]:offsets[e + 1]] = True
    h8 = bits(L.h)
    out8 = bits(L.out_perm)
    assert_fp_close(O.bf16_to_f64(h8)[covered], h_ref[covered], "h (fp8)")
    assert_fp_close(O.bf16_to_f64(out8)[covered], out_ref[covered], "out_perm (fp8)")
    if padded:
        assert np.all(O.bf16_to_f64(out8)[row_token < 0] == 0)
    y8 = O.bf16_to_f64(bits(L.y))
    x_bits, wr, bias = L.host_inputs()
    deq = [O.dequantize_fp8_bits(*q) for q in (og, ou, od)]
    ref = O.forward(x_bits, wr, bias, *deq, cfg.K, cfg.gating,
                    cap=(L.cap if padded else None), logits=np_(L.logits))
    assert_fp_close(y8, ref["y"], "y (fp8 layer)")
    # property: the FP8 kernels equal the bf16 kernels on the dequantised weights
    wg, wu, wd = (_bits_tensor(d) for d in deq)
    h16 = torch.empty_like(L.h)
    out16 = torch.empty_like(L.out_perm)
    moe.expert_gateup(p, L.x_perm, L.offsets, wg, wu, h16)
    moe.expert_down(p, h16, L.offsets, wd, out16)
    torch.cuda.synchronize()
    assert np.array_equal(bits(h16)[covered], h8[covered]), "h: fp8 vs bf16 on dequantised"
    assert np.array_equal(bits(out16)[covered], out8[covered]), "out: fp8 vs bf16 on dequantised"
    # moe_grouped_ffn_fp8 and moe_forward_fp8 run the same kernels
    out2 = torch.empty_like(L.out_perm)
    moe.grouped_ffn_fp8(p, L.x_perm, L.offsets, qg, qu, qd, out2, None, L.ws)
    y2 = torch.empty_like(L.y)
    moe.forward_fp8(p, L.x, L.w_router, L.bias, qg, qu, qd, y2, L.ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out2)[covered], out8[covered])
    assert torch.equal(y2.view(torch.int16), L.y.view(torch.int16))
