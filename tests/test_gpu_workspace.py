"""The forward entry points' workspace.

One layout serves every forward call, and buffers whose lifetimes do not
overlap share memory in it: the routing scratch, x_perm and out_perm one
region; the permutation's scratch, h and the fused launch's h and counters
another.  So no result may depend on what the workspace held before a call.
Each forward below runs on a workspace cleared to zero bytes and on one
filled with 0xFF bytes (NaN patterns in every float view, -1 in every
integer one), after another entry point has used it, and must give the same
y bit for bit, equal to the staged calls on buffers of their own.
"""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import mixture_experts_layer_level_amd as moe  # noqa: E402
import moe_synth as ms  # noqa: E402
from gpu_layer import DEV, SMALL, GeluLayer, Layer, bits  # noqa: E402

pytestmark = pytest.mark.gpu


def _quantize(w):
    rows, cols = w.shape[-2], w.shape[-1]
    codes = torch.empty(w.shape, dtype=torch.uint8, device=DEV)
    scales = torch.empty(w.shape[0], rows // 32, cols // 32, 32, dtype=torch.uint8, device=DEV)
    moe.quantize_fp8(w.numel() // cols, cols, w, codes, scales)
    return codes, scales


def _pack(p, kind, w0, w1=None):
    buf = torch.empty(moe.packed_weight_size(p, kind) // 2, dtype=torch.bfloat16, device=DEV)
    moe.pack_weights(p, kind, w0, w1, buf)
    return buf


def _runs(call, ws, other):
    """y of `call` on a zeroed workspace, on an all-ones one, and after
    `other` (another entry point) has used the workspace."""
    out = []
    for fill in (0x00, 0xFF, None):
        if fill is None:
            other()
        else:
            ws.fill_(fill)
        y = call()
        torch.cuda.synchronize()
        out.append(bits(y))
    return out


# split-ring tiles, small tiles, 128-row tiles, padded layouts (x_perm and
# out_perm then share memory), wide rows
SHAPES = [("large_tiles", False), ("decode_like", False), ("mid_tiles", False),
          ("padded", True), ("wide_rows_padded", True), ("many_large_experts", False)]


@pytest.mark.parametrize("name,padded", SHAPES)
def test_forward_independent_of_workspace_contents(name, padded):
    L = Layer(SMALL[name], padded=padded)
    L.staged()
    ref = bits(L.y)
    p = L.p
    y = torch.empty_like(L.y)

    def fwd():
        moe.forward(p, L.x, L.w_router, L.bias, L.w_gate, L.w_up, L.w_down, y, L.ws)
        return y

    def fused():
        yf = torch.empty_like(L.y)
        moe.forward_fused(p, L.x, L.w_router, L.bias, L.w_gate, L.w_up, L.w_down, yf, L.ws)
        return yf

    other = fwd if padded else fused   # the fused launch takes contiguous layouts only
    for i, got in enumerate(_runs(fwd, L.ws, other)):
        assert np.array_equal(got, ref), f"moe_forward run {i} differs from the staged calls"
    if not padded:
        for i, got in enumerate(_runs(fused, L.ws, fwd)):
            assert np.array_equal(got, ref), f"moe_forward_fused run {i} differs"
        gu = _pack(p, moe.PACK_GATEUP, L.w_gate, L.w_up)
        dn = _pack(p, moe.PACK_DOWN, L.w_down)

        def packed():
            moe.forward_packed(p, L.x, L.w_router, L.bias, gu, dn, y, L.ws)
            return y
        for i, got in enumerate(_runs(packed, L.ws, fused)):
            assert np.array_equal(got, ref), f"moe_forward_packed run {i} differs"


@pytest.mark.parametrize("name,padded", [("large_tiles", False), ("padded", True),
                                         ("two_big_experts", False),
                                         ("padded_small_rows", True)])
def test_fp8_forward_independent_of_workspace_contents(name, padded):
    L = Layer(SMALL[name], padded=padded)
    q = [_quantize(w) for w in (L.w_gate, L.w_up, L.w_down)]
    y = torch.empty_like(L.y)

    def fwd8():
        moe.forward_fp8(L.p, L.x, L.w_router, L.bias, q[0], q[1], q[2], y, L.ws)
        return y

    def fwd():
        moe.forward(L.p, L.x, L.w_router, L.bias, L.w_gate, L.w_up, L.w_down,
                    torch.empty_like(y), L.ws)
    runs = _runs(fwd8, L.ws, fwd)
    for i, got in enumerate(runs[1:], 1):
        assert np.array_equal(got, runs[0]), f"moe_forward_fp8 run {i} differs from run 0"
    if L.cfg.D % 128 == 0 and L.cfg.F % 128 == 0:
        gu8 = torch.empty(moe.packed_weight_size(L.p, moe.PACK_GATEUP_FP8), dtype=torch.uint8,
                          device=DEV)
        moe.pack_weights_fp8(L.p, moe.PACK_GATEUP_FP8, q[0][0], q[1][0], gu8)
        dn8 = torch.empty(moe.packed_weight_size(L.p, moe.PACK_DOWN_FP8), dtype=torch.uint8,
                          device=DEV)
        moe.pack_weights_fp8(L.p, moe.PACK_DOWN_FP8, q[2][0], None, dn8)

        def fwd8p():
            moe.forward_fp8_packed(L.p, L.x, L.w_router, L.bias, gu8, q[0][1], q[1][1], dn8,
                                   q[2][1], y, L.ws)
            return y
        for i, got in enumerate(_runs(fwd8p, L.ws, fwd)):
            assert np.array_equal(got, runs[0]), f"moe_forward_fp8_packed run {i} differs"


@pytest.mark.parametrize("padded", [False, True])
def test_gelu_forward_independent_of_workspace_contents(padded):
    cfg = ms.CONFIGS["gelu_tiny"]
    if padded:
        cfg = cfg.scaled(capacity=(1, 2))   # half the mean rows per expert: many drops
    L = GeluLayer(cfg, padded=padded)
    L.staged()
    ref = bits(L.y)
    y = torch.empty_like(L.y)

    def fwd():
        L.forward(y)
        return y

    def staged_route():
        i = L.inp
        moe.route_mlp(L.p, i["x"], i["w_proj"], i["b_proj"], i["w_out"], i["b_out"], L.logits,
                      L.ids, L.w, L.ws)
    for i, got in enumerate(_runs(fwd, L.ws, staged_route)):
        assert np.array_equal(got, ref), f"moe_forward_gelu run {i} differs from the staged calls"
