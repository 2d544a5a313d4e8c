"""Packed weights: bf16 stacks and FP8 codes.

moe_pack_weights and moe_pack_weights_fp8 are checked against the layout
that include/moe.h documents, rebuilt here with torch indexing on the CPU.
The packed entry points are checked against the unpacked ones, bit for bit,
on every tile shape of the path: split rings, 256-, 128- and 32-row rings
(for FP8 codes the 128-deep rings and the 256-row ring's 64-deep stages,
half an image each), register-staged tiles, padded layouts, more experts
than the split rings' work list holds, and the full-size workloads.
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
from gpu_layer import DEV, SMALL, Layer, bits  # noqa: E402

pytestmark = pytest.mark.gpu


def packed_reference(w0: torch.Tensor, w1, gateup: bool) -> np.ndarray:
    """The documented layout: panels of 128 columns of h (gate/up: gate rows
    in even 32-row blocks, up rows in odd ones) or 256 output columns, 64-deep
    stages, row r at bytes [128 r, 128 r + 128) of a 32 KB stage with chunk c
    at position c ^ ((r / 2) % 8); rows past the matrix repeat its last row."""
    w0 = w0.cpu().view(torch.int16)
    w1 = None if w1 is None else w1.cpu().view(torch.int16)
    E, nout, kd = w0.shape
    cols = 128 if gateup else 256
    ntiles, nk = -(-nout // cols), kd // 64
    r = torch.arange(256)
    pos = torch.arange(8)
    src_chunk = pos[None, :] ^ ((r[:, None] // 2) % 8)            # [256, 8]
    out = torch.empty(E, ntiles, nk, 256, 8, 8, dtype=torch.int16)
    for t in range(ntiles):
        if gateup:
            blk = r // 32
            row = (t * 128 + (blk // 2) * 32 + r % 32).clamp(max=nout - 1)
            sel = torch.where((blk % 2 == 1)[None, :, None], w1[:, row, :], w0[:, row, :])
        else:
            row = (t * 256 + r).clamp(max=nout - 1)
            sel = w0[:, row, :]
        st = sel.view(E, 256, nk, 8, 8).permute(0, 2, 1, 3, 4)    # [E, nk, 256, chunk, 8]
        idx = src_chunk[None, None, :, :, None].expand(E, nk, 256, 8, 8)
        out[:, t] = torch.gather(st, 3, idx)
    return out.numpy().view(np.uint16).reshape(-1)


def _pack(p, kind, w0, w1=None):
    n = moe.packed_weight_size(p, kind)
    buf = torch.empty(n // 2, dtype=torch.bfloat16, device=DEV)
    moe.pack_weights(p, kind, w0, w1, buf)
    return buf


# ragged F (gate/up panels past F) and D (down panels past D), a single
# 64-deep stage, and a D of 320 (five stages)
@pytest.mark.parametrize("name", ["ragged", "tiny", "short_k_large_tiles", "mid_tiles"])
def test_pack_layout(name):
    cfg = SMALL[name] if name in SMALL else ms.CONFIGS[name]
    L = Layer(cfg)
    gu = _pack(L.p, moe.PACK_GATEUP, L.w_gate, L.w_up)
    dn = _pack(L.p, moe.PACK_DOWN, L.w_down)
    torch.cuda.synchronize()
    assert np.array_equal(bits(gu), packed_reference(L.w_gate, L.w_up, True)), "gate/up layout"
    assert np.array_equal(bits(dn), packed_reference(L.w_down, None, False)), "down layout"


CASES = [(n, False) for n in SMALL if not n.startswith("padded")] + \
        [("padded", True), ("padded_small_rows", True), ("wide_rows_padded", True)]


@pytest.mark.parametrize("name,padded", CASES)
def test_packed_calls_match_unpacked(name, padded):
    L = Layer(SMALL[name], padded=padded)
    L.staged()
    p = L.p
    gu = _pack(p, moe.PACK_GATEUP, L.w_gate, L.w_up)
    dn = _pack(p, moe.PACK_DOWN, L.w_down)
    h = torch.full_like(L.h, -1.0)
    moe.expert_gateup_packed(p, L.x_perm, L.offsets, gu, h)
    out = torch.full_like(L.out_perm, -1.0)
    moe.expert_down_packed(p, L.h, L.offsets, dn, out)
    torch.cuda.synchronize()
    R = int(L.offsets[-1].item()) if not padded else L.R
    assert np.array_equal(bits(h[:R]), bits(L.h[:R])), "h"
    assert np.array_equal(bits(out[:R]), bits(L.out_perm[:R])), "out_perm"
    if not padded:
        h1, h2 = torch.full_like(L.h, -1.0), torch.full_like(L.h, -1.0)
        try:
            moe.expert_gateup_gathered(p, L.x, L.row_token, L.offsets, L.w_gate, L.w_up, h1)
        except moe.MoEError:
            # tiles that cannot gather: the packed call refuses them as well
            with pytest.raises(moe.MoEError):
                moe.expert_gateup_packed_gathered(p, L.x, L.row_token, L.offsets, gu, h2)
        else:
            moe.expert_gateup_packed_gathered(p, L.x, L.row_token, L.offsets, gu, h2)
            torch.cuda.synchronize()
            assert np.array_equal(bits(h2[:R]), bits(h1[:R])), "h (gathered)"
    y = torch.zeros_like(L.y)
    moe.forward_packed(p, L.x, L.w_router, L.bias, gu, dn, y, L.ws)
    y_ref = torch.zeros_like(L.y)
    L.forward(y_ref)
    assert np.array_equal(bits(y), bits(y_ref)), "y"
    assert np.array_equal(bits(y), bits(L.y)), "y against the staged path"


@pytest.mark.parametrize("name,padded", [("deepseek_v3", False), ("qwen3_decode", False),
                                         ("mixtral", False), ("hot_skew", True)])
def test_packed_forward_full_size(name, padded):
    """The layer at full size: moe_forward_packed's y equals moe_forward's bit
    for bit (which the full-size parity tests compare with the oracle)."""
    L = Layer(ms.CONFIGS[name], padded=padded)
    p = L.p
    gu = _pack(p, moe.PACK_GATEUP, L.w_gate, L.w_up)
    dn = _pack(p, moe.PACK_DOWN, L.w_down)
    y = torch.zeros_like(L.y)
    moe.forward_packed(p, L.x, L.w_router, L.bias, gu, dn, y, L.ws)
    y_ref = torch.zeros_like(L.y)
    L.forward(y_ref)
    assert np.array_equal(bits(y), bits(y_ref))


# ---------------------------------------------------------------- packed FP8 codes

def _quantize(w):
    rows, cols = w.shape[-2], w.shape[-1]
    codes = torch.empty(w.shape, dtype=torch.uint8, device=DEV)
    scales = torch.empty(w.shape[0], rows // 32, cols // 32, 32, dtype=torch.uint8, device=DEV)
    moe.quantize_fp8(w.numel() // cols, cols, w, codes, scales)
    return codes, scales


def _pack8(p, kind, c0, c1=None):
    buf = torch.empty(moe.packed_weight_size(p, kind), dtype=torch.uint8, device=DEV)
    moe.pack_weights_fp8(p, kind, c0, c1, buf)
    return buf


FP8_SMALL = {
    # 32-row rings (128-deep stages), 128-row rings, 256-row rings (64-deep
    # stages: two per packed stage image, an odd count of images for down)
    "tiny": SMALL["tiny"],
    "decode_like": SMALL["decode_like"],
    "wide_topk": SMALL["wide_topk"],
    "fp8_mid": ms.MoEConfig("fp8_mid", N=600, D=256, E=8, K=2, F=256, gating="softmax",
                            seed=301),
    "two_big_experts": SMALL["two_big_experts"],
    "fp8_large": ms.MoEConfig("fp8_large", N=1200, D=512, E=4, K=1, F=384, gating="sigmoid",
                              seed=302),
    "many_large_experts": SMALL["many_large_experts"],
}


@pytest.mark.parametrize("name", ["tiny", "two_big_experts", "fp8_large"])
def test_pack_fp8_layout(name):
    """The packed codes against the documented layout: the bf16 one applied
    to pairs of codes, i.e. stages of 128 codes."""
    L = Layer(FP8_SMALL[name])
    (gc, _), (uc, _), (dc, _) = [_quantize(w) for w in (L.w_gate, L.w_up, L.w_down)]
    gu = _pack8(L.p, moe.PACK_GATEUP_FP8, gc, uc)
    dn = _pack8(L.p, moe.PACK_DOWN_FP8, dc)
    torch.cuda.synchronize()
    assert np.array_equal(bits(gu), packed_reference(gc.view(torch.int16), uc.view(torch.int16),
                                                     True)), "gate/up layout"
    assert np.array_equal(bits(dn), packed_reference(dc.view(torch.int16), None, False)), \
        "down layout"


FP8_CASES = [(n, False) for n in FP8_SMALL] + [("padded_small_rows", True)]


@pytest.mark.parametrize("name,padded", FP8_CASES)
def test_packed_fp8_calls_match_unpacked(name, padded):
    cfg = FP8_SMALL.get(name) or SMALL[name]
    L = Layer(cfg, padded=padded)
    L.staged()
    p = L.p
    qg, qu, qd = [_quantize(w) for w in (L.w_gate, L.w_up, L.w_down)]
    gu = _pack8(p, moe.PACK_GATEUP_FP8, qg[0], qu[0])
    dn = _pack8(p, moe.PACK_DOWN_FP8, qd[0])
    R = L.R if padded else int(L.offsets[-1].item())
    h_ref, h = torch.full_like(L.h, -1.0), torch.full_like(L.h, -1.0)
    moe.expert_gateup_fp8(p, L.x_perm, L.offsets, qg, qu, h_ref)
    moe.expert_gateup_fp8_packed(p, L.x_perm, L.offsets, gu, qg[1], qu[1], h)
    o_ref, o = torch.full_like(L.out_perm, -1.0), torch.full_like(L.out_perm, -1.0)
    moe.expert_down_fp8(p, h_ref, L.offsets, qd, o_ref)
    moe.expert_down_fp8_packed(p, h_ref, L.offsets, dn, qd[1], o)
    torch.cuda.synchronize()
    assert np.array_equal(bits(h[:R]), bits(h_ref[:R])), "h"
    assert np.array_equal(bits(o[:R]), bits(o_ref[:R])), "out_perm"
    if not padded:
        h2 = torch.full_like(L.h, -1.0)
        moe.expert_gateup_fp8_packed_gathered(p, L.x, L.row_token, L.offsets, gu, qg[1], qu[1],
                                              h2)
        torch.cuda.synchronize()
        assert np.array_equal(bits(h2[:R]), bits(h_ref[:R])), "h (gathered)"
    y_ref, y = torch.zeros_like(L.y), torch.zeros_like(L.y)
    moe.forward_fp8(p, L.x, L.w_router, L.bias, qg, qu, qd, y_ref, L.ws)
    moe.forward_fp8_packed(p, L.x, L.w_router, L.bias, gu, qg[1], qu[1], dn, qd[1], y, L.ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), bits(y_ref)), "y"


@pytest.mark.parametrize("name,padded", [("deepseek_v3", False), ("qwen3_decode", False),
                                         ("mixtral", False), ("hot_skew", True)])
def test_packed_fp8_forward_full_size(name, padded):
    """The FP8 layer at full size: moe_forward_fp8_packed's y equals
    moe_forward_fp8's bit for bit (the FP8 full-size parity tests compare
    the latter with the oracle)."""
    L = Layer(ms.CONFIGS[name], padded=padded)
    p = L.p
    qg, qu, qd = [_quantize(w) for w in (L.w_gate, L.w_up, L.w_down)]
    gu = _pack8(p, moe.PACK_GATEUP_FP8, qg[0], qu[0])
    dn = _pack8(p, moe.PACK_DOWN_FP8, qd[0])
    y_ref, y = torch.zeros_like(L.y), torch.zeros_like(L.y)
    moe.forward_fp8(p, L.x, L.w_router, L.bias, qg, qu, qd, y_ref, L.ws)
    moe.forward_fp8_packed(p, L.x, L.w_router, L.bias, gu, qg[1], qu[1], dn, qd[1], y, L.ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(y), bits(y_ref))
