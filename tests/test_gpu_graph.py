"""The layer captured as a HIP graph: every replay equals the eager result.

The library allocates nothing, issues no memset and never synchronises the
host, so moe_forward and the staged calls can be captured.  Each graph is
replayed several times with eager work of the program (the same layer run
eagerly into other buffers, output clears, host synchronisations) between the
replays, and every replay is compared with the eager result bit for bit.
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

# a split-ring shape, the decode-sized tiles, a padded layout
CASES = [("large_tiles", False), ("decode_like", False), ("padded", True),
         ("qwen3_decode", False)]


def _cfg(name):
    return SMALL[name] if name in SMALL else ms.CONFIGS[name]


@pytest.mark.parametrize("name,padded", CASES)
def test_forward_graph_replays_match_eager(name, padded):
    L = Layer(_cfg(name), padded=padded)
    N, D = L.cfg.N, L.cfg.D
    y_eager = torch.empty(N, D, dtype=torch.bfloat16, device=DEV)
    L.forward(y_eager)
    ref = bits(y_eager)

    y = torch.zeros(N, D, dtype=torch.bfloat16, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.forward(L.p, L.x, L.w_router, L.bias, L.w_gate, L.w_up, L.w_down, y, L.ws)
    torch.cuda.synchronize()
    assert not bits(y).any(), "capture must not run the kernels"
    other = torch.empty_like(y_eager)
    for rep in range(4):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(y), ref), f"replay {rep} differs from the eager forward"
        # eager work of the program between replays, on the same workspace
        L.forward(other)
        assert np.array_equal(bits(other), ref)


@pytest.mark.parametrize("name,padded", CASES[:3])
def test_staged_graph_replays_match_eager(name, padded):
    L = Layer(_cfg(name), padded=padded)
    L.staged()
    ref = {k: getattr(L, k).clone() for k in ("logits", "ids", "w", "counts", "offsets",
                                               "row_token", "slot_row", "h", "y")}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        p = L.p
        moe.route(p, L.x, L.w_router, L.bias, L.logits, L.ids, L.w, L.ws)
        moe.permute(p, L.x, L.ids, L.counts, L.offsets, L.row_token, L.slot_row, L.x_perm,
                    L.ws)
        moe.expert_gateup(p, L.x_perm, L.offsets, L.w_gate, L.w_up, L.h)
        moe.expert_down(p, L.h, L.offsets, L.w_down, L.out_perm)
        moe.unpermute_combine(p, L.out_perm, L.slot_row, L.w, L.y)
    torch.cuda.synchronize()
    for rep in range(3):
        for k in ref:
            getattr(L, k).fill_(-1 if k != "y" else 0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(getattr(L, k).view(torch.uint8), v.view(torch.uint8)), \
                f"replay {rep}: {k} differs from the eager staged path"
        L.staged()   # eager work between the replays


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


@pytest.mark.parametrize("kind", ["fp8", "fused", "gelu", "packed", "packed_decode",
                                  "fp8_packed_decode"])
def test_forward_variants_graph_replays_match_eager(kind):
    """moe_forward_fp8 (split-ring-sized rows), moe_forward_fused,
    moe_forward_gelu, moe_forward_packed (split-ring and decode-sized rows)
    and moe_forward_fp8_packed (decode-sized rows) captured once and replayed
    with eager calls between."""
    if kind == "gelu":
        from gpu_layer import GeluLayer
        L = GeluLayer(ms.CONFIGS["gelu_tiny"])
        i = L.inp

        def call(out):
            moe.forward_gelu(L.p, i["x"], i["w_proj"], i["b_proj"], i["w_out"], i["b_out"],
                             i["w1"], i["b1"], i["w2"], i["b2"], out, L.ws)
        N, D = L.cfg.N, L.cfg.D
    elif kind == "fp8_packed_decode":
        L = Layer(ms.CONFIGS["qwen3_decode"])
        q = [_quantize(w) for w in (L.w_gate, L.w_up, L.w_down)]
        gu8 = torch.empty(moe.packed_weight_size(L.p, moe.PACK_GATEUP_FP8), dtype=torch.uint8,
                          device=DEV)
        moe.pack_weights_fp8(L.p, moe.PACK_GATEUP_FP8, q[0][0], q[1][0], gu8)
        dn8 = torch.empty(moe.packed_weight_size(L.p, moe.PACK_DOWN_FP8), dtype=torch.uint8,
                          device=DEV)
        moe.pack_weights_fp8(L.p, moe.PACK_DOWN_FP8, q[2][0], None, dn8)

        def call(out):
            moe.forward_fp8_packed(L.p, L.x, L.w_router, L.bias, gu8, q[0][1], q[1][1], dn8,
                                   q[2][1], out, L.ws)
        N, D = L.cfg.N, L.cfg.D
    elif kind.startswith("packed"):
        L = Layer(ms.CONFIGS["qwen3_decode"] if kind == "packed_decode" else SMALL["large_tiles"])
        gu = _pack(L.p, moe.PACK_GATEUP, L.w_gate, L.w_up)
        dn = _pack(L.p, moe.PACK_DOWN, L.w_down)

        def call(out):
            moe.forward_packed(L.p, L.x, L.w_router, L.bias, gu, dn, out, L.ws)
        N, D = L.cfg.N, L.cfg.D
    else:
        L = Layer(SMALL["mid_tiles" if kind == "fused" else "large_tiles"])
        if kind == "fp8":
            q = [_quantize(w) for w in (L.w_gate, L.w_up, L.w_down)]

            def call(out):
                moe.forward_fp8(L.p, L.x, L.w_router, L.bias, q[0], q[1], q[2], out, L.ws)
        else:
            def call(out):
                moe.forward_fused(L.p, L.x, L.w_router, L.bias, L.w_gate, L.w_up, L.w_down,
                                  out, L.ws)
        N, D = L.cfg.N, L.cfg.D
    y_eager = torch.empty(N, D, dtype=torch.bfloat16, device=DEV)
    call(y_eager)
    torch.cuda.synchronize()
    ref = bits(y_eager)
    y = torch.zeros(N, D, dtype=torch.bfloat16, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(y)
    torch.cuda.synchronize()
    other = torch.empty_like(y)
    for rep in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(y), ref), f"{kind}: replay {rep} differs from eager"
        call(other)
        torch.cuda.synchronize()
        assert np.array_equal(bits(other), ref)
    if kind == "fused":
        off = moe.fused_error_offset(L.p, whole_layer=True)
        assert int(L.ws[off:off + 4].view(torch.int32).item()) == 0
    if kind.startswith("packed"):
        y_unpacked = torch.empty_like(y)
        L.forward(y_unpacked)
        assert np.array_equal(bits(y_unpacked), ref), "packed and unpacked layers differ"
