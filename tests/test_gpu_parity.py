"""GPU parity: every ABI call against the CPU oracle on seeded inputs.

Bars: routing ids, counts, offsets and the permutation bit-exact (selection
compared on identical fp32 logits); x_perm bit-exact; logits within the fp32
dot-product error bound; router weights within 1e-6; h, out_perm and y within
max|d| <= 1e-2 * max|ref| and per-element rtol 2e-2 (bf16 storage, fp32
accumulation against the oracle's float64).
"""
import numpy as np
import pytest
import torch

import moe_synth as ms
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

from gpu_layer import (DEV, SMALL, Layer, assert_fp_close, assert_logits_bound, bits,  # noqa: E402
                       check_permutation, check_routing, np_, sample_tokens,
                       check_sampled_outputs)
import mixture_experts_layer_level_amd as moe  # noqa: E402

@pytest.mark.parametrize("name", list(SMALL))
def test_staged_path_small(name):
    cfg = SMALL[name]
    padded = cfg.capacity is not None
    print(f"[staged] {name} N={cfg.N} D={cfg.D} E={cfg.E} K={cfg.K} F={cfg.F}", flush=True)
    L = Layer(cfg, padded=padded)
    L.staged()
    check_routing(L)
    offsets, row_token, slot_row = check_permutation(L)
    if name == "empty_experts":
        assert (np_(L.counts) == 0).any()
    xg = bits(L.x)
    assert np.array_equal(bits(L.x_perm), O.gather_rows(xg, row_token)), "x_perm"
    # FFN on the GPU's own (bit-exact) x_perm and offsets
    wg, wu, wd = bits(L.w_gate), bits(L.w_up), bits(L.w_down)
    h_ref, out_ref = O.expert_ffn(bits(L.x_perm), offsets, wg, wu, wd)
    covered = np.zeros(L.R, dtype=bool)
    for e in range(cfg.E):
        covered[offsets[e]:offsets[e + 1]] = True
    assert_fp_close(O.bf16_to_f64(bits(L.h))[covered], h_ref[covered], "h")
    out_gpu = O.bf16_to_f64(bits(L.out_perm))
    assert_fp_close(out_gpu[covered], out_ref[covered], "out_perm")
    if padded:
        assert np.all(out_gpu[row_token < 0] == 0), "padding rows of out_perm must be zero"
    # combine on the GPU's own out_perm
    y_ref = O.combine(out_gpu, slot_row, np_(L.w))
    y = O.bf16_to_f64(bits(L.y))
    assert_fp_close(y, y_ref, "y (combine)")
    assert np.mean(y == y_ref) > 0.97
    # whole layer against the oracle (selection on the same fp32 logits)
    x_bits, wr, bias = L.host_inputs()
    ref = O.forward(x_bits, wr, bias, wg, wu, wd, cfg.K, cfg.gating,
                    cap=(L.cap if padded else None), logits=np_(L.logits))
    assert_fp_close(y, ref["y"], "y (layer)")
    # moe_forward runs the same kernels (the router in its split form on the
    # workspace, bit-identical by construction): bit-identical to the staged
    # calls, routing outputs included
    y2 = torch.empty_like(L.y)
    L.forward(y2)
    assert torch.equal(y2.view(torch.int16), L.y.view(torch.int16))
    outs = {k: torch.full_like(getattr(L, k), -7) for k in ("logits", "ids", "w", "counts",
                                                            "offsets")}
    moe.forward(L.p, L.x, L.w_router, L.bias, L.w_gate, L.w_up, L.w_down, y2, L.ws,
                logits=outs["logits"], topk_ids=outs["ids"], topk_weights=outs["w"],
                counts=outs["counts"], offsets=outs["offsets"])
    torch.cuda.synchronize()
    for k, v in outs.items():
        assert torch.equal(v.view(torch.uint8), getattr(L, k).view(torch.uint8)), k


@pytest.mark.parametrize("E,K,kind", [(3, 1, "ties"), (8, 2, "ties"), (64, 8, "zeros_nan"),
                                      (256, 8, "random"), (1000, 5, "ties"), (128, 64, "random")])
@pytest.mark.parametrize("gating", ["softmax", "sigmoid"])
def test_route_on_given_logits(E, K, kind, gating):
    """moe_route with x = NULL: selection and weights on caller-given logits."""
    rng = np.random.default_rng(E * 131 + K)
    N = 777
    lg = rng.standard_normal((N, E)).astype(np.float32)
    if kind == "ties":
        lg = (np.round(lg * 2) / 2).astype(np.float32)
    elif kind == "zeros_nan":
        lg = np.round(lg).astype(np.float32)
        lg[rng.random((N, E)) < 0.2] = -0.0
        lg[rng.random((N, E)) < 0.05] = np.nan
    bias = (np.round(rng.standard_normal(E) * 4) / 8).astype(np.float32)
    p = moe.problem(N, 64, 64, E, K, gating)
    logits = torch.from_numpy(lg).to(DEV)
    ids = torch.empty(N, K, dtype=torch.int32, device=DEV)
    w = torch.empty(N, K, dtype=torch.float32, device=DEV)
    moe.route(p, None, None, torch.from_numpy(bias).to(DEV), logits, ids, w)
    torch.cuda.synchronize()
    ids_ref, w_ref = O.route_from_logits(lg, bias, K, gating)
    assert np.array_equal(np_(ids), ids_ref)
    assert np.abs(np_(w).astype(np.float64) - w_ref).max() <= 1e-6


@pytest.mark.parametrize("N,E,K,cap", [(1, 1, 1, None), (1000, 3, 2, None), (4097, 256, 8, None),
                                       (333, 1024, 6, None), (2500, 64, 2, (5, 4)),
                                       (999, 8, 3, (1, 3)), (64, 128, 8, (1, 1)),
                                       # at and just past the one-workgroup limit of 1024 slots
                                       (128, 64, 8, None), (129, 64, 8, None),
                                       (100, 1024, 10, None), (512, 2, 2, (1, 2)),
                                       (60, 16, 12, None)])
def test_permute_random_routing(N, E, K, cap):
    rng = np.random.default_rng(N + E)
    # skewed, distinct experts per token
    p_e = rng.dirichlet(np.full(E, 0.3))
    ids = np.stack([rng.choice(E, size=K, replace=False, p=p_e) for _ in range(N)]).astype(np.int32)
    D = 64
    x = torch.randn(N, D, device=DEV).to(torch.bfloat16)
    p = moe.problem(N, D, 64, E, K, "softmax", cap)
    R, c = moe.permuted_rows(p)
    g = lambda *s: torch.empty(*s, dtype=torch.int32, device=DEV)
    counts, offsets, row_token, slot_row = g(E), g(E + 1), g(R), g(N * K)
    x_perm = torch.empty(R, D, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(moe.workspace_size(p), dtype=torch.uint8, device=DEV)
    moe.permute(p, x, torch.from_numpy(ids).to(DEV), counts, offsets, row_token, slot_row,
                x_perm, ws)
    torch.cuda.synchronize()
    ref = O.permute(ids, E, c if cap else None)
    for got, exp, nm in zip((counts, offsets, row_token, slot_row), ref,
                            ("counts", "offsets", "row_token", "slot_row")):
        assert np.array_equal(np_(got), exp), nm
    assert np.array_equal(bits(x_perm), O.gather_rows(bits(x), ref[2]))
    # x_perm = NULL: the same routing tables (padding rows of row_token -1
    # included), no row copy
    for t in (counts, offsets, row_token, slot_row):
        t.fill_(12345)
    moe.permute(p, x, torch.from_numpy(ids).to(DEV), counts, offsets, row_token, slot_row,
                None, ws)
    torch.cuda.synchronize()
    for got, exp, nm in zip((counts, offsets, row_token, slot_row), ref,
                            ("counts", "offsets", "row_token", "slot_row")):
        assert np.array_equal(np_(got), exp), nm + " (x_perm NULL)"


def test_deterministic_reruns():
    L = Layer(SMALL["ragged"])
    L.staged()
    first = [t.clone() for t in (L.ids, L.slot_row, L.row_token, L.y)]
    for _ in range(2):
        L.staged()
        for a, b in zip(first, (L.ids, L.slot_row, L.row_token, L.y)):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_generator_is_device_independent():
    a = ms.normal_bf16(100003, 0.7, 99, 3, offset=12345, device=DEV).cpu()
    b = ms.normal_bf16(100003, 0.7, 99, 3, offset=12345, device="cpu")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("E,scale,decay,step", [(1, 10, 0.99, 0.1), (8, 100, 0.99, 0.1),
                                                (256, 40, 0.9, -0.05), (1024, 3, 0.5, 0.1),
                                                (64, 0, 0.99, 0.1)])
def test_routing_stats(E, scale, decay, step):
    """moe_routing_stats against the oracle.  Bounds from the fp32 operations:
    ema: a divide, two products and a sum (<= 8 roundings, relative); bias:
    frac = ema / (tree sum of <= 1024 positive terms) is within 24u
    relative, so |d bias| <= |step| (E frac 24u + 2u) + 2u |bias|."""
    rng = np.random.default_rng(E + scale)
    counts = rng.integers(0, scale + 1, E).astype(np.int32)
    ema0 = rng.dirichlet(np.ones(E)).astype(np.float32)
    bias0 = rng.standard_normal(E).astype(np.float32)
    c_d = torch.from_numpy(counts).to(DEV)
    ema_d = torch.from_numpy(ema0).to(DEV)
    bias_d = torch.from_numpy(bias0).to(DEV)
    moe.routing_stats(E, c_d, ema_d, bias_d, decay, step)
    torch.cuda.synchronize()
    ema_ref, bias_ref = O.routing_stats(counts, ema0, bias0, decay, step)
    u = 2.0 ** -24
    assert np.all(np.abs(np_(ema_d) - ema_ref) <= 8 * u * np.abs(ema_ref) + 1e-30)
    frac = ema_ref / ema_ref.sum()
    tol = abs(step) * (E * frac * 24 * u + 2 * u) + 2 * u * np.abs(bias_ref)
    assert np.all(np.abs(np_(bias_d) - bias_ref) <= tol)
    if counts.sum() == 0:
        assert np.array_equal(np_(ema_d), ema0) and np.array_equal(np_(bias_d), bias0)


def test_routing_stats_from_a_layer():
    """Fed by the expert_counts of a real permute, ten updates in a row track
    the float64 oracle run on the same counts."""
    L = Layer(SMALL["decode_like"])
    L.staged()
    E = L.cfg.E
    ema_d = torch.full((E,), 1.0 / E, dtype=torch.float32, device=DEV)
    bias_d = torch.zeros(E, dtype=torch.float32, device=DEV)
    ema, bias = np.full(E, 1.0 / E), np.zeros(E)
    counts = np_(L.counts)
    for _ in range(10):
        moe.routing_stats(E, L.counts, ema_d, bias_d)
        torch.cuda.synchronize()
        ema, bias = O.routing_stats(counts, ema, bias)
    assert np.allclose(np_(ema_d), ema, rtol=1e-5, atol=1e-9)
    assert np.allclose(np_(bias_d), bias, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("N,D,E,K,gating", [(64, 2048, 128, 8, "softmax"), (17, 640, 45, 3, "sigmoid"),
                                            (100, 1088, 48, 4, "softmax"), (1, 64, 8, 2, "softmax"),
                                            (300, 4096, 8, 2, "softmax"),
                                            # LDS-staged 128 x 256 tiles: a ragged last token
                                            # tile, two expert tiles, a single k part
                                            (1100, 640, 256, 8, "sigmoid"),
                                            (2048, 1088, 512, 6, "softmax"),
                                            (1024, 64, 256, 2, "softmax")])
def test_route_split_form_is_bit_identical(N, D, E, K, gating):
    """moe_route given a workspace runs the router GEMM split over more
    workgroups and sums the partial logits in the unsplit kernel's order:
    logits, ids and weights bit for bit those of the call without one, and
    logits within the fp32 bound of the exact dot products."""
    cfg = ms.MoEConfig("r", N=N, D=D, E=E, K=K, F=64, gating=gating, seed=N + D + E)
    inp = ms.make_inputs(cfg, device=DEV, with_experts=False)
    p = moe.problem(N, D, 64, E, K, gating)
    out = []
    for ws in (None, torch.empty(moe.workspace_size(p), dtype=torch.uint8, device=DEV)):
        lg = torch.full((N, E), float("nan"), device=DEV)
        ids = torch.empty(N, K, dtype=torch.int32, device=DEV)
        w = torch.empty(N, K, device=DEV)
        moe.route(p, inp["x"], inp["w_router"], None, lg, ids, w, ws)
        torch.cuda.synchronize()
        out.append((lg, ids, w))
    for a, b in zip(*out):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                           b.view(torch.int32) if b.dtype == torch.float32 else b)
    assert_logits_bound(np_(out[1][0]), bits(inp["x"]), np_(inp["w_router"]))
