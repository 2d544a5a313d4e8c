"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test fixes one part of the oracle to something independent: the pages'
worked example, a closed form, a library routine, an exactly rounded sum, an
invariant of the definition, or brute force on tiny inputs.  CPU only.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special as sps
import torch

import moe_synth as ms
from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _tiny_layer(N, D, E, K, F, seed, bias=False, gating="softmax"):
    cfg = ms.MoEConfig("t", N=N, D=D, E=E, K=K, F=F, gating=gating, seed=seed)
    inp = ms.make_inputs(cfg)
    b = None
    if bias:
        b = ms.zipf_bias(E, 1.2, 0.5, seed).numpy()
    return (cfg, _bits(inp["x"]), inp["w_router"].numpy(), b, _bits(inp["w_gate"]),
            _bits(inp["w_up"]), _bits(inp["w_down"]))


# ---------------------------------------------------------------- permutation

def test_worked_example_contiguous():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    counts, offsets, row_token, slot_row = O.permute(np.array(g["topk_ids"]), g["E"])
    assert offsets.tolist() == g["expert_offsets"]
    for e, seg in enumerate(g["segments"]):
        assert row_token[offsets[e]:offsets[e + 1]].tolist() == seg
    d = g["derived_from_the_segments"]
    assert counts.tolist() == d["expert_counts"]
    assert row_token.tolist() == d["row_token"]
    assert slot_row.tolist() == d["slot_row"]


def test_worked_example_padded():
    g = json.load(open(os.path.join(GOLDEN, "padded_example.json")))
    ids = np.array([[0], [2], [0], [1], [2], [0], [1], [2]])
    for case in g["cases"]:
        num, den = case["capacity_factor"]
        cap = O.capacity(8, 1, 3, num, den)
        assert cap == case["capacity"]
        counts, offsets, row_token, slot_row = O.permute(ids, 3, cap)
        assert offsets.tolist() == [0, cap, 2 * cap, 3 * cap]
        assert row_token.reshape(3, cap).tolist() == case["buffers"]
        dropped = sorted(int(i) for i in np.nonzero(slot_row < 0)[0])
        assert dropped == case["dropped_tokens"]


@pytest.mark.parametrize("N,E,K,seed", [(1, 1, 1, 0), (37, 5, 2, 1), (100, 16, 4, 2),
                                         (64, 8, 8, 3), (50, 300, 6, 4), (3, 40, 3, 5)])
def test_permute_invariants(N, E, K, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(N)])
    counts, offsets, row_token, slot_row = O.permute(ids, E)
    S = N * K
    assert counts.sum() == S and offsets[0] == 0 and offsets[-1] == S
    assert sorted(slot_row.tolist()) == list(range(S))             # bijection onto rows
    assert all(row_token[slot_row[i]] == i // K for i in range(S))
    for e in range(E):                                               # brute-force segment contents
        expect = [n for n in range(N) if e in ids[n]]
        assert row_token[offsets[e]:offsets[e + 1]].tolist() == expect
        assert counts[e] == len(expect)


def test_capacity_formula():
    for (N, K, E, num, den) in [(16384, 2, 64, 5, 4), (8, 1, 3, 3, 2), (7, 3, 5, 5, 4),
                                (1, 1, 64, 5, 4), (4096, 8, 256, 1, 1), (0, 2, 8, 5, 4)]:
        assert O.capacity(N, K, E, num, den) == math.ceil(Fraction(num * N * K, den * E))
    assert O.capacity(16384, 2, 64, 5, 4) == 640


def test_padded_drop_set():
    rng = np.random.default_rng(7)
    N, E, K = 200, 6, 2
    # skewed routing so some experts overflow
    p = np.array([0.5, 0.2, 0.1, 0.1, 0.05, 0.05])
    ids = np.stack([rng.choice(E, size=K, replace=False, p=p) for _ in range(N)])
    cap = O.capacity(N, K, E, 5, 4)
    counts, offsets, row_token, slot_row = O.permute(ids, E, cap)
    flat = ids.reshape(-1)
    assert int((slot_row < 0).sum()) == int(np.maximum(counts - cap, 0).sum())
    for e in range(E):
        slots = [i for i in range(N * K) if flat[i] == e]
        kept = slots[:cap]
        assert [i for i in slots if slot_row[i] >= 0] == kept
        seg = row_token[e * cap:(e + 1) * cap].tolist()
        assert seg == [i // K for i in kept] + [-1] * (cap - len(kept))


# ---------------------------------------------------------------- top-K / weights

def _kpass_argmax(keys, K):
    """Independent selection: K passes, each taking the strictly largest untaken key."""
    N, E = keys.shape
    out = np.empty((N, K), dtype=np.int64)
    for n in range(N):
        taken = set()
        for k in range(K):
            best = None
            for e in range(E):
                if e in taken:
                    continue
                if best is None or keys[n, e] > keys[n, best]:
                    best = e
            taken.add(best)
            out[n, k] = best
    return out


@pytest.mark.parametrize("kind", ["random", "ties", "signed_zero_nan"])
def test_topk_bruteforce(kind):
    rng = np.random.default_rng(11)
    N, E = 60, 12
    if kind == "random":
        keys = rng.standard_normal((N, E)).astype(np.float32)
    elif kind == "ties":
        keys = (np.round(rng.standard_normal((N, E)) * 4) / 4).astype(np.float32)
    else:
        keys = (np.round(rng.standard_normal((N, E)))).astype(np.float32)
        keys[rng.random((N, E)) < 0.2] = -0.0
        keys[rng.random((N, E)) < 0.1] = np.nan
    k_or = O.gating_keys(keys)
    k_ref = np.where(np.isnan(keys), -np.inf, keys).astype(np.float32)
    for K in (1, 3, E):
        assert np.array_equal(O.select_topk(k_or, K), _kpass_argmax(k_ref, K))


def test_tie_breaks_to_lower_id():
    keys = np.array([[1.0, 2.0, 2.0, 0.0, 2.0], [0.0, -0.0, 0.0, -0.0, -1.0]], dtype=np.float32)
    ids = O.select_topk(O.gating_keys(keys), 3)
    assert ids.tolist() == [[1, 2, 4], [0, 1, 2]]


def test_bias_is_added_before_selection():
    logits = np.array([[1.0, 0.5, 0.0]], dtype=np.float32)
    bias = np.array([0.0, 0.75, 0.0], dtype=np.float32)
    ids, w = O.route_from_logits(logits, bias, 1, "softmax")
    assert ids.tolist() == [[1]]
    ids, w = O.route_from_logits(logits, bias, 2, "softmax")
    assert ids.tolist() == [[1, 0]]
    assert abs(w[0, 0] - 1.0 / (1.0 + math.exp(1.0 - 1.25))) < 1e-7


def test_softmax_closed_forms():
    rng = np.random.default_rng(3)
    keys = rng.standard_normal((40, 9)).astype(np.float32)
    ids, w = O.route_from_logits(keys, None, 1, "softmax")
    assert np.all(w == 1.0)
    ids, w = O.route_from_logits(keys, None, 2, "softmax")
    k0 = np.take_along_axis(keys, ids[:, :1].astype(np.int64), 1)[:, 0].astype(np.float64)
    k1 = np.take_along_axis(keys, ids[:, 1:].astype(np.int64), 1)[:, 0].astype(np.float64)
    np.testing.assert_allclose(w[:, 0], 1.0 / (1.0 + np.exp(k1 - k0)), rtol=0, atol=1e-7)
    # K = E is the full softmax over all experts (the classic dense gate)
    ids, w = O.route_from_logits(keys, None, 9, "softmax")
    full = sps.softmax(keys.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(full, ids.astype(np.int64), 1), atol=1e-7)
    np.testing.assert_allclose(w.astype(np.float64).sum(1), 1.0, atol=1e-6)


def test_sigmoid_renorm_closed_forms():
    rng = np.random.default_rng(4)
    keys = rng.standard_normal((40, 16)).astype(np.float32)
    ids, w = O.route_from_logits(keys, None, 1, "sigmoid")
    assert np.all(w == 1.0)
    ids, w = O.route_from_logits(keys, None, 8, "sigmoid")
    s = sps.expit(np.take_along_axis(keys, ids.astype(np.int64), 1).astype(np.float64))
    np.testing.assert_allclose(w, s / s.sum(1, keepdims=True), atol=1e-7)
    np.testing.assert_allclose(w.astype(np.float64).sum(1), 1.0, atol=1e-6)
    # selection on the key equals selection on sigmoid(key) when sigmoid does not collapse
    order = np.argsort(-sps.expit(keys.astype(np.float64)), axis=1, kind="stable")[:, :8]
    assert np.array_equal(ids, order)


# ---------------------------------------------------------------- number formats and router

def test_round_bf16_matches_library_cast():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    # exact halfway cases: dropped 16 bits = 0x8000, kept mantissa bits of both parities
    r = rng.integers(0, 128, 2000).astype(np.uint32)
    ex = rng.integers(100, 150, 2000).astype(np.uint32) << np.uint32(23)
    hw = ex | (r << np.uint32(16)) | np.uint32(0x8000)
    v = np.concatenate([v, hw.view(np.float32), -hw.view(np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f64_to_bf16_bits(v.astype(np.float64)), ref)
    assert np.array_equal(O.bf16_to_f64(ref), torch.from_numpy(v).to(torch.bfloat16).double().numpy())


def test_router_logits_exactly_rounded():
    cfg, x, wr, *_ = _tiny_layer(8, 96, 5, 2, 16, seed=21)
    logits = O.router_logits(x, wr)
    xf = O.bf16_to_f64(x)
    wf = wr.astype(np.float64)
    for n in range(8):
        for e in range(5):
            exact = math.fsum(float(xf[n, d]) * float(wf[e, d]) for d in range(96))
            assert logits[n, e] == np.float32(exact)


# ---------------------------------------------------------------- FFN and combine

def test_swiglu_closed_form():
    D, F = 8, 12
    rng = np.random.default_rng(6)
    x = O.round_bf16(rng.standard_normal((3, D)))
    a = rng.integers(0, D, F)
    b = rng.integers(0, D, F)
    c = rng.integers(0, F, D)
    wg = np.zeros((F, D)); wg[np.arange(F), a] = 1.0
    wu = np.zeros((F, D)); wu[np.arange(F), b] = 2.0
    wd = np.zeros((D, F)); wd[np.arange(D), c] = 0.5
    h, out = O.swiglu_rows(x, O.f64_to_bf16_bits(wg), O.f64_to_bf16_bits(wu), O.f64_to_bf16_bits(wd))
    g = x[:, a]
    href = g * sps.expit(g) * (2.0 * x[:, b])
    np.testing.assert_allclose(h, href, rtol=2 ** -8, atol=0)
    assert np.array_equal(out, O.round_bf16(0.5 * h[:, c]))


def _dense_bruteforce(x, wr, bias, wg, wu, wd, K, gating, cap=None):
    """Every expert on every token, then masked by the routing: no permutation at all."""
    logits, ids, w = O.route(x, wr, bias, K, gating)
    N = x.shape[0]
    E = wr.shape[0]
    xs = O.bf16_to_f64(x)
    outs = np.stack([O.swiglu_rows(xs, wg[e], wu[e], wd[e])[1] for e in range(E)])  # [E,N,D]
    keep = np.ones((N, K), dtype=bool)
    if cap is not None:
        seen = np.zeros(E, dtype=np.int64)
        for n in range(N):
            for k in range(K):
                e = ids[n, k]
                keep[n, k] = seen[e] < cap
                seen[e] += 1
    y = np.zeros((N, x.shape[1]))
    for k in range(K):
        sel = outs[ids[:, k], np.arange(N)]
        y += np.where(keep[:, k:k + 1], w[:, k:k + 1].astype(np.float64) * sel, 0.0)
    return O.round_bf16(y)


@pytest.mark.parametrize("gating,bias,K,cap", [("softmax", False, 2, None), ("sigmoid", False, 3, None),
                                               ("softmax", True, 2, None), ("softmax", True, 2, (5, 4)),
                                               ("softmax", False, 1, None), ("sigmoid", True, 4, (1, 1))])
def test_sparse_equals_dense_bruteforce(gating, bias, K, cap):
    N, D, E, F = 24, 32, 6, 48
    cfg, x, wr, b, wg, wu, wd = _tiny_layer(N, D, E, K, F, seed=31, bias=bias, gating=gating)
    c = O.capacity(N, K, E, *cap) if cap else None
    res = O.forward(x, wr, b, wg, wu, wd, K, gating, cap=c)
    ref = _dense_bruteforce(x, wr, b, wg, wu, wd, K, gating, cap=c)
    np.testing.assert_allclose(res["y"], ref, rtol=2 ** -7, atol=1e-12)
    assert np.mean(res["y"] == ref) > 0.99
    if c is not None:
        pad = res["row_token"] < 0
        assert np.all(res["out_perm"][pad] == 0) and np.all(res["x_perm"][pad] == 0)


def test_wd_scaling_is_exact():
    cfg, x, wr, b, wg, wu, wd = _tiny_layer(16, 32, 4, 2, 40, seed=41)
    y1 = O.forward(x, wr, b, wg, wu, wd, 2, "softmax")["y"]
    wd2 = O.f64_to_bf16_bits(2.0 * O.bf16_to_f64(wd))
    y2 = O.forward(x, wr, b, wg, wu, wd2, 2, "softmax")["y"]
    assert np.array_equal(y2, 2.0 * y1)


def test_expert_relabelling_invariance():
    cfg, x, wr, b, wg, wu, wd = _tiny_layer(20, 32, 5, 2, 24, seed=51, bias=True)
    y1 = O.forward(x, wr, b, wg, wu, wd, 2, "softmax")["y"]
    p = np.array([3, 0, 4, 1, 2])
    y2 = O.forward(x, wr[p], b[p], wg[p], wu[p], wd[p], 2, "softmax")["y"]
    np.testing.assert_allclose(y2, y1, rtol=2 ** -7, atol=1e-12)


def test_token_permutation_equivariance():
    cfg, x, wr, b, wg, wu, wd = _tiny_layer(20, 32, 5, 2, 24, seed=61)
    y1 = O.forward(x, wr, b, wg, wu, wd, 2, "sigmoid")["y"]
    p = np.random.default_rng(0).permutation(20)
    y2 = O.forward(x[p], wr, b, wg, wu, wd, 2, "sigmoid")["y"]
    np.testing.assert_allclose(y2, y1[p], rtol=2 ** -7, atol=1e-12)


def test_k1_combine_is_a_gather():
    cfg, x, wr, b, wg, wu, wd = _tiny_layer(16, 32, 4, 1, 40, seed=71)
    r = O.forward(x, wr, b, wg, wu, wd, 1, "softmax")
    assert np.array_equal(r["y"], r["out_perm"][r["slot_row"]])


def test_degenerate_shapes():
    # N = 0: nothing routed, all offsets zero
    r = O.forward(np.zeros((0, 16), np.uint16), np.zeros((4, 16), np.float32), None,
                  np.zeros((4, 8, 16), np.uint16), np.zeros((4, 8, 16), np.uint16),
                  np.zeros((4, 16, 8), np.uint16), 2, "softmax")
    assert r["y"].shape == (0, 16) and r["expert_offsets"].tolist() == [0] * 5
    # E = 1, K = 1: one segment holding every token in order, weight 1
    cfg, x, wr, b, wg, wu, wd = _tiny_layer(9, 16, 1, 1, 8, seed=81)
    r = O.forward(x, wr, b, wg, wu, wd, 1, "softmax")
    assert r["expert_offsets"].tolist() == [0, 9] and r["row_token"].tolist() == list(range(9))
    assert np.all(r["topk_weights"] == 1.0)
    # K = E: every token visits every expert
    cfg, x, wr, b, wg, wu, wd = _tiny_layer(5, 16, 3, 3, 8, seed=82)
    r = O.forward(x, wr, b, wg, wu, wd, 3, "softmax")
    assert r["expert_counts"].tolist() == [5, 5, 5]


def test_large_capacity_equals_contiguous():
    N, K, E = 30, 2, 5
    cfg, x, wr, b, wg, wu, wd = _tiny_layer(N, 32, E, K, 24, seed=91, bias=True)
    rc = O.forward(x, wr, b, wg, wu, wd, K, "softmax")
    rp = O.forward(x, wr, b, wg, wu, wd, K, "softmax", cap=N)
    assert np.all(rp["slot_row"] >= 0)
    assert np.array_equal(rc["y"], rp["y"])


def test_token_outputs_matches_forward():
    cfg, x, wr, b, wg, wu, wd = _tiny_layer(12, 32, 4, 2, 24, seed=95)
    r = O.forward(x, wr, b, wg, wu, wd, 2, "softmax")
    sel = np.array([0, 3, 7, 11])
    y, _ = O.token_outputs(x[sel], r["topk_ids"][sel], r["topk_weights"][sel],
                           np.ones((4, 2), bool), lambda e: (wg[e], wu[e], wd[e]))
    assert np.array_equal(y, r["y"][sel])


# ---------------------------------------------------------------- workload generator

def test_generator_is_counter_based():
    a = ms.normal_f32(4096, 1.0, 123, 0)
    b = ms.normal_f32(100, 1.0, 123, 0, offset=1000)
    assert torch.equal(a[1000:1100], b)
    assert abs(float(a.mean())) < 0.05 and abs(float(a.std()) - 1.0) < 0.05
    assert not torch.equal(ms.normal_f32(64, 1.0, 123, 1), ms.normal_f32(64, 1.0, 123, 2))


def test_hot_skew_top_expert_share():
    cfg = ms.CONFIGS["hot_skew"]
    n = 1024
    x = _bits(ms.normal_bf16(n * cfg.D, 1.0, cfg.seed, ms.STREAM_X).view(n, cfg.D))
    wr = ms.normal_f32(cfg.E * cfg.D, 1.0 / math.sqrt(cfg.D), cfg.seed, ms.STREAM_WR).view(cfg.E, cfg.D)
    bias = ms.zipf_bias(cfg.E, cfg.zipf_s, cfg.zipf_alpha, cfg.seed).numpy()
    _, ids, _ = O.route(x, wr.numpy(), bias, cfg.K, cfg.gating)
    share = np.bincount(ids.reshape(-1), minlength=cfg.E).max() / ids.size
    assert 0.21 <= share <= 0.29
    assert O.capacity(cfg.N, cfg.K, cfg.E, *cfg.capacity) == 640


# ---------------------------------------------------------------- routing statistics

def test_routing_stats_uniform_is_a_fixed_point():
    """Uniform counts and a uniform EMA: the EMA stays 1/E and the bias moves
    by (E * 1/E - 1) * step = 0 (ybb.press 4.1)."""
    E = 16
    ema, bias = O.routing_stats(np.full(E, 5), np.full(E, 1 / E), np.arange(E) * 0.25)
    assert np.allclose(ema, 1 / E, rtol=0, atol=1e-15)
    assert np.allclose(bias, np.arange(E) * 0.25, rtol=0, atol=1e-15)


def test_routing_stats_single_hot_expert_closed_form():
    """All slots on expert 0, EMA uniform: ema_0 = d/E + (1-d), ema_e = d/E;
    the EMA still sums to 1, so frac = ema and bias_e += (E*ema_e - 1)*step."""
    E, d, st = 8, 0.9, 0.1
    counts = np.zeros(E, dtype=np.int64)
    counts[0] = 40
    ema, bias = O.routing_stats(counts, np.full(E, 1 / E), np.zeros(E), decay=d, step=st)
    want = np.full(E, d / E)
    want[0] += 1 - d
    assert np.allclose(ema, want, rtol=0, atol=1e-15)
    assert np.allclose(bias, (E * want - 1) * st, rtol=0, atol=1e-15)
    assert bias[0] > 0 > bias[1]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_routing_stats_invariants(seed):
    """The EMA is a convex combination (its sum stays 1 when it starts at 1)
    and the bias updates sum to zero over the experts (sum_e (E f_e - 1) = 0);
    scaling the counts changes nothing (only fractions enter)."""
    rng = np.random.default_rng(seed)
    E = int(rng.integers(2, 300))
    counts = rng.integers(0, 50, E)
    counts[0] += 1
    ema0 = rng.dirichlet(np.ones(E))
    bias0 = rng.standard_normal(E)
    ema, bias = O.routing_stats(counts, ema0, bias0, decay=0.97, step=-0.05)
    assert abs(ema.sum() - 1) < 1e-12
    assert abs((bias - bias0).sum()) < 1e-9
    ema3, bias3 = O.routing_stats(counts * 3, ema0, bias0, decay=0.97, step=-0.05)
    assert np.allclose(ema3, ema, rtol=1e-14, atol=0) and np.allclose(bias3, bias, rtol=1e-14, atol=0)


def test_routing_stats_empty_batch_changes_nothing():
    E = 5
    ema0, bias0 = np.full(E, 0.2), np.linspace(-1, 1, E)
    ema, bias = O.routing_stats(np.zeros(E, dtype=np.int64), ema0, bias0)
    assert np.array_equal(ema, ema0) and np.array_equal(bias, bias0)
