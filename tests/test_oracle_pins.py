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
    return O.round_bf16(O.round_f32(y).astype(np.float64))


@pytest.mark.parametrize("gating,bias,K,cap", [("softmax", False, 2, None), ("sigmoid", False, 3, None),
                                               ("softmax", True, 2, None), ("softmax", True, 2, (5, 4)),
                                               ("softmax", False, 1, None), ("sigmoid", True, 4, (1, 1))])
def test_sparse_equals_dense_bruteforce(gating, bias, K, cap):
    N, D, E, F = 24, 32, 6, 48
    cfg, x, wr, b, wg, wu, wd = _tiny_layer(N, D, E, K, F, seed=31, bias=bias, gating=gating)
    c = O.capacity(N, K, E, *cap) if cap else None
    res = O.forward(x, wr, b, wg, wu, wd, K, gating, cap=c)
    ref = _dense_bruteforce(x, wr, b, wg, wu, wd, K, gating, cap=c)
    # bit for bit (an exactly rounded brute force written from the definition,
    # independent of swiglu_rows, is tests/test_oracle_cpp.py's)
    assert np.array_equal(res["y"], ref)
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


# ------------------------------------------------------ block-scaled FP8 weights
# Independent references: torch's float8_e4m3fn conversions (a separate
# implementation of the OCP E4M3 format), closed forms of the format, and exact
# round trips of values built from known codes and exponents.

def _all_codes():
    return np.arange(256, dtype=np.uint8)


def test_e4m3_decode_matches_torch():
    c = _all_codes()
    mine = O.e4m3_decode(c)
    ref = torch.from_numpy(c).view(torch.float8_e4m3fn).float().double().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.isnan(mine).sum() == 2 and np.isnan(mine[[0x7F, 0xFF]]).all()
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])


@pytest.mark.parametrize("seed", [0, 1])
def test_e4m3_encode_matches_torch(seed):
    """Random fp32 values across every binade of the format, plus every
    midpoint between neighbouring codes (ties go to the even code)."""
    rng = np.random.default_rng(seed)
    v = (rng.standard_normal(100000) * np.exp2(rng.integers(-16, 9, 100000))).astype(np.float32)
    v = v[np.abs(v) <= O.E4M3_MAX]
    d = O.e4m3_decode(_all_codes())[:127]
    mids = ((d[:-1] + d[1:]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids, [0.0, -0.0]]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(v.astype(np.float64)), ref)


def test_e4m3_encode_closed_forms():
    cases = {448.0: 0x7E, -448.0: 0xFE, 1.0: 0x38, 2.0 ** -9: 0x01, 2.0 ** -6: 0x08,
             2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02, 1.0625: 0x38, 1.1875: 0x3A,
             15.5: 0x58,          # tie between 15 (0x57) and 16: even mantissa
             464.0: 0x7E, 500.0: 0x7E, 1e30: 0x7E, -1e30: 0xFE,
             math.inf: 0x7F, -math.inf: 0xFF, math.nan: 0x7F, -0.0: 0x80,
             -(2.0 ** -11): 0x80}
    got = O.e4m3_encode(np.array(list(cases.keys())))
    assert got.tolist() == list(cases.values())


def test_mx_block_scale_closed_forms():
    """Shared exponent floor(log2 amax) - 8: the block maximum lands in
    [256, 512) and saturates to 448 above it; zero and tiny blocks take the
    lower clamp -117 (byte 10), the largest bf16 block the upper 119 (byte 246)."""
    def q(vals):
        w = np.zeros((1, 32))
        w[0, :len(vals)] = vals
        return O.quantize_fp8(O.f64_to_bf16_bits(w))
    c, s = q([1.0, 0.5, -0.25])
    assert s.tolist() == [[119]] and c[0, :3].tolist() == [0x78, 0x70, 0xE8]
    c, s = q([1.9921875])                           # 1.99 * 2^8 = 510 -> 448
    assert s.tolist() == [[119]] and c[0, 0] == 0x7E
    c, s = q([-3.0, 2.0 ** -20])                    # -3 * 2^7 = -1.5 * 2^8; 2^-13 -> 0
    assert s.tolist() == [[120]] and c[0, :2].tolist() == [0xFC, 0x00]
    c, s = q([])
    assert s.tolist() == [[10]] and not c.any()
    c, s = q([2.0 ** -130])                         # a bf16 subnormal
    assert s.tolist() == [[10]] and c[0, 0] == 0
    bmax = O.bf16_to_f64(np.array([0x7F7F], dtype=np.uint16))[0]
    c, s = q([bmax, -bmax])
    assert s.tolist() == [[246]] and c[0, :2].tolist() == [0x7E, 0xFE]
    c, s = q([2.0, math.inf, math.nan])             # non-finite: NaN code, scale from the finite ones
    assert s.tolist() == [[120]] and c[0, :3].tolist() == [0x78, 0x7F, 0x7F]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fp8_round_trip_exact(seed):
    """Weights built as code * 2^s, with one code of each block in the top
    binade [256, 448], quantise back to exactly those codes and exponents,
    on a 3-D [E, F, D] tensor (rows and blocks must not mix)."""
    rng = np.random.default_rng(seed)
    E, F, D = 3, 5, 128
    nb = D // 32
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    codes = rng.choice(finite, size=(E, F, D)).astype(np.uint8)
    top = rng.integers(0x78, 0x7F, size=(E, F, nb)) | (rng.integers(0, 2, (E, F, nb)) << 7)
    pos = rng.integers(0, 32, size=(E, F, nb))
    for idx in np.ndindex(E, F, nb):
        codes[idx[0], idx[1], idx[2] * 32 + pos[idx]] = top[idx]
    s = rng.integers(O.MX_SCALE_MIN, O.MX_SCALE_MAX + 1, size=(E, F, nb))
    w = np.ldexp(O.e4m3_decode(codes).reshape(E, F, nb, 32), s[..., None]).reshape(E, F, D)
    w_bits = O.f64_to_bf16_bits(w)
    assert np.array_equal(O.bf16_to_f64(w_bits), w)          # the weights are bf16 values
    qc, qs = O.quantize_fp8(w_bits)
    assert qs.shape == (E, F, nb) and qs.dtype == np.uint8
    assert np.array_equal(qc, codes) and np.array_equal(qs.astype(np.int64), s + 127)
    assert np.array_equal(O.dequantize_fp8_bits(qc, qs), w_bits)


@pytest.mark.parametrize("seed", [0, 1])
def test_fp8_error_bound_and_exactness(seed):
    """Each dequantised value is within half a grid step of the weight
    (2^(floor(log2|w/2^s|) - 4) in the normal range, 2^-10 below, times 2^s),
    saturated values excepted; dequantised values are bf16 numbers; the
    rounding is monotone within a block."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((16, 256)) * 0.02
    w[rng.random(w.shape) < 0.01] *= 40                    # outliers
    w_bits = O.f64_to_bf16_bits(w)
    w = O.bf16_to_f64(w_bits)
    c, s = O.quantize_fp8(w_bits)
    deq = O.dequantize_fp8(c, s)
    assert np.array_equal(O.round_bf16(deq), deq)
    sc = np.repeat(np.ldexp(1.0, s.astype(np.int64) - 127), 32, axis=-1)
    t = np.abs(w) / sc
    _, ex = np.frexp(t)
    half = np.where(t >= O.E4M3_MIN_NORMAL, np.ldexp(1.0, ex - 1 - 4), 2.0 ** -10)
    sat = t > O.E4M3_MAX
    assert np.all(np.abs(deq - w)[~sat] <= (half * sc)[~sat])
    assert np.all(np.abs(deq[sat]) == O.E4M3_MAX * sc[sat])
    order = np.argsort(w[0, :32], kind="stable")
    assert np.all(np.diff(deq[0, :32][order]) >= 0)


def test_expert_ffn_fp8_on_representable_weights():
    """With weights that FP8 represents exactly, the FP8 FFN equals the bf16
    FFN bit for bit (gate and up not swapped, down not transposed)."""
    rng = np.random.default_rng(7)
    E, F, D, R = 3, 64, 96, 10

    def rep(shape):
        codes = rng.integers(0x20, 0x50, size=shape).astype(np.uint8) | \
            (rng.integers(0, 2, shape) << 7).astype(np.uint8)
        codes[..., ::32] = 0x78                          # pin each block's exponent
        s = np.full(shape[:-1] + (shape[-1] // 32,), 127 - 12, dtype=np.uint8)
        return codes, s

    wg, wu, wd = rep((E, F, D)), rep((E, F, D)), rep((E, D, F))
    x = O.f64_to_bf16_bits(rng.standard_normal((R, D)))
    offs = np.array([0, 4, 4, R])
    want = O.expert_ffn(x, offs, O.dequantize_fp8_bits(*wg), O.dequantize_fp8_bits(*wu),
                        O.dequantize_fp8_bits(*wd))
    for q in (wg, wu, wd):
        assert np.array_equal(O.quantize_fp8(O.dequantize_fp8_bits(*q))[0], q[0])
    got = O.expert_ffn_fp8(x, offs, wg, wu, wd)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    assert np.abs(got[1]).max() > 0


# ------------------------------------------ GELU experts and the MLP router
# Independent references: torch's own GELU and nn.Linear / nn.Sequential in
# float64 (the module structure of the page's MoELayer), closed forms of
# Phi, and a dense brute force of the whole layer.

def _gelu_layer(N, D, E, K, F, seed):
    cfg = ms.MoEConfig("g", N=N, D=D, E=E, K=K, F=F, gating="softmax", seed=seed, expert="gelu")
    i = ms.make_gelu_inputs(cfg)
    return cfg, {k: (_bits(v) if v.dtype == torch.bfloat16 else v.numpy()) for k, v in i.items()}


def test_gelu_against_torch_and_closed_forms():
    v = np.concatenate([np.linspace(-12, 12, 2001), [0.0, 1.0, -1.0, 1e-8, -40.0, 40.0]])
    ref = torch.nn.functional.gelu(torch.from_numpy(v)).numpy()       # exact erf form
    assert np.allclose(O.gelu(v), ref, rtol=1e-14, atol=1e-15)   # torch cancels to 0 for v < -8.3
    assert O.gelu(0.0) == 0.0
    assert abs(O.gelu(1.0) - 0.8413447460685429) < 1e-15             # Phi(1)
    assert np.allclose(O.gelu(v) - O.gelu(-v), v, rtol=0, atol=1e-13)  # Phi(v) + Phi(-v) = 1
    assert O.gelu(40.0) == 40.0 and O.gelu(-40.0) == 0.0


def _torch_linear(w, b):
    lin = torch.nn.Linear(w.shape[1], w.shape[0]).double()
    with torch.no_grad():
        lin.weight.copy_(torch.from_numpy(w))
        lin.bias.copy_(torch.from_numpy(np.asarray(b, dtype=np.float64)))
    return lin


def test_mlp_router_matches_torch_modules():
    """gate_proj -> GELU -> (bf16 storage) -> gate_out, built as torch modules
    in float64 from the same weights: features, logits + bias, top-K ids and
    softmax weights agree."""
    cfg, t = _gelu_layer(N=40, D=128, E=8, K=2, F=256, seed=71)
    proj = _torch_linear(O.bf16_to_f64(t["w_proj"]), t["b_proj"])
    out = _torch_linear(t["w_out"].astype(np.float64), t["b_out"])
    x = torch.from_numpy(O.bf16_to_f64(t["x"]))
    with torch.no_grad():
        a_t = torch.nn.GELU()(proj(x)).to(torch.bfloat16).to(torch.float64)
        g_t = out(a_t)                                         # biased gate logits
    a = O.mlp_router_features(t["x"], t["w_proj"], t["b_proj"])
    assert np.mean(a == a_t.numpy()) > 0.999 and np.abs(a - a_t.numpy()).max() <= 2 ** -6
    logits = O.mlp_router_logits(a_t.numpy(), t["w_out"])
    np.testing.assert_allclose(logits + t["b_out"].astype(np.float64), g_t.numpy(),
                               rtol=1e-6, atol=1e-6)
    ids, w = O.route_from_logits(logits, t["b_out"], 2, "softmax")
    tv, ti = torch.topk(g_t, 2, dim=-1)
    assert np.array_equal(ids, ti.numpy())
    np.testing.assert_allclose(w, torch.softmax(tv, dim=-1).numpy(), rtol=0, atol=1e-6)


def test_gelu_expert_matches_torch_sequential():
    """One expert as nn.Sequential(Linear(D, F), GELU(), Linear(F, D)) in
    float64 with the bf16 rounding of the hidden activations: outputs agree
    to the bf16 rounding (gate/up order, transposes and biases pinned)."""
    cfg, t = _gelu_layer(N=16, D=64, E=3, K=1, F=256, seed=72)
    e = 1
    l1 = _torch_linear(O.bf16_to_f64(t["w1"][e]), t["b1"][e])
    l2 = _torch_linear(O.bf16_to_f64(t["w2"][e]), t["b2"][e])
    x = O.bf16_to_f64(t["x"][:16])
    with torch.no_grad():
        h_t = torch.nn.GELU()(l1(torch.from_numpy(x))).to(torch.bfloat16).to(torch.float64)
        o_t = l2(h_t).to(torch.bfloat16).to(torch.float64).numpy()
    h, o = O.gelu_ffn_rows(x, t["w1"][e], t["b1"][e], t["w2"][e], t["b2"][e])
    assert np.mean(h == h_t.numpy()) > 0.999
    o2 = O.gelu_ffn_rows(x, t["w1"][e], t["b1"][e], t["w2"][e], t["b2"][e])[1]
    assert np.array_equal(o, o2)
    assert np.mean(o == o_t) > 0.99 and np.abs(o - o_t).max() <= 2 ** -6 * np.abs(o_t).max()


@pytest.mark.parametrize("K,cap", [(2, None), (1, None), (2, (5, 4)), (3, (1, 2))])
def test_gelu_layer_sparse_equals_dense(K, cap):
    """Every GELU expert on every token, masked by the routing (no
    permutation), equals the sparse layer; padding rows of a padded buffer
    hold the experts' response to a zero row and never reach y."""
    N, D, E, F = 24, 64, 6, 96
    cfg, t = _gelu_layer(N, D, E, K, F, seed=73)
    c = O.capacity(N, K, E, *cap) if cap else None
    res = O.forward_gelu(t["x"], t["w_proj"], t["b_proj"], t["w_out"], t["b_out"], t["w1"],
                         t["b1"], t["w2"], t["b2"], K, cap=c)
    ids, w = res["topk_ids"], res["topk_weights"]
    xs = O.bf16_to_f64(t["x"])
    outs = np.stack([O.gelu_ffn_rows(xs, t["w1"][e], t["b1"][e], t["w2"][e], t["b2"][e])[1]
                     for e in range(E)])
    keep = res["slot_row"].reshape(N, K) >= 0
    y = np.zeros((N, D))
    for k in range(K):
        y += np.where(keep[:, k:k + 1], w[:, k:k + 1].astype(np.float64) * outs[ids[:, k], np.arange(N)], 0.0)
    ref = O.round_bf16(O.round_f32(y).astype(np.float64))
    assert np.array_equal(res["y"], ref)
    if c is not None:
        pad = res["row_token"] < 0
        zero_row = np.stack([O.gelu_ffn_rows(np.zeros((1, D)), t["w1"][e], t["b1"][e], t["w2"][e],
                                             t["b2"][e])[1][0] for e in range(E)])
        seg = np.repeat(np.arange(E), c)
        assert np.array_equal(res["out_perm"][pad], zero_row[seg[pad]])


def test_token_outputs_gelu_matches_forward_gelu():
    N, D, E, K, F = 20, 64, 5, 2, 128
    cfg, t = _gelu_layer(N, D, E, K, F, seed=74)
    res = O.forward_gelu(t["x"], t["w_proj"], t["b_proj"], t["w_out"], t["b_out"], t["w1"],
                         t["b1"], t["w2"], t["b2"], K)
    tok = np.array([0, 3, 7, 19])
    y, _ = O.token_outputs(t["x"][tok], res["topk_ids"][tok], res["topk_weights"][tok],
                           np.ones((len(tok), K), dtype=bool),
                           lambda e: (t["w1"][e], t["b1"][e], t["w2"][e], t["b2"][e]),
                           rows_fn=O.gelu_ffn_rows)
    assert np.array_equal(y, res["y"][tok])
