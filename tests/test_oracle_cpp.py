"""Pins of the C++ oracle (oracle/moe_oracle.cpp), CPU only.

The same facts that pin the numpy oracle pin the C++ one: the pages' worked
permutation example, invariants of the permutation and of the capacity fill,
an independent K-pass selection, closed forms of the router weights, exactly
rounded sums, and a dense brute force on tiny inputs written here from the
definition with math.fsum (every expert on every token, masked), which both
oracles must equal bit for bit.  Then the two oracles against each other:
routing and permutation bit for bit, h / out_perm / y within the layer's
tolerance, on the tiny workload and on sampled tokens of the DeepSeek-V3-shape
workload.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import moe_synth as ms
from oracle import cpp as C
from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
IMPLS = {"numpy": O, "cpp": C}


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _tiny_layer(N, D, E, K, F, seed, bias=False, gating="softmax"):
    cfg = ms.MoEConfig("t", N=N, D=D, E=E, K=K, F=F, gating=gating, seed=seed)
    inp = ms.make_inputs(cfg)
    b = ms.zipf_bias(E, 1.2, 0.5, seed).numpy() if bias else None
    return (_bits(inp["x"]), inp["w_router"].numpy(), b, _bits(inp["w_gate"]),
            _bits(inp["w_up"]), _bits(inp["w_down"]))


def _f32(v: float) -> float:
    return float(np.float32(v))


def _bf16(v: float) -> float:
    """Round a float to bf16 (nearest even) by exact rational arithmetic."""
    if v == 0.0 or not math.isfinite(v):
        return v
    m, e = math.frexp(v)                      # v = m 2^e, 0.5 <= |m| < 1
    q = Fraction(m) * 256                     # 8 significant bits before the point
    r = round(q)                              # Python rounds half to even
    return math.ldexp(float(r), e - 8)


# ---------------------------------------------------------------- permutation

@pytest.mark.parametrize("impl", list(IMPLS))
def test_worked_example(impl):
    """zoe.im 范式 A: ids [0,2,0,1,2,0,1,2] give expert_offsets [0,3,5,8]."""
    M = IMPLS[impl]
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    counts, offsets, row_token, slot_row = M.permute(np.array(g["topk_ids"]), g["E"])
    assert offsets.tolist() == g["expert_offsets"]
    d = g["derived_from_the_segments"]
    assert counts.tolist() == d["expert_counts"]
    assert row_token.tolist() == d["row_token"]
    assert slot_row.tolist() == d["slot_row"]


@pytest.mark.parametrize("impl", list(IMPLS))
def test_worked_example_padded(impl):
    M = IMPLS[impl]
    g = json.load(open(os.path.join(GOLDEN, "padded_example.json")))
    ids = np.array([[0], [2], [0], [1], [2], [0], [1], [2]])
    for case in g["cases"]:
        num, den = case["capacity_factor"]
        cap = C.capacity(8, 1, 3, num, den)
        assert cap == case["capacity"]
        counts, offsets, row_token, slot_row = M.permute(ids, 3, cap)
        assert row_token.reshape(3, cap).tolist() == case["buffers"]
        assert sorted(int(i) for i in np.nonzero(slot_row < 0)[0]) == case["dropped_tokens"]


def test_capacity_is_the_exact_ceiling():
    for (N, K, E, num, den) in [(16384, 2, 64, 5, 4), (8, 1, 3, 3, 2), (7, 3, 5, 5, 4),
                                (1, 1, 64, 5, 4), (4096, 8, 256, 1, 1), (0, 2, 8, 5, 4),
                                (10 ** 9, 64, 7, 3, 2)]:
        assert C.capacity(N, K, E, num, den) == math.ceil(Fraction(num * N * K, den * E))


@pytest.mark.parametrize("N,E,K,cap,seed", [(1, 1, 1, None, 0), (37, 5, 2, None, 1),
                                             (100, 16, 4, None, 2), (50, 300, 6, None, 4),
                                             (200, 6, 2, 67, 7), (90, 4, 3, 20, 8)])
def test_permute_invariants_and_fill(N, E, K, cap, seed):
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.full(E, 0.5))
    ids = np.stack([rng.choice(E, size=K, replace=False, p=p) for _ in range(N)])
    counts, offsets, row_token, slot_row = C.permute(ids, E, cap)
    flat = ids.reshape(-1)
    S = N * K
    assert counts.tolist() == np.bincount(flat, minlength=E).tolist()
    for e in range(E):
        slots = [i for i in range(S) if flat[i] == e]
        kept = slots if cap is None else slots[:cap]
        assert [i for i in slots if slot_row[i] >= 0] == kept
        seg = row_token[offsets[e]:offsets[e + 1]].tolist()
        pad = [] if cap is None else [-1] * (cap - len(kept))
        assert seg == [i // K for i in kept] + pad
        assert all(slot_row[i] == offsets[e] + j for j, i in enumerate(kept))
    if cap is None:
        assert sorted(slot_row.tolist()) == list(range(S))            # bijection onto rows


# ---------------------------------------------------------------- top-K / weights

def _kpass_argmax(keys, K):
    """K passes, each taking the strictly largest untaken key (lower id on ties)."""
    N, E = keys.shape
    out = np.empty((N, K), dtype=np.int64)
    for n in range(N):
        taken = set()
        for k in range(K):
            best = None
            for e in range(E):
                if e not in taken and (best is None or keys[n, e] > keys[n, best]):
                    best = e
            taken.add(best)
            out[n, k] = best
    return out


@pytest.mark.parametrize("kind", ["random", "ties", "signed_zero_nan"])
def test_topk_against_kpass_argmax(kind):
    rng = np.random.default_rng(13)
    N, E, K = 60, 12, 5
    lg = rng.standard_normal((N, E)).astype(np.float32)
    if kind == "ties":
        lg = (np.round(lg * 2) / 2).astype(np.float32)
    if kind == "signed_zero_nan":
        lg = np.round(lg).astype(np.float32)
        lg[rng.random((N, E)) < 0.3] = -0.0
        lg[rng.random((N, E)) < 0.1] = np.nan
    ids, _ = C.route_from_logits(lg, None, K, "softmax")
    keys = np.where(np.isnan(lg), -np.inf, lg).astype(np.float64)
    assert np.array_equal(ids, _kpass_argmax(keys, K))


def test_bias_enters_as_one_fp32_add():
    lg = np.array([[1.0, 1.0 + 2 ** -23, 0.5]], dtype=np.float32)
    bias = np.array([2 ** -24, 0.0, 0.5 + 2 ** -24], dtype=np.float32)
    ids, _ = C.route_from_logits(lg, bias, 3, "softmax")
    # fp32: 1 + 2^-24 rounds to 1 (tie to even), so expert 1 leads; 0.5 +
    # (0.5 + 2^-24) = 1 + 2^-24 -> 1, tying expert 0, and the lower id wins
    assert ids.tolist() == [[1, 0, 2]]


def test_weight_closed_forms():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((40, 9)).astype(np.float32)
    # K = 1: weight exactly 1
    _, w = C.route_from_logits(lg, None, 1, "softmax")
    assert np.all(w == 1.0)
    _, w = C.route_from_logits(lg, None, 1, "sigmoid")
    assert np.all(w == 1.0)
    # K = 2 softmax: w0 = 1 / (1 + e^(k1 - k0))
    ids, w = C.route_from_logits(lg, None, 2, "softmax")
    k = np.take_along_axis(lg, ids.astype(np.int64), axis=1).astype(np.float64)
    assert np.allclose(w[:, 0], 1.0 / (1.0 + np.exp(k[:, 1] - k[:, 0])), rtol=0, atol=2e-7)
    # K = E softmax: the full softmax of the row (textbook)
    ids, w = C.route_from_logits(lg, None, 9, "softmax")
    full = np.exp(lg.astype(np.float64) - lg.max(1, keepdims=True))
    full /= full.sum(1, keepdims=True)
    assert np.allclose(w, np.take_along_axis(full, ids.astype(np.int64), 1), rtol=0, atol=2e-7)
    # sigmoid renormalised: w_j = s_j / sum s, sums to 1
    ids, w = C.route_from_logits(lg, None, 4, "sigmoid")
    s = 1.0 / (1.0 + np.exp(-np.take_along_axis(lg, ids.astype(np.int64), 1).astype(np.float64)))
    assert np.allclose(w, s / s.sum(1, keepdims=True), rtol=0, atol=2e-7)
    assert np.allclose(w.astype(np.float64).sum(1), 1.0, atol=1e-6)
    # every selected key -inf (NaN logits): the zero denominator gives 1/K
    ids, w = C.route_from_logits(np.full((1, 4), np.nan, np.float32), None, 2, "softmax")
    assert ids.tolist() == [[0, 1]] and w.tolist() == [[0.5, 0.5]]


def test_router_logits_are_exactly_rounded():
    x, wr, *_ = _tiny_layer(7, 96, 5, 1, 8, seed=21)
    lg = C.router_logits(x, wr)
    xv = O.bf16_to_f64(x)
    for n in range(7):
        for e in range(5):
            exact = math.fsum(float(a) * float(b) for a, b in zip(xv[n], wr[e].astype(np.float64)))
            assert lg[n, e] == np.float32(exact)


# ---------------------------------------------------------------- dense brute force

def _dense_fsum(x, wr, bias, wg, wu, wd, K, gating, cap=None):
    """Every expert on every token with exactly rounded sums, masked by the
    routing, rounded where the layer holds or stores values; the routing is
    the K-pass argmax of the keys and the weights the closed forms."""
    xv, wgv, wuv, wdv = (O.bf16_to_f64(a) for a in (x, wg, wu, wd))
    N, D = xv.shape
    E, F, _ = wgv.shape
    lg = np.array([[_f32(math.fsum(xv[n] * wr[e].astype(np.float64))) for e in range(E)]
                   for n in range(N)], dtype=np.float32)
    key = lg if bias is None else (lg + bias.astype(np.float32)).astype(np.float32)
    ids = _kpass_argmax(key.astype(np.float64), K)
    kept = np.ones((N, K), bool)
    if cap is not None:
        seen = np.zeros(E, int)
        for n in range(N):
            for k in range(K):
                kept[n, k] = seen[ids[n, k]] < cap
                seen[ids[n, k]] += 1
    y = np.zeros((N, D))
    for n in range(N):
        ks = [float(key[n, ids[n, k]]) for k in range(K)]
        if gating == "softmax":
            z = [math.exp(v - ks[0]) for v in ks]
        else:
            z = [1.0 / (1.0 + math.exp(-v)) for v in ks]
        w = [_f32(v / math.fsum(z)) for v in z]
        terms = [[] for _ in range(D)]
        for k in range(K):
            if not kept[n, k]:
                continue
            e = ids[n, k]
            h = []
            for j in range(F):
                g = _f32(math.fsum(xv[n] * wgv[e, j]))
                u = _f32(math.fsum(xv[n] * wuv[e, j]))
                h.append(_bf16(_f32(g / (1.0 + math.exp(-g)) * u)))
            h = np.array(h)
            for c in range(D):
                o = _bf16(_f32(math.fsum(h * wdv[e, c])))
                terms[c].append(w[k] * o)
        for c in range(D):
            y[n, c] = _bf16(_f32(math.fsum(terms[c])))
    return ids, y


@pytest.mark.parametrize("impl", list(IMPLS))
@pytest.mark.parametrize("gating,bias,K,cap", [("softmax", False, 2, None),
                                               ("sigmoid", False, 3, None),
                                               ("softmax", True, 2, (5, 4)),
                                               ("sigmoid", True, 4, (1, 1)),
                                               ("softmax", False, 1, None)])
def test_sparse_equals_dense_bruteforce_exactly(impl, gating, bias, K, cap):
    M = IMPLS[impl]
    N, D, E, F = 12, 24, 5, 20
    x, wr, b, wg, wu, wd = _tiny_layer(N, D, E, K, F, seed=33, bias=bias, gating=gating)
    c = C.capacity(N, K, E, *cap) if cap else None
    res = M.forward(x, wr, b, wg, wu, wd, K, gating, cap=c)
    ids, y = _dense_fsum(x, wr, b, wg, wu, wd, K, gating, cap=c)
    assert np.array_equal(res["topk_ids"], ids)
    assert np.array_equal(res["y"], y), f"{int((res['y'] != y).sum())} elements differ"


# ---------------------------------------------------------------- invariants

def test_wd_scaling_and_k1_gather():
    x, wr, b, wg, wu, wd = _tiny_layer(16, 32, 4, 1, 40, seed=71)
    r = C.forward(x, wr, b, wg, wu, wd, 1, "softmax")
    assert np.array_equal(r["y"], r["out_perm"][r["slot_row"]])          # K = 1, w = 1
    wd2 = O.f64_to_bf16_bits(2.0 * O.bf16_to_f64(wd))
    r2 = C.forward(x, wr, b, wg, wu, wd2, 1, "softmax")
    assert np.array_equal(r2["y"], 2.0 * r["y"])


def test_large_capacity_equals_contiguous_and_padding_is_zero():
    N, K, E = 30, 2, 5
    x, wr, b, wg, wu, wd = _tiny_layer(N, 32, E, K, 24, seed=91, bias=True)
    rc = C.forward(x, wr, b, wg, wu, wd, K, "softmax")
    rp = C.forward(x, wr, b, wg, wu, wd, K, "softmax", cap=N)
    assert np.array_equal(rc["y"], rp["y"])
    pad = rp["row_token"] < 0
    assert pad.any() and np.all(rp["out_perm"][pad] == 0) and np.all(rp["h"][pad] == 0)


def test_results_do_not_depend_on_threads():
    """Each output is summed by one thread in index order."""
    import subprocess
    import sys
    code = ("import numpy as np, sys; sys.path.insert(0, %r); from oracle import cpp as C; "
            "from tests.test_oracle_cpp import _tiny_layer; "
            "x,wr,b,wg,wu,wd=_tiny_layer(40,64,6,2,48,seed=3,bias=True); "
            "r=C.forward(x,wr,b,wg,wu,wd,2,'sigmoid'); "
            "sys.stdout.write(str(int(np.frombuffer(np.ascontiguousarray(r['y']).tobytes(),"
            "np.uint64).sum() %% (1<<61))))") % os.path.dirname(os.path.dirname(
                os.path.abspath(__file__)))
    outs = set()
    for t in ("1", "3"):
        env = dict(os.environ, OMP_NUM_THREADS=t)
        outs.add(subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                                text=True, check=True).stdout)
    assert len(outs) == 1


# ---------------------------------------------------------------- the two oracles agree

def _assert_close(got, ref, what):
    M = float(np.abs(ref).max())
    d = np.abs(got - ref)
    assert d.max() <= 1e-2 * M and np.all(d <= 1e-2 * M + 2e-2 * np.abs(ref)), what


@pytest.mark.parametrize("name,padded", [("tiny", False), ("tiny", True), ("gelu_tiny", False)])
def test_cpp_equals_numpy_on_the_tiny_workload(name, padded):
    cfg = ms.CONFIGS[name]
    inp = ms.make_inputs(cfg.scaled(expert="swiglu"))
    x, wr = _bits(inp["x"]), inp["w_router"].numpy()
    wg, wu, wd = _bits(inp["w_gate"]), _bits(inp["w_up"]), _bits(inp["w_down"])
    cap = C.capacity(cfg.N, cfg.K, cfg.E, 1, 2) if padded else None
    a = O.forward(x, wr, None, wg, wu, wd, cfg.K, cfg.gating, cap=cap)
    b = C.forward(x, wr, None, wg, wu, wd, cfg.K, cfg.gating, cap=cap)
    for k in ("logits", "topk_ids", "expert_counts", "expert_offsets", "row_token", "slot_row"):
        assert np.array_equal(a[k], b[k]), k
    assert np.abs(a["topk_weights"].astype(np.float64) - b["topk_weights"]).max() <= 1e-6
    for k in ("h", "out_perm", "y"):
        _assert_close(b[k], a[k], k)
        assert np.mean(a[k] == b[k]) > 0.999, k


def test_cpp_equals_numpy_on_sampled_deepseek_v3_tokens():
    """Two tokens of the DeepSeek-V3-shape workload (D = 7168, E = 256, K = 8,
    F = 2048, sigmoid), with the weights of the experts they reach."""
    cfg = ms.CONFIGS["deepseek_v3"]
    tokens = [0, 5000]
    x = np.concatenate([_bits(ms.normal_bf16(cfg.D, 1.0, cfg.seed, ms.STREAM_X, offset=t * cfg.D))
                        [None] for t in tokens])
    wr = ms.normal_f32(cfg.E * cfg.D, 1.0 / math.sqrt(cfg.D), cfg.seed,
                       ms.STREAM_WR).view(cfg.E, cfg.D).numpy()
    la, ia, wa = O.route(x, wr, None, cfg.K, cfg.gating)
    lb, ib, wb = C.route(x, wr, None, cfg.K, cfg.gating)
    assert np.array_equal(la, lb) and np.array_equal(ia, ib)
    assert np.abs(wa.astype(np.float64) - wb).max() <= 1e-6
    assert np.array_equal(O.permute(ia, cfg.E)[2], C.permute(ib, cfg.E)[2])
    experts = sorted(set(ia.reshape(-1).tolist()))
    slot = {e: i for i, e in enumerate(experts)}
    W = {w: np.stack([_bits(ms.expert_weight(cfg, w, e)) for e in experts])
         for w in ("gate", "up", "down")}
    re = np.array([slot[e] for e in ia.reshape(-1)], dtype=np.int32)
    rt = np.repeat(np.arange(len(tokens)), cfg.K).astype(np.int32)
    _, out_c = C.ffn_rows(re, rt, x, W["gate"], W["up"], W["down"], want_h=False)
    y_c = (wb.astype(np.float64)[:, :, None] * out_c.reshape(len(tokens), cfg.K, cfg.D)).sum(1)
    y_c = O.round_bf16(O.round_f32(y_c).astype(np.float64))
    y_n, out_n = O.token_outputs(x, ia, wa, np.ones_like(ia, dtype=bool),
                                 lambda e: (W["gate"][slot[e]], W["up"][slot[e]],
                                            W["down"][slot[e]]))
    _assert_close(out_c.reshape(out_n.shape), out_n, "out")
    _assert_close(y_c, y_n, "y")
    assert np.mean(out_c.reshape(out_n.shape) == out_n) > 0.999


# ---------------------------------------------------------------- FP8 weights

@pytest.mark.parametrize("kind", ["normal", "all_bits", "specials"])
def test_cpp_fp8_quantizer_equals_numpy(kind):
    """Codes and scale bytes bit for bit those of the numpy quantiser (itself
    pinned to torch's E4M3 conversions): normal weights, uniformly random bf16
    bit patterns (subnormals, huge values, infinities, NaNs) and hand-built
    blocks (all zero, one subnormal, saturating, ties)."""
    rng = np.random.default_rng({"normal": 1, "all_bits": 2, "specials": 3}[kind])
    if kind == "normal":
        w = O.f64_to_bf16_bits(rng.standard_normal((96, 256)) * 0.02)
    elif kind == "all_bits":
        w = rng.integers(0, 65536, (128, 512), dtype=np.uint16)
    else:
        v = np.zeros((4, 32))
        v[1, 3] = 2.0 ** -133                          # a bf16 subnormal alone in its block
        v[2] = np.linspace(-3.0e38, 3.0e38, 32)         # near the top of bf16
        v[3] = (np.arange(32) - 16) * 2.0 ** -4 * 17    # many exact ties after scaling
        w = O.f64_to_bf16_bits(v)
    a, b = O.quantize_fp8(w), C.quantize_fp8(w)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    da, db = O.dequantize_fp8_bits(*a), C.dequantize_fp8_bits(*b)
    nan = np.isnan(O.bf16_to_f64(da))
    assert np.array_equal(da[~nan], db[~nan]) and np.all(np.isnan(O.bf16_to_f64(db)[nan]))


def test_cpp_e4m3_decoder_against_torch():
    """Every E4M3 code dequantised with scale 2^0 equals torch's float8_e4m3fn value."""
    codes = np.arange(256, dtype=np.uint8).reshape(8, 32)
    scales = np.full((8, 1), 127, dtype=np.uint8)
    got = O.bf16_to_f64(C.dequantize_fp8_bits(codes, scales))
    ref = torch.from_numpy(codes.reshape(-1)).view(torch.float8_e4m3fn).to(torch.float64)
    ref = ref.numpy().reshape(8, 32)
    both_nan = np.isnan(got) & np.isnan(ref)
    assert np.array_equal(got[~both_nan], ref[~both_nan]) and both_nan.sum() == 2
