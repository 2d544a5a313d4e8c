"""CPU oracle of the single-GPU MoE-layer forward pass.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check in
``__graft_entry__`` and the benchmark's CPU-baseline leg may import or run
this module.  The product library never imports, links or calls it, and it
shares no code with the HIP path (only the seeded input generator in
``moe_synth`` feeds both sides).

What it computes, step by step, in the order and notation of the pages:

* Router: a bias-free linear layer ``logits = W_gate x`` of shape (N, E)
  ["MoE 推理完整机制" (zoe.im), 第一层: Router 与 Top-K 的算法细节; the
  ``gate = nn.Linear(hidden_dim, num_experts, bias=False)`` of
  "MoE 大规模分布式推理工程实战" (ybb.press), 4.1 Router 辅助损失的工程化实现].
* Optional per-expert bias added to the logits before top-K
  [ybb.press 4.1, ``logits + self.dynamic_bias``].
* Top-K per token, then either softmax over the K selected values (weights
  sum to 1) [zoe.im 第一层] or the sigmoid variant where the selected
  sigmoid scores are divided by their sum [zoe.im 第一层, "DeepSeek 的
  sigmoid + norm 变体"].
* Contiguous permutation: tokens regrouped into one buffer with one segment
  per expert, plus ``expert_offsets`` [zoe.im 第二层, 范式 A Step 1]; counts
  by histogram and offsets by exclusive prefix sum [ybb.press 2.2,
  ``moe_alltoall_start`` steps 1-2].
* Capacity-padded variant: a fixed capacity per expert, filled in token
  order, overflow dropped [zoe.im 第二层, 范式 B; capacity formula of
  "MoE工程实战" (jsqmd.com) 3.2].
* Per-expert FFN, two GEMMs (m_e, D) -> (m_e, F) -> (m_e, D), empty experts
  skipped [zoe.im 范式 A Step 2; jsqmd.com 4.2 ``numel() > 0``].  The FFN
  is SwiGLU: ``h = silu(x Wg^T) * (x Wu^T)``, ``out = h Wd^T``.
* Un-permutation: results put back in token order, multiplied by the router
  weights and summed [zoe.im 范式 A Step 3 and the opening dataflow].
* Routing statistics (outside the forward pass): the batch's per-expert
  fraction of slots folded into an EMA, and the per-expert bias moved by
  (E * normalised EMA - 1) * step [ybb.press 4.1, ``_update_load_balance_stats``
  and the bias update in ``load_balance_loss``].
* The second layer of the pages: experts ``Linear(D, 4D) - GELU -
  Linear(4D, D)`` with biases, and a router that first compresses the hidden
  state with a 2-layer MLP (D -> D/4, GELU) before the gate Linear
  ["MoE工程实战" (jsqmd.com), 3.1 输入表征 and the ``MoELayer`` of 4.2].
* Block-scaled FP8 expert weights: E4M3 codes with one power-of-two scale
  per 32 values along a weight row's input dimension, and the FFN run on
  their dequantised values [zoe.im 第四层 DeepGEMM & MegaMoE Kernel (FP8
  weights); jsqmd.com 5.3 技巧2 (8-bit expert weights, dequantised for use)].

Precision: every sum is taken in float64.  Values are rounded where the GPU
holds or stores them: the logits, the gate and up pre-activations g and u,
the product silu(g) * u, the down dot and the combine sum to fp32 (the GPU's
arithmetic type), and then the bf16 tensors ``h`` (FFN intermediate),
``out_perm`` (FFN output rows) and ``y`` (layer output) to bf16, each with
round-to-nearest-even; the router weights are computed in float64 and rounded
to fp32.  Top-K is decided on fp32 keys.

Readings where the pages are silent:
ties in top-K go to the lower expert id, -0.0 equals +0.0 and NaN keys sort
last; the K outputs are in descending key order; selection in sigmoid mode is
done on the key itself (sigmoid is strictly increasing); the bias is one fp32
add and also feeds the weights; a sigmoid sum of zero gives weights 1/K;
within a segment rows are in ascending slot order n*K+k; capacity is
``ceil(num*N*K/(den*E))`` and the first ``cap`` slots (slot order) of each
expert are kept, dropped slots contribute nothing and the kept weights are not
renormalised; padding rows are zero.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erfc

GATING_SOFTMAX = "softmax"
GATING_SIGMOID = "sigmoid"


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """Decode raw bf16 bit patterns (uint16) to float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_bf16(v) -> np.ndarray:
    """Round float64 values to bf16 (8 significant bits), nearest-even.

    frexp gives v = m * 2**ex with 0.5 <= |m| < 1, so m * 2**8 has 8 integer
    bits; np.rint rounds half to even.  Normal range only (the layer's values
    stay far from bf16 overflow and underflow).
    """
    v = np.asarray(v, dtype=np.float64)
    m, ex = np.frexp(v)
    return np.ldexp(np.rint(np.ldexp(m, 8)), ex - 8)


def f64_to_bf16_bits(v) -> np.ndarray:
    r = round_bf16(v).astype(np.float32)          # exact: 8 significant bits
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def round_f32(v) -> np.ndarray:
    return np.asarray(v, dtype=np.float64).astype(np.float32)


def _f32(v) -> np.ndarray:
    """fp32 rounding of float64 values, kept as float64 (IEEE nearest even)."""
    return round_f32(v).astype(np.float64)


# --------------------------------------------------------------------------
# router and gating
# --------------------------------------------------------------------------

def router_logits(x_bits, w_router) -> np.ndarray:
    """logits[n, e] = sum_d x[n, d] * W_gate[e, d], float64 sum, rounded to fp32.

    zoe.im 第一层 (``logits = W_gate @ x``); W_gate in nn.Linear [E, D] layout
    (ybb.press 4.1).  Each product bf16*fp32 is exact in float64.
    """
    x = bf16_to_f64(x_bits)
    w = np.asarray(w_router, dtype=np.float32).astype(np.float64)
    return round_f32(x @ w.T)


def gating_keys(logits, bias=None) -> np.ndarray:
    """Selection keys: logits plus the per-expert bias (one fp32 add), as fp32.

    ybb.press 4.1 adds the dynamic bias to the logits before ``torch.topk``.
    -0.0 becomes +0.0 and NaN becomes -inf, so equal values compare equal and
    a NaN is never selected ahead of a number.
    """
    key = np.asarray(logits, dtype=np.float32)
    if bias is not None:
        key = key + np.asarray(bias, dtype=np.float32)[None, :]   # float32 + float32
    key = key.astype(np.float32, copy=True)
    key[key == 0] = np.float32(0.0)
    key[np.isnan(key)] = np.float32(-np.inf)
    return key


def select_topk(keys, K: int) -> np.ndarray:
    """Ids of the K largest keys per row, largest first, equal keys by lower id.

    zoe.im 第一层 (``torch.topk(logits, k=K)``, sorted output).
    """
    keys = np.asarray(keys, dtype=np.float32)
    N, E = keys.shape
    ids = np.arange(E)
    out = np.empty((N, K), dtype=np.int32)
    for n in range(N):
        order = np.lexsort((ids, -keys[n].astype(np.float64)))   # key desc, then id asc
        out[n] = order[:K]
    return out


def topk_weights(sel_keys, gating: str) -> np.ndarray:
    """Router weights of the K selected experts (float64 math, fp32 result).

    softmax: w_j = exp(k_j - max) / sum_i exp(k_i - max)     (zoe.im 第一层)
    sigmoid: s_j = 1/(1+exp(-k_j)), w_j = s_j / sum_i s_i     (zoe.im sigmoid + norm)
    A row whose selected keys give a zero denominator gets w = 1/K.
    """
    k = np.asarray(sel_keys, dtype=np.float32).astype(np.float64)
    K = k.shape[1]
    if gating == GATING_SOFTMAX:
        kmax = k.max(axis=1, keepdims=True)
        finite = np.isfinite(kmax[:, 0])
        z = np.zeros_like(k)
        z[finite] = np.exp(k[finite] - kmax[finite])
    elif gating == GATING_SIGMOID:
        z = 1.0 / (1.0 + np.exp(-k))
    else:
        raise ValueError(gating)
    tot = z.sum(axis=1, keepdims=True)
    w = np.where(tot > 0, z / np.where(tot > 0, tot, 1.0), 1.0 / K)
    return round_f32(w)


def route_from_logits(logits, bias, K: int, gating: str):
    """(topk_ids [N,K] int32, topk_weights [N,K] fp32) from fp32 logits."""
    keys = gating_keys(logits, bias)
    ids = select_topk(keys, K)
    sel = np.take_along_axis(keys, ids.astype(np.int64), axis=1)
    return ids, topk_weights(sel, gating)


def route(x_bits, w_router, bias, K: int, gating: str):
    logits = router_logits(x_bits, w_router)
    ids, w = route_from_logits(logits, bias, K, gating)
    return logits, ids, w


# --------------------------------------------------------------------------
# permutation
# --------------------------------------------------------------------------

def capacity(N: int, K: int, E: int, num: int, den: int) -> int:
    """Per-expert capacity ceil((num/den) * N*K / E) in exact integer arithmetic.

    zoe.im 范式 B (``ceil(1.5 * N * K / num_experts)``) with the factor as a
    parameter; jsqmd.com 3.2 gives the same product tokens*k/E*factor.
    """
    return -((-num * N * K) // (den * E))


def permute(topk_ids, E: int, cap: int | None = None):
    """Group the N*K slots by expert.

    Slots are numbered i = n*K + k.  Histogram then exclusive prefix sum give
    ``expert_offsets`` (ybb.press 2.2; zoe.im 范式 A, offsets [0,3,5,8] for
    its 8-token example).  Walking the slots in ascending order, each takes
    the next free row of its expert's segment, so every segment lists its
    tokens in token order, as in the example.

    cap None : contiguous segments, offsets[e+1] = offsets[e] + counts[e].
    cap int  : padded segments [e*cap, (e+1)*cap); slots past the capacity
               are dropped (slot_row = -1); unused rows have row_token = -1.

    Returns counts [E] (raw, before any drop), offsets [E+1], row_token [R],
    slot_row [N*K].
    """
    ids = np.asarray(topk_ids, dtype=np.int64)
    N, K = ids.shape
    flat = ids.reshape(-1)
    S = N * K
    counts = np.zeros(E, dtype=np.int64)
    for i in range(S):
        counts[flat[i]] += 1
    if cap is None:
        offsets = np.zeros(E + 1, dtype=np.int64)
        for e in range(E):
            offsets[e + 1] = offsets[e] + counts[e]
        R = S
    else:
        offsets = np.arange(E + 1, dtype=np.int64) * cap
        R = E * cap
    run = np.zeros(E, dtype=np.int64)
    row_token = np.full(R, -1, dtype=np.int64)
    slot_row = np.full(S, -1, dtype=np.int64)
    for i in range(S):
        e = flat[i]
        if cap is None or run[e] < cap:
            row = offsets[e] + run[e]
            row_token[row] = i // K
            slot_row[i] = row
        run[e] += 1
    return (counts.astype(np.int32), offsets.astype(np.int32),
            row_token.astype(np.int32), slot_row.astype(np.int32))


def gather_rows(x_bits, row_token) -> np.ndarray:
    """x_perm[row] = x[row_token[row]] (bit copy); padding rows are zero."""
    x = np.asarray(x_bits, dtype=np.uint16)
    rt = np.asarray(row_token, dtype=np.int64)
    out = np.zeros((rt.shape[0], x.shape[1]), dtype=np.uint16)
    valid = rt >= 0
    out[valid] = x[rt[valid]]
    return out


# --------------------------------------------------------------------------
# expert FFN and combine
# --------------------------------------------------------------------------

def silu(g):
    return g / (1.0 + np.exp(-g))


def swiglu_rows(a, wg_bits, wu_bits, wd_bits):
    """One expert's FFN on rows a [m, D] (float64 values).

    g = fl32(a Wg^T), u = fl32(a Wu^T) (float64 sums rounded to fp32);
    h = bf16(fl32(silu(g) * u)); out = bf16(fl32(h Wd^T)).  Wg, Wu are [F, D]
    and Wd is [D, F] (nn.Linear layout).  Returns (h, out) as float64 arrays
    holding bf16 values.
    """
    wg = bf16_to_f64(wg_bits)
    wu = bf16_to_f64(wu_bits)
    wd = bf16_to_f64(wd_bits)
    g = _f32(a @ wg.T)
    u = _f32(a @ wu.T)
    h = round_bf16(_f32(silu(g) * u))
    out = round_bf16(_f32(h @ wd.T))
    return h, out


def expert_ffn(x_perm_bits, offsets, w_gate_bits, w_up_bits, w_down_bits):
    """Run each expert's FFN over its own segment of the permuted buffer.

    zoe.im 范式 A Step 2: expert e maps its (m_e, D) rows to (m_e, F) and back
    to (m_e, D).  Experts with an empty segment are skipped (jsqmd.com 4.2).
    Returns (h [R, F], out_perm [R, D]) as float64 arrays of bf16 values.
    """
    xp = bf16_to_f64(x_perm_bits)
    offsets = np.asarray(offsets, dtype=np.int64)
    E = offsets.shape[0] - 1
    R, D = xp.shape
    F = np.asarray(w_gate_bits).shape[1]
    h_all = np.zeros((R, F))
    out = np.zeros((R, D))
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        h, o = swiglu_rows(xp[lo:hi], w_gate_bits[e], w_up_bits[e], w_down_bits[e])
        h_all[lo:hi] = h
        out[lo:hi] = o
    return h_all, out


def combine(out_perm, slot_row, topk_w) -> np.ndarray:
    """y[n] = bf16(fl32( sum_k w[n,k] * out_perm[slot_row[n*K+k]] )), k ascending, kept slots only.

    zoe.im 范式 A Step 3: restore token order and multiply by the router
    weights; the opening dataflow then sums the K weighted results.
    """
    op = np.asarray(out_perm, dtype=np.float64)
    w = np.asarray(topk_w, dtype=np.float32).astype(np.float64)
    N, K = w.shape
    sr = np.asarray(slot_row, dtype=np.int64).reshape(N, K)
    y = np.zeros((N, op.shape[1]))
    for k in range(K):
        rows = sr[:, k]
        kept = rows >= 0
        y[kept] += w[kept, k][:, None] * op[rows[kept]]
    return round_bf16(_f32(y))


# --------------------------------------------------------------------------
# whole layer
# --------------------------------------------------------------------------

def forward(x_bits, w_router, bias, w_gate_bits, w_up_bits, w_down_bits,
            K: int, gating: str, cap: int | None = None, logits=None) -> dict:
    """The whole layer.  If ``logits`` is given it replaces the router GEMM
    (used to check selection on exactly the fp32 logits another side produced).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    E = np.asarray(w_router).shape[0]
    if logits is None:
        logits = router_logits(x_bits, w_router)
    ids, w = route_from_logits(logits, bias, K, gating)
    counts, offsets, row_token, slot_row = permute(ids, E, cap)
    x_perm = gather_rows(x_bits, row_token)
    h, out_perm = expert_ffn(x_perm, offsets, w_gate_bits, w_up_bits, w_down_bits)
    y = combine(out_perm, slot_row, w)
    return dict(logits=logits, topk_ids=ids, topk_weights=w, expert_counts=counts,
                expert_offsets=offsets, row_token=row_token, slot_row=slot_row,
                x_perm=x_perm, h=h, out_perm=out_perm, y=y)


def token_outputs(x_bits, topk_ids, topk_w, kept_mask, expert_weights, rows_fn=None):
    """y for a subset of tokens, one token at a time (for large layers).

    x_bits [n, D]; topk_ids / topk_w / kept_mask [n, K]; ``expert_weights(e)``
    returns the weights of expert e as ``rows_fn`` takes them after the rows:
    (Wg, Wu, Wd) bf16 bit arrays for the SwiGLU expert (default), (W1, b1,
    W2, b2) with ``rows_fn=gelu_ffn_rows``.  Per token:
    y = bf16(sum_k w_k * out_k) with out_k the expert FFN of that token's row.
    Returns (y [n, D], out [n, K, D]) as float64 arrays of bf16 values.
    """
    rows_fn = swiglu_rows if rows_fn is None else rows_fn
    xs = bf16_to_f64(x_bits)
    n, K = np.asarray(topk_ids).shape
    D = xs.shape[1]
    outs = np.zeros((n, K, D))
    need = {}
    for t in range(n):
        for k in range(K):
            if kept_mask[t, k]:
                need.setdefault(int(topk_ids[t, k]), []).append((t, k))
    for e, pairs in sorted(need.items()):
        rows = np.stack([xs[t] for t, _ in pairs])
        _, o = rows_fn(rows, *expert_weights(e))
        for j, (t, k) in enumerate(pairs):
            outs[t, k] = o[j]
    w = np.asarray(topk_w, dtype=np.float32).astype(np.float64)
    y = np.zeros((n, D))
    for k in range(K):
        y += np.where(np.asarray(kept_mask)[:, k:k + 1], w[:, k:k + 1] * outs[:, k], 0.0)
    return round_bf16(_f32(y)), outs


# --------------------------------------------------------------------------
# routing statistics (ybb.press 4.1)
# --------------------------------------------------------------------------

def routing_stats(counts, ema, bias, decay: float = 0.99, step: float = 0.1):
    """One update of the router's load statistics and dynamic bias.

    ybb.press 4.1: the batch's expert fraction f_e = count_e / sum(count)
    (``_update_load_balance_stats``), the EMA ema_e <- decay*ema_e +
    (1-decay)*f_e, then ``expert_fraction = ema / ema.sum()`` and
    ``dynamic_bias += (E * expert_fraction - 1) * step`` (``load_balance_loss``,
    step 0.1 on the page).  As printed the update raises the bias of experts
    above the uniform share; ``step`` is a parameter, so a caller wanting the
    opposite direction passes a negative step.

    Reading for a batch with no slots (sum of counts 0): nothing changes.
    Returns (ema, bias) as float64.
    """
    c = np.asarray(counts, dtype=np.float64)
    ema = np.asarray(ema, dtype=np.float64)
    bias = np.asarray(bias, dtype=np.float64)
    E = c.shape[0]
    tot = c.sum()
    if tot == 0:
        return ema.copy(), bias.copy()
    f = c / tot
    ema_new = decay * ema + (1.0 - decay) * f
    frac = ema_new / ema_new.sum()
    bias_new = bias + (E * frac - 1.0) * step
    return ema_new, bias_new


# --------------------------------------------------------------------------
# block-scaled FP8 expert weights
# --------------------------------------------------------------------------
#
# The pages store expert weights in fewer bits: FP8 weights inside the
# grouped-GEMM kernel ("MoE 推理完整机制" (zoe.im), 第四层 DeepGEMM & MegaMoE
# Kernel) and 8-bit expert weights dequantised before use ("MoE工程实战"
# (jsqmd.com), 5.3 技巧2).  Neither fixes a format.  Reading taken here: the
# OCP microscaling layout with FP8 E4M3 elements -- blocks of 32 consecutive
# values along the contraction (input) dimension of a weight row share one
# power-of-two scale 2^s stored as a biased 8-bit exponent (E8M0, byte
# s + 127); each element is an E4M3 code (1 sign, 4 exponent bits with bias
# 7, 3 mantissa bits; the all-ones magnitude S.1111.111 is NaN, there is no
# infinity, the largest finite value is 448).

E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUBNORMAL_STEP = 2.0 ** -9
MX_BLOCK = 32
MX_EMAX_ELEM = 8          # exponent of the largest E4M3 binade (448 = 1.75 * 2^8)
MX_SCALE_MIN = -117       # 2^-9 * 2^-117 = 2^-126: every dequantised value stays normal
MX_SCALE_MAX = 119        # floor(log2(largest bf16)) - 8


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 codes (uint8) -> float64 values.

    exponent field 0: subnormal, M * 2^-9; else (8 + M) * 2^(E - 10), i.e.
    (1 + M/8) * 2^(E - 7); S.1111.111 is NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    neg = (c >> 7) & 1
    ef = (c >> 3) & 15
    mf = c & 7
    mag = np.where(ef == 0, mf * E4M3_SUBNORMAL_STEP,
                   np.ldexp((8 + mf).astype(np.float64), ef - 10))
    mag = np.where((ef == 15) & (mf == 7), np.nan, mag)
    return np.where(neg == 1, -mag, mag)


def e4m3_encode(t) -> np.ndarray:
    """float64 values -> E4M3 codes, round to nearest even, saturating.

    Finite magnitudes above 448 become 448 (the OCP MX conversion saturates);
    non-finite values become NaN (0x7F with the input's sign bit).  The grid
    step is 2^(floor(log2|t|) - 3) in the normal range (|t| >= 2^-6) and
    2^-9 below it; a carry out of the mantissa moves to the next binade.
    """
    t = np.asarray(t, dtype=np.float64)
    neg = np.signbit(t)
    fin = np.isfinite(t)
    a = np.where(fin, np.minimum(np.abs(t), E4M3_MAX), 0.0)
    _, ex = np.frexp(a)                       # a = m * 2^ex, 0.5 <= m < 1
    step = np.where(a >= E4M3_MIN_NORMAL, ex - 1 - 3, -9)
    v = np.ldexp(np.rint(np.ldexp(a, -step)), step)   # rounded magnitude
    mv, ev = np.frexp(v)
    normal = v >= E4M3_MIN_NORMAL
    mag = np.where(normal,
                   ((ev - 1 + 7) << 3) + np.rint((2.0 * mv - 1.0) * 8).astype(np.int64),
                   np.rint(v / E4M3_SUBNORMAL_STEP).astype(np.int64))
    mag = np.where(fin, mag, 0x7F)
    return (mag | (neg.astype(np.int64) << 7)).astype(np.uint8)


def mx_block_exponent(amax) -> np.ndarray:
    """Shared exponent of a block from its largest finite magnitude.

    floor(log2(amax)) - 8, so the block's largest value lands in the top
    E4M3 binade [256, 512) (saturating above 448); clamped to
    [-117, 119] so that every dequantised value is a normal bf16 number.  An
    all-zero block takes the lower clamp.
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)
    e = np.where(amax > 0, ex - 1 - MX_EMAX_ELEM, MX_SCALE_MIN)
    return np.clip(e, MX_SCALE_MIN, MX_SCALE_MAX).astype(np.int64)


def quantize_fp8(w_bits):
    """bf16 weights [..., K] -> (codes uint8 [..., K], scales uint8 [..., K/32]).

    Per block of 32 consecutive values of the last (contraction) axis:
    s = mx_block_exponent(largest finite |w|), element code =
    e4m3_encode(w / 2^s) (the division by a power of two is exact), scale
    byte = s + 127.
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    K = w_bits.shape[-1]
    if K % MX_BLOCK:
        raise ValueError("contraction length must be a multiple of 32")
    flat = w_bits.reshape(-1, K)
    codes = np.empty(flat.shape, dtype=np.uint8)
    scales = np.empty((flat.shape[0], K // MX_BLOCK), dtype=np.uint8)
    for r0 in range(0, flat.shape[0], 256):     # rows are independent; 256 at a time
        blk = bf16_to_f64(flat[r0:r0 + 256]).reshape(-1, K // MX_BLOCK, MX_BLOCK)
        amax = np.max(np.where(np.isfinite(blk), np.abs(blk), 0.0), axis=-1)
        s = mx_block_exponent(amax)
        codes[r0:r0 + 256] = e4m3_encode(np.ldexp(blk, -s[..., None])).reshape(-1, K)
        scales[r0:r0 + 256] = s + 127
    return (codes.reshape(w_bits.shape),
            scales.reshape(w_bits.shape[:-1] + (K // MX_BLOCK,)))


def dequantize_fp8(codes, scales) -> np.ndarray:
    """value = e4m3_decode(code) * 2^(scale - 127), float64 (exact in bf16)."""
    c = np.asarray(codes, dtype=np.uint8)
    s = np.asarray(scales, dtype=np.uint8).astype(np.int64) - 127
    K = c.shape[-1]
    v = e4m3_decode(c).reshape(c.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    return np.ldexp(v, s[..., None]).reshape(c.shape)


def dequantize_fp8_bits(codes, scales) -> np.ndarray:
    """dequantize_fp8 as raw bf16 bit patterns (the conversion is exact)."""
    return f64_to_bf16_bits(dequantize_fp8(codes, scales))


def expert_ffn_fp8(x_perm_bits, offsets, wg_q, wu_q, wd_q):
    """Grouped SwiGLU FFN with block-scaled FP8 weights.

    Each weight argument is a (codes, scales) pair from quantize_fp8.  The
    weights enter the FFN as their dequantised values (exact bf16 numbers),
    so this is expert_ffn on those values.
    """
    return expert_ffn(x_perm_bits, offsets, dequantize_fp8_bits(*wg_q),
                      dequantize_fp8_bits(*wu_q), dequantize_fp8_bits(*wd_q))


# --------------------------------------------------------------------------
# GELU-expert layer with an MLP router (jsqmd.com 3.1 and 4.2)
# --------------------------------------------------------------------------
#
# Readings: nn.Linear carries a bias unless told otherwise, so every Linear
# here has one; nn.GELU's default is the exact (erf) form.  Storage points as
# in the SwiGLU layer: the router's compressed features, the expert hidden
# activations and the expert outputs are bf16; the gate logits are fp32.  The
# gate Linear's bias enters the top-K as the per-expert bias (key = logit +
# bias, one fp32 add), which is the same selection and softmax as on the
# biased logits.

def gelu(v):
    """v * Phi(v), Phi(v) = 0.5 (1 + erf(v / sqrt(2))) = 0.5 erfc(-v / sqrt(2)); the
    erfc form keeps full relative accuracy where 1 + erf cancels (v << 0)."""
    v = np.asarray(v, dtype=np.float64)
    return 0.5 * v * erfc(-v / math.sqrt(2.0))


def mlp_router_features(x_bits, w_proj_bits, b_proj) -> np.ndarray:
    """a = bf16(GELU(x W_proj^T + b_proj)), [N, D/4]: the compression MLP in
    front of the gate (jsqmd.com 3.1 输入表征; ``gate_proj`` + ``gate_act``)."""
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_proj_bits)
    b = np.asarray(b_proj, dtype=np.float32).astype(np.float64)
    return round_bf16(_f32(gelu(_f32(_f32(x @ w.T) + b))))


def mlp_router_logits(a, w_out) -> np.ndarray:
    """logits = fp32(a W_out^T) over the compressed features (``gate_out``
    without its bias, which joins the selection as the per-expert bias)."""
    a = np.asarray(a, dtype=np.float64)
    w = np.asarray(w_out, dtype=np.float32).astype(np.float64)
    return round_f32(a @ w.T)


def gelu_ffn_rows(a, w1_bits, b1, w2_bits, b2):
    """One GELU expert on rows a [m, D]: h = bf16(fl32(GELU(v))) with
    v = fl32(fl32(a W1^T) + b1), out = bf16(fl32(fl32(h W2^T) + b2)); W1 [F, D],
    W2 [D, F] (nn.Linear layout).  fl32 marks the fp32 roundings of the GPU's
    arithmetic: the dot, the bias add, the activation."""
    w1 = bf16_to_f64(w1_bits)
    w2 = bf16_to_f64(w2_bits)
    b1 = np.asarray(b1, dtype=np.float32).astype(np.float64)
    b2 = np.asarray(b2, dtype=np.float32).astype(np.float64)
    h = round_bf16(_f32(gelu(_f32(_f32(a @ w1.T) + b1))))
    out = round_bf16(_f32(_f32(h @ w2.T) + b2))
    return h, out


def expert_ffn_gelu(x_perm_bits, offsets, w1_bits, b1, w2_bits, b2):
    """Each GELU expert over its own segment; empty experts skipped
    (jsqmd.com 4.2 ``numel() > 0``).  Padding rows of a capacity-padded
    buffer are zero inputs and get the expert's response to a zero row.
    Returns (h [R, F], out_perm [R, D]) as float64 arrays of bf16 values."""
    xp = bf16_to_f64(x_perm_bits)
    offsets = np.asarray(offsets, dtype=np.int64)
    E = offsets.shape[0] - 1
    R, D = xp.shape
    F = np.asarray(w1_bits).shape[1]
    h_all = np.zeros((R, F))
    out = np.zeros((R, D))
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        h, o = gelu_ffn_rows(xp[lo:hi], w1_bits[e], b1[e], w2_bits[e], b2[e])
        h_all[lo:hi] = h
        out[lo:hi] = o
    return h_all, out


def forward_gelu(x_bits, w_proj_bits, b_proj, w_out, b_out, w1_bits, b1, w2_bits, b2,
                 K: int, cap: int | None = None, logits=None,
                 gating: str = GATING_SOFTMAX) -> dict:
    """The GELU-expert layer: MLP router, top-K with softmax over the K
    selected (jsqmd.com 4.2; ``gating`` may also name the sigmoid variant),
    permutation, GELU experts, weighted combine.  If ``logits`` is given it
    replaces the router (selection on exactly the fp32 logits another side
    produced)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    E = np.asarray(w_out).shape[0]
    feats = None
    if logits is None:
        feats = mlp_router_features(x_bits, w_proj_bits, b_proj)
        logits = mlp_router_logits(feats, w_out)
    ids, w = route_from_logits(logits, b_out, K, gating)
    counts, offsets, row_token, slot_row = permute(ids, E, cap)
    x_perm = gather_rows(x_bits, row_token)
    h, out_perm = expert_ffn_gelu(x_perm, offsets, w1_bits, b1, w2_bits, b2)
    y = combine(out_perm, slot_row, w)
    return dict(features=feats, logits=logits, topk_ids=ids, topk_weights=w,
                expert_counts=counts, expert_offsets=offsets, row_token=row_token,
                slot_row=slot_row, x_perm=x_perm, h=h, out_perm=out_perm, y=y)
