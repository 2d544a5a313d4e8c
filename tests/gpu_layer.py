"""Shared helpers of the GPU parity tests: run the layer through the C ABI on
seeded inputs and compare it with the CPU oracle.  Imported by the GPU tests
only; nothing here runs a kernel at import time."""
from __future__ import annotations

import math

import numpy as np
import torch

import mixture_experts_layer_level_amd as moe
import moe_synth as ms
from oracle import moe_oracle as O

DEV = "cuda"

# Small workloads that together cover every tile shape and edge case of the
# path; each runs in seconds against the oracle.
C = ms.MoEConfig
SMALL = {
    "tiny": ms.CONFIGS["tiny"],
    # ragged: N not a tile multiple, F = 192 leaves a half-empty column tile
    "ragged": C("ragged", N=333, D=320, E=6, K=2, F=192, gating="softmax", seed=101),
    # small-row tiles (about 6 rows per expert), sigmoid gating
    "decode_like": C("decode_like", N=50, D=128, E=32, K=4, F=256, gating="sigmoid", seed=102),
    # two experts of about 350 rows: two row tiles each, the second ragged
    "two_big_experts": C("two_big_experts", N=700, D=256, E=2, K=1, F=128, gating="softmax",
                         seed=103),
    "single_expert": C("single_expert", N=300, D=192, E=1, K=1, F=128, gating="softmax", seed=104),
    "k_equals_e": C("k_equals_e", N=40, D=128, E=4, K=4, F=64, gating="sigmoid", seed=105),
    # strong Zipf bias: several experts receive no token at all
    "empty_experts": C("empty_experts", N=90, D=128, E=16, K=2, F=128, gating="softmax",
                       seed=106, zipf_s=1.2, zipf_alpha=4.0),
    # about 550 rows per expert: 256 x 256 ring tiles, ragged last row tile,
    # F = 192 leaves half of the second h column tile empty
    "large_tiles": C("large_tiles", N=1100, D=320, E=2, K=1, F=192, gating="softmax", seed=109),
    # about 240 rows per expert: 128 x 256 ring tiles
    "mid_tiles": C("mid_tiles", N=960, D=384, E=8, K=2, F=320, gating="sigmoid", seed=110),
    # K = 12: the combine and copy kernels take the slots of a token in groups of 8
    "wide_topk": C("wide_topk", N=80, D=128, E=32, K=12, F=128, gating="softmax", seed=111),
    # 100 experts, 200 rows each on average under a Zipf bias (8 empty, most
    # under 32 rows, the largest 5837 rows: 23 row tiles in bands): 256 x 256
    # split-ring tiles with the work list in four registers per lane
    "many_large_experts": C("many_large_experts", N=10000, D=128, E=100, K=2, F=128,
                            gating="sigmoid", seed=112, zipf_s=1.2, zipf_alpha=0.7),
    # 256 x 256 tiles with one 64-deep stage in the gate/up GEMM (D = 64) and
    # two in the down GEMM (F = 128): the rings' shortest prologues
    "short_k_large_tiles": C("short_k_large_tiles", N=1300, D=64, E=2, K=1, F=128,
                             gating="softmax", seed=113),
    # 300 experts of about 200 rows: 256 x 256 tiles with more experts than the
    # split rings' register work list holds (the 2-slot ring, and the fused
    # FFN on it)
    "many_experts_ring": C("many_experts_ring", N=30000, D=128, E=300, K=2, F=192,
                           gating="softmax", seed=114),
    # few router tiles over a long k: 8 waves share a 32 x 32 router tile's 17
    # k blocks (one takes three), ragged token and expert tiles
    "wide_router": C("wide_router", N=40, D=1088, E=48, K=4, F=128, gating="sigmoid",
                     seed=115),
    # 1100 tokens of D = 1024: the combine runs one workgroup per token with
    # the slot rows and weights in scalar registers (padded: with drops)
    "wide_rows": C("wide_rows", N=1100, D=1024, E=8, K=3, F=128, gating="softmax", seed=116),
    "wide_rows_padded": C("wide_rows_padded", N=1100, D=1024, E=8, K=3, F=128, gating="sigmoid",
                          seed=117, zipf_s=1.2, zipf_alpha=1.0, capacity=(1, 2)),
    # 1040 chunks of 8 values per row: more than one chunk per combine thread
    "very_wide_rows": C("very_wide_rows", N=1024, D=8320, E=4, K=2, F=64, gating="softmax",
                        seed=118),
    "padded": C("padded", N=200, D=256, E=8, K=2, F=320, gating="softmax", seed=107,
                zipf_s=1.2, zipf_alpha=1.0, capacity=(5, 4)),
    "padded_small_rows": C("padded_small_rows", N=60, D=128, E=16, K=2, F=128,
                           gating="softmax", seed=108, zipf_s=1.2, zipf_alpha=1.0,
                           capacity=(1, 2)),
}


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def np_(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def assert_fp_close(got, ref, what: str):
    """max|d| <= 1e-2 * max|ref| and |d_i| <= 1e-2 * max|ref| + 2e-2 * |ref_i|."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if ref.size == 0:
        return
    M = float(np.abs(ref).max())
    d = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert d.max() <= 1e-2 * M, f"{what}: max|d| {d.max():.3g} > 1e-2 * {M:.3g}"
    bad = d > 1e-2 * M + 2e-2 * np.abs(ref)
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside rtol 2e-2"


def assert_logits_bound(gpu_logits, x_bits, w_router, rows=None):
    """Router logits against the exact dot products, within the fp32
    summation bound.

    The kernel evaluates x.w as an fp32 sum of exact products: each fp32
    weight is cut exactly into three bf16 pieces (|pieces| sum to at most
    (1 + 2**-7)|w|) and every bf16 x bf16 product is exact in fp32.  Each
    product passes through at most 2D + 8 fp32 additions, so
    |gpu - exact| <= gamma_(2D+8) * (1 + 2**-7) * sum_d |x_d w_d|,
    gamma_n = n u / (1 - n u), u = 2**-24.
    """
    x = O.bf16_to_f64(x_bits if rows is None else x_bits[rows])
    w = np.asarray(w_router, dtype=np.float64)
    exact = x @ w.T
    mag = np.abs(x) @ np.abs(w).T
    D = x.shape[1]
    u = 2.0 ** -24
    n = 2 * D + 8
    gamma = n * u / (1 - n * u)
    g = np.asarray(gpu_logits if rows is None else gpu_logits[rows], dtype=np.float64)
    err = np.abs(g - exact)
    assert np.all(err <= gamma * (1 + 2.0 ** -7) * mag + 1e-30)
    # and the observed error is that of a well-conditioned fp32 sum, far
    # inside the worst case
    assert err.max() <= 64 * u * max(1.0, float(np.abs(exact).max())) * np.sqrt(D)


class Layer:
    """Inputs on the GPU plus every buffer of the staged path."""

    def __init__(self, cfg: ms.MoEConfig, padded: bool = False, bias=None):
        self.cfg = cfg
        inp = ms.make_inputs(cfg, device=DEV)
        self.x = inp["x"]
        self.w_router = inp["w_router"]
        self.bias = inp["bias"] if bias is None else bias.to(DEV)
        self.w_gate, self.w_up, self.w_down = inp["w_gate"], inp["w_up"], inp["w_down"]
        cap = cfg.capacity if padded else None
        self.p = moe.problem(cfg.N, cfg.D, cfg.F, cfg.E, cfg.K, cfg.gating, cap)
        self.R, self.cap = moe.permuted_rows(self.p)
        N, D, E, K, F, R = cfg.N, cfg.D, cfg.E, cfg.K, cfg.F, self.R
        z = lambda *s, dt=torch.float32: torch.empty(*s, dtype=dt, device=DEV)
        self.logits = z(N, E)
        self.ids = z(N, K, dt=torch.int32)
        self.w = z(N, K)
        self.counts = z(E, dt=torch.int32)
        self.offsets = z(E + 1, dt=torch.int32)
        self.row_token = z(R, dt=torch.int32)
        self.slot_row = z(N * K, dt=torch.int32)
        self.x_perm = z(R, D, dt=torch.bfloat16)
        self.h = z(R, F, dt=torch.bfloat16)
        self.out_perm = z(R, D, dt=torch.bfloat16)
        self.y = z(N, D, dt=torch.bfloat16)
        self.ws = torch.empty(max(moe.workspace_size(self.p), 256), dtype=torch.uint8, device=DEV)

    def staged(self):
        p = self.p
        moe.route(p, self.x, self.w_router, self.bias, self.logits, self.ids, self.w)
        moe.permute(p, self.x, self.ids, self.counts, self.offsets, self.row_token,
                    self.slot_row, self.x_perm, self.ws)
        moe.expert_gateup(p, self.x_perm, self.offsets, self.w_gate, self.w_up, self.h)
        moe.expert_down(p, self.h, self.offsets, self.w_down, self.out_perm)
        moe.unpermute_combine(p, self.out_perm, self.slot_row, self.w, self.y)
        torch.cuda.synchronize()

    def forward(self, y_out):
        moe.forward(self.p, self.x, self.w_router, self.bias, self.w_gate, self.w_up,
                    self.w_down, y_out, self.ws)
        torch.cuda.synchronize()

    # host copies ---------------------------------------------------------
    def host_inputs(self):
        b = None if self.bias is None else np_(self.bias)
        return bits(self.x), np_(self.w_router), b

    def expert_bits(self, e: int):
        return bits(self.w_gate[e]), bits(self.w_up[e]), bits(self.w_down[e])


def check_routing(L: Layer, sample_rows=None):
    """Logits within the fp32 bound; ids bit-exact and weights within 1e-6 of
    the oracle's selection on the very same fp32 logits."""
    x_bits, wr, bias = L.host_inputs()
    lg = np_(L.logits)
    assert_logits_bound(lg, x_bits, wr, rows=sample_rows)
    ids, w = O.route_from_logits(lg, bias, L.cfg.K, L.cfg.gating)
    assert np.array_equal(np_(L.ids), ids), "top-K ids differ from the oracle"
    assert np.abs(np_(L.w).astype(np.float64) - w).max() <= 1e-6
    return ids, w


def check_permutation(L: Layer):
    cap = L.cap if L.cap else None
    counts, offsets, row_token, slot_row = O.permute(np_(L.ids), L.cfg.E, cap)
    assert np.array_equal(np_(L.counts), counts), "expert_counts"
    assert np.array_equal(np_(L.offsets), offsets), "expert_offsets"
    assert np.array_equal(np_(L.row_token), row_token), "row_token"
    assert np.array_equal(np_(L.slot_row), slot_row), "slot_row"
    return offsets, row_token, slot_row


def sample_tokens(N: int, n: int = 16):
    idx = sorted(set(np.linspace(0, N - 1, n).astype(int).tolist()))
    return np.array(idx, dtype=np.int64)


def check_sampled_outputs(L: Layer, y_gpu: torch.Tensor, tokens):
    """y of sampled tokens against the oracle, one token at a time."""
    x_bits = bits(L.x[torch.as_tensor(tokens, device=DEV)])
    ids = np_(L.ids)[tokens]
    w = np_(L.w)[tokens]
    kept = (np_(L.slot_row).reshape(L.cfg.N, L.cfg.K)[tokens] >= 0)
    y_ref, _ = O.token_outputs(x_bits, ids, w, kept, L.expert_bits)
    y = O.bf16_to_f64(bits(y_gpu)[tokens])
    assert_fp_close(y, y_ref, f"y[{len(tokens)} sampled tokens]")


class GeluLayer:
    """Inputs of the GELU-expert layer on the GPU plus every buffer of its staged path."""

    def __init__(self, cfg: ms.MoEConfig, padded: bool = False):
        self.cfg = cfg
        self.inp = ms.make_gelu_inputs(cfg, device=DEV)
        cap = cfg.capacity if padded else None
        self.p = moe.problem(cfg.N, cfg.D, cfg.F, cfg.E, cfg.K, cfg.gating, cap)
        self.R, self.cap = moe.permuted_rows(self.p)
        N, D, E, K, F, R = cfg.N, cfg.D, cfg.E, cfg.K, cfg.F, self.R
        z = lambda *s, dt=torch.float32: torch.empty(*s, dtype=dt, device=DEV)
        self.feats = z(N, D // 4, dt=torch.bfloat16)
        self.logits = z(N, E)
        self.ids = z(N, K, dt=torch.int32)
        self.w = z(N, K)
        self.counts = z(E, dt=torch.int32)
        self.offsets = z(E + 1, dt=torch.int32)
        self.row_token = z(R, dt=torch.int32)
        self.slot_row = z(N * K, dt=torch.int32)
        self.x_perm = z(R, D, dt=torch.bfloat16)
        self.h = z(R, F, dt=torch.bfloat16)
        self.out_perm = z(R, D, dt=torch.bfloat16)
        self.y = z(N, D, dt=torch.bfloat16)
        self.ws = torch.empty(max(moe.workspace_size(self.p), 256), dtype=torch.uint8, device=DEV)

    def staged(self):
        i, p = self.inp, self.p
        moe.route_mlp(p, i["x"], i["w_proj"], i["b_proj"], i["w_out"], i["b_out"], self.logits,
                      self.ids, self.w, self.ws, features=self.feats)
        moe.permute(p, i["x"], self.ids, self.counts, self.offsets, self.row_token,
                    self.slot_row, self.x_perm, self.ws)
        moe.expert_up_gelu(p, self.x_perm, self.offsets, i["w1"], i["b1"], self.h)
        moe.expert_down_bias(p, self.h, self.offsets, i["w2"], i["b2"], self.out_perm)
        moe.unpermute_combine(p, self.out_perm, self.slot_row, self.w, self.y)
        torch.cuda.synchronize()

    def forward(self, y_out):
        i = self.inp
        moe.forward_gelu(self.p, i["x"], i["w_proj"], i["b_proj"], i["w_out"], i["b_out"],
                         i["w1"], i["b1"], i["w2"], i["b2"], y_out, self.ws)
        torch.cuda.synchronize()

    def host(self, name):
        t = self.inp[name]
        return bits(t) if t.dtype == torch.bfloat16 else np_(t)

    def expert(self, e):
        return (bits(self.inp["w1"][e]), np_(self.inp["b1"][e]), bits(self.inp["w2"][e]),
                np_(self.inp["b2"][e]))
