"""Seeded synthetic inputs for the single-GPU MoE-layer forward pass.

This module is shared by the oracle tests, the GPU parity tests and the
benchmark.  It draws the layer's inputs (hidden states, router weights,
per-expert bias and expert weights) and holds none of the layer's own
arithmetic: no routing, no permutation, no FFN, no combine.

Generator (device independent, bit-identical on CPU and GPU)
-----------------------------------------------------------
* Counter-based: element ``i`` of stream ``s`` under seed ``seed`` is a pure
  function of ``(seed, s, i)``.  Two 32-bit words are drawn per element from
  counters ``2i`` and ``2i+1`` with Chris Wellons' "lowbias32" integer mixer
  (xorshift-multiply, constants 0x7feb352d / 0x846ca68b), applied twice.
* The four 16-bit halves of those words are summed (an Irwin-Hall(4) draw),
  centred and scaled: ``v = fp32(2*sum - 4*65535) * fp32(std / sd_IH)``.
  The integer part is exact in fp32 and the scaling is one IEEE fp32
  multiply, so every backend produces the same bits.  The draw has mean 0 and
  standard deviation ``std`` and is bounded at +-sqrt(12)*std (about
  3.46 std); it is a standard stand-in for a normal variate.
* bf16 tensors are the fp32 draw rounded to nearest-even (torch's cast).

All integer work stays below 2**63 in int64: the 32-bit multiply is split
into 16-bit halves, so no signed overflow happens on any device.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import torch

_MASK32 = 0xFFFFFFFF
_C1 = 0x7FEB352D
_C2 = 0x846CA68B


def _mul32_t(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2**32 for int64 tensors holding values in [0, 2**32)."""
    lo = c & 0xFFFF
    hi = c >> 16
    return (x * lo + (((x * hi) & 0xFFFF) << 16)) & _MASK32


def _hash32_t(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32_t(x, _C1)
    x = x ^ (x >> 15)
    x = _mul32_t(x, _C2)
    return x ^ (x >> 16)


def _hash32(x: int) -> int:
    x &= _MASK32
    x ^= x >> 16
    x = (x * _C1) & _MASK32
    x ^= x >> 15
    x = (x * _C2) & _MASK32
    return x ^ (x >> 16)


def stream_key(seed: int, stream: int) -> int:
    """32-bit key of one named stream under one seed."""
    return _hash32(_hash32(seed ^ 0x632BE5AB) ^ _hash32(stream + 0x9E3779B9))


def uint32_words(numel: int, seed: int, stream: int, offset: int = 0,
                 device="cpu") -> Tuple[torch.Tensor, torch.Tensor]:
    """Two independent 32-bit words (as int64) for elements offset..offset+numel-1."""
    key = stream_key(seed, stream)
    idx = torch.arange(offset, offset + numel, dtype=torch.int64, device=device)
    out = []
    for j in (0, 1):
        c = idx * 2 + j
        lo = c & _MASK32
        hi = c >> 32
        h = _hash32_t(lo ^ key)
        h = _hash32_t((h + hi) & _MASK32)
        out.append(h)
    return out[0], out[1]


_IH_SD = math.sqrt(16.0 * (65536.0 ** 2 - 1.0) / 12.0)


def normal_f32(numel: int, std: float, seed: int, stream: int, offset: int = 0,
               device="cpu") -> torch.Tensor:
    """fp32 draws with mean 0 and standard deviation ``std`` (Irwin-Hall(4))."""
    w0, w1 = uint32_words(numel, seed, stream, offset, device)
    s = (w0 & 0xFFFF) + (w0 >> 16) + (w1 & 0xFFFF) + (w1 >> 16)
    centred = (2 * s - 4 * 65535).to(torch.float32)          # exact: |.| < 2**19
    scale = torch.tensor(std / _IH_SD, dtype=torch.float32, device=device)
    return centred * scale                                    # one IEEE fp32 multiply


def normal_bf16(numel: int, std: float, seed: int, stream: int, offset: int = 0,
                device="cpu") -> torch.Tensor:
    return normal_f32(numel, std, seed, stream, offset, device).to(torch.bfloat16)


def uniform_ranks(n: int, seed: int, stream: int) -> list:
    """A seeded permutation of the ranks 1..n (rank of item e at position e)."""
    key = stream_key(seed, stream)
    h = [_hash32(_hash32(e ^ key)) for e in range(n)]
    order = sorted(range(n), key=lambda e: (h[e], e))
    ranks = [0] * n
    for r, e in enumerate(order):
        ranks[e] = r + 1
    return ranks


# ---------------------------------------------------------------------------
# Workloads.  Shapes follow the layers the pages talk about (Mixtral-8x7B,
# DeepSeek-V3, Qwen3-30B-A3B) plus a tiny case and a hot-expert skew case.
# ---------------------------------------------------------------------------

STREAM_X, STREAM_WR, STREAM_WG, STREAM_WU, STREAM_WD, STREAM_BIAS = range(6)
# streams of the GELU-expert layer with the MLP router
(STREAM_WPROJ, STREAM_BPROJ, STREAM_WOUT, STREAM_BOUT, STREAM_W1, STREAM_B1, STREAM_W2,
 STREAM_B2) = range(6, 14)


@dataclass(frozen=True)
class MoEConfig:
    name: str
    N: int            # tokens
    D: int            # hidden size
    E: int            # experts
    K: int            # experts per token
    F: int            # expert FFN width
    gating: str       # "softmax" (softmax over the K selected) or "sigmoid" (renormalised)
    seed: int
    zipf_s: Optional[float] = None       # Zipf exponent of the per-expert bias
    zipf_alpha: Optional[float] = None   # bias = alpha * log Zipf pmf
    capacity: Optional[Tuple[int, int]] = None  # (num, den) capacity factor for the padded run
    note: str = ""
    expert: str = "swiglu"   # "swiglu" (gate/up/down) or "gelu" (Linear-GELU-Linear, MLP router)

    @property
    def S(self) -> int:
        return self.N * self.K

    @property
    def gating_id(self) -> int:
        return 0 if self.gating == "softmax" else 1

    def flops(self) -> float:
        """Algorithmic flops of one forward pass: router + expert FFN over all slots."""
        if self.expert == "gelu":
            R = self.D // 4
            return 2.0 * self.N * (self.D * R + R * self.E) + 4.0 * self.D * self.F * self.S
        return 2.0 * self.N * self.D * self.E + 6.0 * self.D * self.F * self.S

    def scaled(self, **kw) -> "MoEConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return MoEConfig(**d)


CONFIGS: Dict[str, MoEConfig] = {
    "tiny": MoEConfig("tiny", N=64, D=256, E=8, K=2, F=512, gating="softmax",
                      seed=0x5EED0001, note="tiny layer, oracle in seconds"),
    "mixtral": MoEConfig("mixtral", N=4096, D=4096, E=8, K=2, F=14336, gating="softmax",
                         seed=0x5EED0002, note="Mixtral-8x7B layer shape, prefill"),
    "deepseek_v3": MoEConfig("deepseek_v3", N=8192, D=7168, E=256, K=8, F=2048,
                             gating="sigmoid", seed=0x5EED0003,
                             note="DeepSeek-V3 layer shape, all 256 experts on one GPU"),
    "qwen3_decode": MoEConfig("qwen3_decode", N=64, D=2048, E=128, K=8, F=768,
                              gating="softmax", seed=0x5EED0004,
                              note="Qwen3-30B-A3B layer shape, decode step"),
    # the GELU-expert layer: Linear(D, 4D)-GELU-Linear(4D, D) experts with biases
    # and the MLP router D -> D/4 (GELU) -> E; top-2 softmax
    "gelu_mlp": MoEConfig("gelu_mlp", N=4096, D=4096, E=8, K=2, F=16384, gating="softmax",
                          seed=0x5EED0006, expert="gelu",
                          note="GELU-expert layer with MLP router (D=4096, F=4D), prefill"),
    "gelu_tiny": MoEConfig("gelu_tiny", N=64, D=256, E=8, K=2, F=1024, gating="softmax",
                           seed=0x5EED0007, expert="gelu",
                           note="tiny GELU-expert layer, oracle in seconds"),
    # zipf_alpha: chosen so that the most-favoured expert receives about a quarter
    # of all slots at this seed (checked by tests/test_oracle_pins.py with the oracle).
    "hot_skew": MoEConfig("hot_skew", N=16384, D=4096, E=64, K=2, F=8192, gating="softmax",
                          seed=0x5EED0005, zipf_s=1.2, zipf_alpha=0.62, capacity=(5, 4),
                          note="hot-expert skew, Zipf(1.2) bias; contiguous and padded (cf 1.25)"),
}


def zipf_bias(E: int, s: float, alpha: float, seed: int) -> torch.Tensor:
    """bias_e = alpha * log p(rank_e), p = Zipf(s) pmf over ranks 1..E (fp32)."""
    ranks = uniform_ranks(E, seed, STREAM_BIAS)
    H = sum(r ** (-s) for r in range(1, E + 1))
    vals = [alpha * (-s * math.log(r) - math.log(H)) for r in ranks]
    return torch.tensor(vals, dtype=torch.float64).to(torch.float32)


def expert_weight(cfg: MoEConfig, which: str, e: int, device="cpu") -> torch.Tensor:
    """One expert's weight matrix (bf16), [F,D] for gate/up and [D,F] for down."""
    std = 1.0 / math.sqrt(cfg.D)
    stream = {"gate": STREAM_WG, "up": STREAM_WU, "down": STREAM_WD}[which]
    n = cfg.F * cfg.D
    t = normal_bf16(n, std, cfg.seed, stream, offset=e * n, device=device)
    return t.view(cfg.F, cfg.D) if which != "down" else t.view(cfg.D, cfg.F)


def make_inputs(cfg: MoEConfig, device="cpu", with_experts: bool = True) -> dict:
    """All inputs of one layer.

    x [N,D] bf16 ~ std 1; w_router [E,D] fp32 ~ std 1/sqrt(D) (nn.Linear layout);
    w_gate, w_up [E,F,D] and w_down [E,D,F] bf16 ~ std 1/sqrt(D);
    bias [E] fp32 (Zipf case only, else None).
    """
    N, D, E, F = cfg.N, cfg.D, cfg.E, cfg.F
    out = {
        "x": normal_bf16(N * D, 1.0, cfg.seed, STREAM_X, device=device).view(N, D),
        "w_router": normal_f32(E * D, 1.0 / math.sqrt(D), cfg.seed, STREAM_WR,
                               device=device).view(E, D),
        "bias": None,
    }
    if cfg.zipf_s is not None:
        out["bias"] = zipf_bias(E, cfg.zipf_s, cfg.zipf_alpha, cfg.seed).to(device)
    if with_experts:
        for which, shape in (("gate", (F, D)), ("up", (F, D)), ("down", (D, F))):
            t = torch.empty((E,) + shape, dtype=torch.bfloat16, device=device)
            for e in range(E):
                t[e] = expert_weight(cfg, which, e, device)
            out["w_" + which] = t
    return out


def make_gelu_inputs(cfg: MoEConfig, device="cpu") -> dict:
    """All inputs of one GELU-expert layer (nn.Linear layouts, [out, in]).

    Weights have std 1/sqrt(fan_in) and biases std 1/sqrt(3 fan_in) (the
    spread of nn.Linear's default uniform bias init):
    x [N,D] bf16 ~ std 1;
    router: w_proj [D/4, D] bf16, b_proj [D/4] fp32, w_out [E, D/4] fp32, b_out [E] fp32;
    experts: w1 [E,F,D] bf16, b1 [E,F] fp32, w2 [E,D,F] bf16, b2 [E,D] fp32.
    """
    N, D, E, F = cfg.N, cfg.D, cfg.E, cfg.F
    Dr = D // 4
    sd, sdr, sf = 1.0 / math.sqrt(D), 1.0 / math.sqrt(Dr), 1.0 / math.sqrt(F)
    s = cfg.seed
    return {
        "x": normal_bf16(N * D, 1.0, s, STREAM_X, device=device).view(N, D),
        "w_proj": normal_bf16(Dr * D, sd, s, STREAM_WPROJ, device=device).view(Dr, D),
        "b_proj": normal_f32(Dr, sd / math.sqrt(3.0), s, STREAM_BPROJ, device=device),
        "w_out": normal_f32(E * Dr, sdr, s, STREAM_WOUT, device=device).view(E, Dr),
        "b_out": normal_f32(E, sdr / math.sqrt(3.0), s, STREAM_BOUT, device=device),
        "w1": normal_bf16(E * F * D, sd, s, STREAM_W1, device=device).view(E, F, D),
        "b1": normal_f32(E * F, sd / math.sqrt(3.0), s, STREAM_B1, device=device).view(E, F),
        "w2": normal_bf16(E * D * F, sf, s, STREAM_W2, device=device).view(E, D, F),
        "b2": normal_f32(E * D, sf / math.sqrt(3.0), s, STREAM_B2, device=device).view(E, D),
    }
