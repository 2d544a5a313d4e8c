"""GPU pins of the grouped GEMMs' activation epilogues, element by element.

With x_perm rows one-hot at column 0 and the weights nonzero only in column
0, every pre-activation the kernel sees is one exact bf16 weight value (one
exact product, exact fp32 sums of zeros), so each output is the activation of
a known number.  The values sweep [-12, 12], far tails included, and every
output must lie within one bf16 ulp of the oracle's activation of the same
number rounded to bf16 (the kernel rounds fp32 -> bf16, the oracle float64 ->
bf16; an fp32 activation accurate to a few ulps only moves a tie).  Rows
counts pick each kernel of the family: about 40 rows per expert run the
register-staged tiles, 150 the 128 x 256 ring, 300 the 256 x 256 split ring.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

import mixture_experts_layer_level_amd as moe  # noqa: E402

DEV = "cuda"
D = 64


def sweep(n, lo=-12.0, hi=12.0):
    """n distinct bf16 values over [lo, hi] (bits), including 0 and tiny ones."""
    v = np.linspace(lo, hi, n - 4)
    v = np.concatenate([v, [0.0, 1e-3, -1e-3, 2.0 ** -20]])
    return O.f64_to_bf16_bits(v)


def one_hot_rows(rows):
    x = np.zeros((rows, D), dtype=np.uint16)
    x[:, 0] = O.f64_to_bf16_bits(np.array([1.0]))[0]
    return x


def to_dev(bits):
    return torch.from_numpy(bits.view(np.int16).copy()).to(DEV).view(torch.bfloat16)


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def within_one_ulp(got_bits, ref, what):
    got = O.bf16_to_f64(got_bits)
    ref_b = O.bf16_to_f64(O.f64_to_bf16_bits(ref))
    # one bf16 ulp of the reference: 2^(e - 7) for |ref| in [2^e, 2^(e+1))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.abs(ref_b)))
    ulp = np.where(ref_b == 0, 0.0, np.exp2(e - 7))
    bad = np.abs(got - ref_b) > ulp
    assert not bad.any(), (f"{what}: {int(bad.sum())} outputs off by more than one bf16 ulp, "
                           f"first at ref {ref[bad][0]!r}, got {got[bad][0]!r}")


@pytest.mark.parametrize("rows", [40, 150, 300])
def test_gelu_epilogue_pin(rows):
    F = 2048
    vals = sweep(F)
    w1 = np.zeros((1, F, D), dtype=np.uint16)
    w1[0, :, 0] = vals
    p = moe.problem(rows, D, F, 1, 1, "softmax")
    offsets = torch.tensor([0, rows], dtype=torch.int32, device=DEV)
    h = torch.empty(rows, F, dtype=torch.bfloat16, device=DEV)
    b1 = torch.zeros(1, F, dtype=torch.float32, device=DEV)
    moe.expert_up_gelu(p, to_dev(one_hot_rows(rows)), offsets, to_dev(w1), b1, h)
    torch.cuda.synchronize()
    ref = O.gelu(O.bf16_to_f64(vals))
    got = host_bits(h)
    assert (got == got[0]).all(), "every row sees the same pre-activations"
    within_one_ulp(got[0], ref, f"GELU epilogue, {rows} rows")


@pytest.mark.parametrize("rows", [40, 150, 300])
def test_swiglu_epilogue_pin(rows):
    F = 1024
    g = sweep(F)
    rng = np.random.default_rng(rows)
    u = O.f64_to_bf16_bits(rng.choice([-3.0, -1.0, 0.5, 1.0, 2.5], F))
    wg = np.zeros((1, F, D), dtype=np.uint16)
    wu = np.zeros((1, F, D), dtype=np.uint16)
    wg[0, :, 0] = g
    wu[0, :, 0] = u
    p = moe.problem(rows, D, F, 1, 1, "softmax")
    offsets = torch.tensor([0, rows], dtype=torch.int32, device=DEV)
    h = torch.empty(rows, F, dtype=torch.bfloat16, device=DEV)
    moe.expert_gateup(p, to_dev(one_hot_rows(rows)), offsets, to_dev(wg), to_dev(wu), h)
    torch.cuda.synchronize()
    gf, uf = O.bf16_to_f64(g), O.bf16_to_f64(u)
    ref = O.silu(gf) * uf
    got = host_bits(h)
    assert (got == got[0]).all(), "every row sees the same pre-activations"
    within_one_ulp(got[0], ref, f"SwiGLU epilogue, {rows} rows")
