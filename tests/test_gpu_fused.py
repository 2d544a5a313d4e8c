"""GPU parity of the fused FFN (one persistent launch, rows gathered from x):
against the oracle's expert FFN to the FFN bar, and bit for bit against the
staged grouped GEMMs, whose k order and tiles it shares; its error word (a
bounded wait that ran out) stays zero."""
import numpy as np
import pytest
import torch

import moe_synth as ms
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

from gpu_layer import (DEV, SMALL, Layer, assert_fp_close, bits, check_permutation,  # noqa: E402
                       np_, sample_tokens, check_sampled_outputs)
import mixture_experts_layer_level_amd as moe  # noqa: E402

CONTIGUOUS = [n for n, c in SMALL.items() if c.capacity is None]


def error_word(L, whole_layer):
    off = moe.fused_error_offset(L.p, whole_layer)
    return int(L.ws[off:off + 4].view(torch.int32).item())


@pytest.mark.parametrize("name", CONTIGUOUS)
def test_fused_ffn_small(name):
    cfg = SMALL[name]
    print(f"[fused] {name} N={cfg.N} D={cfg.D} E={cfg.E} K={cfg.K} F={cfg.F}", flush=True)
    L = Layer(cfg)
    L.staged()
    offsets, row_token, slot_row = check_permutation(L)
    out = torch.empty_like(L.out_perm)
    moe.fused_ffn(L.p, L.x, L.row_token, L.offsets, L.w_gate, L.w_up, L.w_down, out, L.ws)
    torch.cuda.synchronize()
    assert error_word(L, False) == 0
    covered = np.zeros(L.R, dtype=bool)
    for e in range(cfg.E):
        covered[offsets[e]:offsets[e + 1]] = True
    _, out_ref = O.expert_ffn(O.gather_rows(bits(L.x), row_token), offsets, bits(L.w_gate),
                              bits(L.w_up), bits(L.w_down))
    assert_fp_close(O.bf16_to_f64(bits(out))[covered], out_ref[covered], "out_perm (fused)")
    assert np.array_equal(bits(out)[covered], bits(L.out_perm)[covered]), "fused vs staged"
    y = torch.empty_like(L.y)
    moe.forward_fused(L.p, L.x, L.w_router, L.bias, L.w_gate, L.w_up, L.w_down, y, L.ws)
    torch.cuda.synchronize()
    assert error_word(L, True) == 0
    assert torch.equal(y.view(torch.int16), L.y.view(torch.int16)), "forward_fused vs staged"
