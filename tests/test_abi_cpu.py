"""The C-ABI library on the host: it loads, exports every declared entry
point, and rejects bad arguments before any HIP call (no GPU is touched:
every call here returns from the host-side checks)."""
import ctypes
import math
import os
import re
from fractions import Fraction

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
moe = pytest.importorskip("mixture_experts_layer_level_amd")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 0x7F0000000000          # 16-byte aligned address that is never dereferenced


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert "moe_forward" in names and len(names) >= 10
    for n in names:
        assert hasattr(moe.lib, n), n


def test_abi_version_and_status_strings():
    assert moe.abi_version() == 1
    assert moe.status_str(OK) == "ok"
    assert "workspace" in moe.status_str(WORKSPACE)


def P(N=64, D=256, F=512, E=8, K=2, g=0, cn=0, cd=1):
    return moe.MoEProblem(N, D, F, E, K, g, cn, cd)


def ws_status(p):
    n = ctypes.c_size_t()
    return moe.lib.moe_workspace_size(ctypes.byref(p), ctypes.byref(n))


@pytest.mark.parametrize("kw,status", [
    (dict(), OK),
    (dict(N=-1), INVALID), (dict(K=0), INVALID), (dict(K=9), INVALID), (dict(E=0), INVALID),
    (dict(g=2), INVALID), (dict(cn=5, cd=0), INVALID), (dict(cn=-1), INVALID),
    (dict(D=0), INVALID), (dict(F=-64), INVALID),
    (dict(D=100), UNSUPPORTED), (dict(F=96), UNSUPPORTED), (dict(E=2048, K=2), UNSUPPORTED),
    (dict(E=128, K=65), UNSUPPORTED), (dict(N=1 << 29, K=8), UNSUPPORTED),
])
def test_problem_validation(kw, status):
    assert ws_status(P(**kw)) == status


def test_null_problem():
    n = ctypes.c_size_t()
    assert moe.lib.moe_workspace_size(None, ctypes.byref(n)) == INVALID
    assert moe.lib.moe_workspace_size(ctypes.byref(P()), None) == INVALID


@pytest.mark.parametrize("N,K,E,cn,cd", [(16384, 2, 64, 5, 4), (8, 1, 3, 3, 2), (7, 3, 5, 5, 4),
                                         (64, 8, 128, 1, 1), (100, 2, 8, 0, 1)])
def test_permuted_rows(N, K, E, cn, cd):
    rows, cap = moe.permuted_rows(P(N=N, K=K, E=E, cn=cn, cd=cd))
    if cn == 0:
        assert (rows, cap) == (N * K, 0)
    else:
        c = math.ceil(Fraction(cn * N * K, cd * E))
        assert (rows, cap) == (E * c, c)


def test_workspace_covers_staged_buffers():
    """The forward's workspace holds the permuted rows (x_perm, and out_perm
    written over it once the gate/up GEMM has read it) and h; the routing
    scratch, the permutation's scratch and the fused launch's region share
    memory with those, so it is less than x_perm, out_perm and h apart."""
    p = P(N=4096, D=4096, F=14336, E=8, K=2)
    need = moe.workspace_size(p)
    S, D, F = 8192, 4096, 14336
    assert need >= S * D * 2 + S * F * 2
    assert need < 2 * S * D * 2 + S * F * 2


def _call_forward(p, ws_bytes, x=FAKE, y=FAKE, ws=FAKE):
    return moe.lib.moe_forward(ctypes.byref(p), x, FAKE, None, FAKE, FAKE, FAKE, y,
                               None, None, None, None, None, ws, ws_bytes, 0)


def test_forward_argument_errors():
    p = P()
    need = moe.workspace_size(p)
    assert _call_forward(p, need - 1) == WORKSPACE
    assert _call_forward(p, need, ws=None) == WORKSPACE
    assert _call_forward(p, need, x=None) == INVALID
    assert _call_forward(p, need, y=None) == INVALID
    assert _call_forward(p, need, x=FAKE + 2) == UNSUPPORTED
    assert _call_forward(p, need, ws=FAKE + 8) == UNSUPPORTED
    # N = 0 is a no-op: returns OK without touching (fake) memory
    assert _call_forward(P(N=0), 0, ws=None) == OK


def test_staged_argument_errors():
    p = P()
    L = moe.lib
    bp = ctypes.byref(p)
    # route: logits/ids/weights required; with x, w_router required
    assert L.moe_route(bp, FAKE, None, None, FAKE, FAKE, FAKE, None, 0, 0) == INVALID
    assert L.moe_route(bp, None, None, None, None, FAKE, FAKE, None, 0, 0) == INVALID
    assert L.moe_route(bp, FAKE + 4, FAKE, None, FAKE, FAKE, FAKE, None, 0, 0) == UNSUPPORTED
    # permute: workspace checked
    assert L.moe_permute(bp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 0) == WORKSPACE
    assert L.moe_permute(bp, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, 0) == INVALID
    assert L.moe_permute(bp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 2, FAKE, 1 << 20, 0) \
        == UNSUPPORTED                                                # misaligned x_perm
    # grouped FFN: workspace needed only without h
    assert L.moe_grouped_ffn(bp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, 0) == WORKSPACE
    assert L.moe_grouped_ffn(bp, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, 0, 0) == INVALID
    assert L.moe_expert_gateup(bp, FAKE, FAKE, FAKE, FAKE, None, 0) == INVALID
    assert L.moe_expert_down(bp, FAKE, FAKE, FAKE, FAKE + 2, 0) == UNSUPPORTED
    assert L.moe_unpermute_combine(bp, FAKE, FAKE, None, FAKE, 0) == INVALID
    # gathered gate/up: row_token required; refused for the padded layout, for
    # x of 4 GiB or more and for the register-staged tiles (<= 48 rows per
    # expert with D < 1024: P()'s 16 rows per expert, D = 256)
    big = ctypes.byref(P(N=4096))                     # 1024 rows per expert
    gg = L.moe_expert_gateup_gathered
    assert gg(big, FAKE, None, FAKE, FAKE, FAKE, FAKE, 0) == INVALID
    assert gg(big, FAKE + 2, FAKE, FAKE, FAKE, FAKE, FAKE, 0) == UNSUPPORTED
    assert gg(ctypes.byref(P(N=4096, cn=5, cd=4)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0) \
        == UNSUPPORTED
    assert gg(ctypes.byref(P(N=1 << 20, D=2048)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0) \
        == UNSUPPORTED                                                 # 4 GiB of x
    assert gg(bp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0) == UNSUPPORTED
    g8 = L.moe_expert_gateup_fp8_gathered
    assert g8(big, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0) == INVALID
    assert g8(big, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 0) == INVALID
    assert g8(ctypes.byref(P(N=4096, cn=5, cd=4)), *([FAKE] * 8), 0) == UNSUPPORTED
    assert g8(bp, *([FAKE] * 8), 0) == UNSUPPORTED                  # D = 256
    gl = L.moe_expert_up_gelu_gathered
    assert gl(big, FAKE, FAKE, FAKE, FAKE, None, FAKE, 0) == INVALID
    assert gl(ctypes.byref(P(N=4096, cn=5, cd=4)), *([FAKE] * 6), 0) == UNSUPPORTED
    assert gl(bp, *([FAKE] * 6), 0) == UNSUPPORTED
    # every entry point accepts N = 0 without launching
    z = ctypes.byref(P(N=0))
    assert L.moe_route(z, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, 0, 0) == OK
    assert L.moe_permute(z, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 0) == OK
    assert L.moe_grouped_ffn(z, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 0) == OK
    assert L.moe_expert_gateup(z, FAKE, FAKE, FAKE, FAKE, FAKE, 0) == OK
    assert L.moe_expert_gateup_gathered(z, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0) == OK
    assert L.moe_expert_gateup_fp8_gathered(z, *([FAKE] * 8), 0) == OK
    assert L.moe_expert_up_gelu_gathered(z, *([FAKE] * 6), 0) == OK
    assert L.moe_expert_down(z, FAKE, FAKE, FAKE, FAKE, 0) == OK
    assert L.moe_unpermute_combine(z, FAKE, FAKE, FAKE, FAKE, 0) == OK


def test_product_does_not_use_the_oracle():
    """The package and its library never reference the test oracle."""
    pkg = os.path.join(ROOT, "mixture_experts_layer_level_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "oracle" not in txt.lower(), f
                assert "moe_synth" not in txt, f


def test_routing_stats_argument_checks():
    f = moe.lib.moe_routing_stats
    assert f(0, FAKE, FAKE, FAKE, 0.9, 0.1, None) == INVALID
    assert f(8, None, FAKE, FAKE, 0.9, 0.1, None) == INVALID
    assert f(8, FAKE, FAKE, FAKE, 1.5, 0.1, None) == INVALID
    assert f(8, FAKE, FAKE, FAKE, float("nan"), 0.1, None) == INVALID
    assert f(8, FAKE, FAKE, FAKE, 0.9, float("nan"), None) == INVALID
    assert f(2048, FAKE, FAKE, FAKE, 0.9, 0.1, None) == UNSUPPORTED
    assert f(8, FAKE, FAKE, FAKE, 0.9, float("inf"), None) == INVALID


def test_fp8_argument_checks():
    L = moe.lib
    q = L.moe_quantize_fp8
    assert q(64, 128, None, FAKE, FAKE, None) == INVALID
    assert q(-32, 128, FAKE, FAKE, FAKE, None) == INVALID
    assert q(64, 0, FAKE, FAKE, FAKE, None) == INVALID
    assert q(48, 128, FAKE, FAKE, FAKE, None) == UNSUPPORTED      # rows not a multiple of 32
    assert q(64, 80, FAKE, FAKE, FAKE, None) == UNSUPPORTED       # cols not a multiple of 32
    assert q(64, 128, FAKE + 2, FAKE, FAKE, None) == UNSUPPORTED
    assert q(0, 128, FAKE, FAKE, FAKE, None) == OK                # nothing to do
    p = P()
    bp = ctypes.byref(p)
    g = L.moe_expert_gateup_fp8
    assert g(bp, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == INVALID
    assert g(bp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 8, FAKE, None) == UNSUPPORTED
    assert g(ctypes.byref(P(N=0)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == OK
    d = L.moe_expert_down_fp8
    assert d(bp, FAKE, FAKE, None, FAKE, FAKE, None) == INVALID
    assert d(bp, FAKE, FAKE, FAKE + 4, FAKE, FAKE, None) == UNSUPPORTED
    ffn = L.moe_grouped_ffn_fp8
    assert ffn(bp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) \
        == WORKSPACE
    assert ffn(bp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, 0, None) \
        == INVALID
    fw = L.moe_forward_fp8
    need = moe.workspace_size(p)
    args = [bp, FAKE, FAKE, None] + [FAKE] * 6 + [FAKE] + [None] * 5
    bad = list(args)
    bad[5] = None                                                 # gate scales missing
    assert fw(*bad, FAKE, need, None) == INVALID
    bad = list(args)
    bad[9] = FAKE + 1                                             # down scales misaligned
    assert fw(*bad, FAKE, need, None) == UNSUPPORTED
    assert fw(*args, FAKE, need - 1, None) == WORKSPACE
    assert fw(ctypes.byref(P(N=0)), *args[1:], None, 0, None) == OK


def test_packed_weight_argument_checks():
    L = moe.lib
    n = ctypes.c_size_t()
    # sizes: E * ceil(F / 128) * (D / 64) * 32 KB (gate/up), E * ceil(D / 256) * (F / 64) * 32 KB
    for D, F in ((256, 512), (320, 192), (7168, 2048)):
        bp = ctypes.byref(P(D=D, F=F))
        assert L.moe_packed_weight_size(bp, 0, ctypes.byref(n)) == OK
        assert n.value == 8 * math.ceil(F / 128) * (D // 64) * 32768
        assert L.moe_packed_weight_size(bp, 1, ctypes.byref(n)) == OK
        assert n.value == 8 * math.ceil(D / 256) * (F // 64) * 32768
    bp = ctypes.byref(P())
    assert L.moe_packed_weight_size(bp, 4, ctypes.byref(n)) == INVALID     # no such kind
    assert L.moe_packed_weight_size(bp, -1, ctypes.byref(n)) == INVALID
    assert L.moe_packed_weight_size(bp, 0, None) == INVALID
    assert L.moe_packed_weight_size(ctypes.byref(P(D=100)), 0, ctypes.byref(n)) == UNSUPPORTED
    pk = L.moe_pack_weights
    assert pk(bp, 2, FAKE, FAKE, FAKE, None) == INVALID          # FP8 kinds: moe_pack_weights_fp8
    assert pk(bp, 0, FAKE, None, FAKE, None) == INVALID          # gate/up needs both stacks
    assert pk(bp, 1, None, None, FAKE, None) == INVALID
    assert pk(bp, 1, FAKE, None, None, None) == INVALID
    assert pk(bp, 0, FAKE, FAKE + 2, FAKE, None) == UNSUPPORTED
    assert pk(bp, 1, FAKE, None, FAKE + 8, None) == UNSUPPORTED
    g = L.moe_expert_gateup_packed
    assert g(bp, FAKE, FAKE, None, FAKE, None) == INVALID
    assert g(bp, FAKE, FAKE, FAKE + 4, FAKE, None) == UNSUPPORTED
    assert g(ctypes.byref(P(N=0)), FAKE, FAKE, FAKE, FAKE, None) == OK
    gg = L.moe_expert_gateup_packed_gathered
    big = ctypes.byref(P(N=4096))
    assert gg(big, FAKE, None, FAKE, FAKE, FAKE, None) == INVALID
    assert gg(ctypes.byref(P(N=4096, cn=5, cd=4)), *([FAKE] * 5), None) == UNSUPPORTED
    assert gg(bp, *([FAKE] * 5), None) == UNSUPPORTED             # register-staged tiles
    assert gg(ctypes.byref(P(N=0)), *([FAKE] * 5), None) == OK
    d = L.moe_expert_down_packed
    assert d(bp, FAKE, None, FAKE, FAKE, None) == INVALID
    assert d(bp, FAKE, FAKE, FAKE, FAKE + 2, None) == UNSUPPORTED
    assert d(ctypes.byref(P(N=0)), FAKE, FAKE, FAKE, FAKE, None) == OK
    fw = L.moe_forward_packed
    need = moe.workspace_size(P())
    args = [bp, FAKE, FAKE, None, FAKE, FAKE, FAKE] + [None] * 5
    bad = list(args)
    bad[5] = None                                                 # down stack missing
    assert fw(*bad, FAKE, need, None) == INVALID
    bad = list(args)
    bad[4] = FAKE + 2                                             # gate/up stack misaligned
    assert fw(*bad, FAKE, need, None) == UNSUPPORTED
    assert fw(*args, FAKE, need - 1, None) == WORKSPACE
    assert fw(ctypes.byref(P(N=0)), *args[1:], None, 0, None) == OK


def test_packed_fp8_argument_checks():
    L = moe.lib
    n = ctypes.c_size_t()
    by = ctypes.byref
    # sizes: E * ceil(F / 128) * (D / 128) * 32 KB (gate/up), E * ceil(D / 256) * (F / 128) * 32 KB
    for D, F in ((256, 512), (384, 640), (7168, 2048)):
        bp = by(P(D=D, F=F))
        assert L.moe_packed_weight_size(bp, 2, by(n)) == OK
        assert n.value == 8 * math.ceil(F / 128) * (D // 128) * 32768
        assert L.moe_packed_weight_size(bp, 3, by(n)) == OK
        assert n.value == 8 * math.ceil(D / 256) * (F // 128) * 32768
    # the contraction length (D for gate/up, F for down) must be a multiple of 128
    odd = by(P(D=320, F=192))
    assert L.moe_packed_weight_size(odd, 2, by(n)) == UNSUPPORTED
    assert L.moe_packed_weight_size(odd, 3, by(n)) == UNSUPPORTED
    assert L.moe_packed_weight_size(by(P(D=320, F=256)), 3, by(n)) == OK
    bp = by(P())
    pk = L.moe_pack_weights_fp8
    assert pk(bp, 0, FAKE, FAKE, FAKE, None) == INVALID          # a bf16 kind
    assert pk(bp, 2, FAKE, None, FAKE, None) == INVALID          # gate/up needs both stacks
    assert pk(bp, 3, None, None, FAKE, None) == INVALID
    assert pk(bp, 3, FAKE, None, None, None) == INVALID
    assert pk(odd, 2, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    assert pk(bp, 2, FAKE, FAKE + 2, FAKE, None) == UNSUPPORTED
    g = L.moe_expert_gateup_fp8_packed       # p, x_perm, offsets, packed, gate scales, up scales, h
    assert g(bp, FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == INVALID
    assert g(bp, FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == INVALID
    assert g(odd, *([FAKE] * 6), None) == UNSUPPORTED
    assert g(bp, FAKE, FAKE, FAKE + 4, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    assert g(by(P(N=0)), *([FAKE] * 6), None) == OK
    gg = L.moe_expert_gateup_fp8_packed_gathered   # p, x, row_token, offsets, packed, gs, us, h
    assert gg(bp, FAKE, None, *([FAKE] * 5), None) == INVALID
    assert gg(by(P(cn=5, cd=4)), *([FAKE] * 7), None) == UNSUPPORTED    # padded layout
    assert gg(odd, *([FAKE] * 7), None) == UNSUPPORTED
    assert gg(by(P(N=0)), *([FAKE] * 7), None) == OK
    d = L.moe_expert_down_fp8_packed         # p, h, offsets, packed, down scales, out_perm
    assert d(bp, FAKE, FAKE, FAKE, None, FAKE, None) == INVALID
    assert d(by(P(F=192)), *([FAKE] * 5), None) == UNSUPPORTED
    assert d(by(P(N=0)), *([FAKE] * 5), None) == OK
    fw = L.moe_forward_fp8_packed
    need = moe.workspace_size(P())
    args = [bp, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE] + [None] * 5
    bad = list(args)
    bad[8] = None                                                 # down scales missing
    assert fw(*bad, FAKE, need, None) == INVALID
    p320 = P(D=320)
    assert fw(by(p320), *args[1:], FAKE, moe.workspace_size(p320), None) == UNSUPPORTED
    assert fw(*args, FAKE, need - 1, None) == WORKSPACE
    assert fw(by(P(N=0)), *args[1:], None, 0, None) == OK


def test_gelu_layer_argument_checks():
    L = moe.lib
    p = P(D=256)
    bp = ctypes.byref(p)
    need = moe.workspace_size(p)
    r = L.moe_route_mlp
    # x, w_proj, b_proj, w_out required; b_out optional
    assert r(bp, FAKE, None, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, need, None) == INVALID
    assert r(bp, FAKE, FAKE, None, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, need, None) == INVALID
    assert r(bp, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, need - 1, None) == WORKSPACE
    assert r(ctypes.byref(P(D=192)), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE,
             1 << 30, None) == UNSUPPORTED                              # D % 256 != 0
    assert r(bp, FAKE + 2, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, need, None) \
        == UNSUPPORTED
    assert r(ctypes.byref(P(N=0, D=256)), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE,
             None, 0, None) == OK
    u = L.moe_expert_up_gelu
    assert u(bp, FAKE, FAKE, FAKE, None, FAKE, None) == INVALID         # b1 required
    assert u(bp, FAKE, FAKE, FAKE, FAKE + 4, FAKE, None) == UNSUPPORTED
    d = L.moe_expert_down_bias
    assert d(bp, FAKE, FAKE, FAKE, None, FAKE, None) == INVALID
    f = L.moe_grouped_ffn_gelu
    assert f(bp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == WORKSPACE
    assert f(bp, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, 0, None) == INVALID
    fw = L.moe_forward_gelu
    args = [bp, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE] + [None] * 5
    assert fw(*args, FAKE, need - 1, None) == WORKSPACE
    bad = list(args)
    bad[9] = None                                                       # b2 missing
    assert fw(*bad, FAKE, need, None) == INVALID
    bad = list(args)
    bad[7] = FAKE + 8                                                   # b1 misaligned
    assert fw(*bad, FAKE, need, None) == UNSUPPORTED
    args192 = [ctypes.byref(P(D=192))] + args[1:]
    assert fw(*args192, FAKE, 1 << 30, None) == UNSUPPORTED             # D % 256 != 0
    assert fw(ctypes.byref(P(N=0, D=256)), *args[1:], None, 0, None) == OK


def test_fused_argument_checks():
    L = moe.lib
    p = P()
    bp = ctypes.byref(p)
    need = moe.workspace_size(p)
    f = L.moe_fused_ffn
    assert f(bp, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == INVALID
    assert f(bp, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == WORKSPACE
    assert f(ctypes.byref(P(cn=5, cd=4)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need,
             None) == UNSUPPORTED                                     # padded layout
    assert f(bp, FAKE + 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == UNSUPPORTED
    assert f(ctypes.byref(P(N=0)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == OK
    fw = L.moe_forward_fused
    args = [bp, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE] + [None] * 5
    assert fw(*args, FAKE, need - 1, None) == WORKSPACE
    assert fw(*([bp, FAKE, None] + args[3:]), FAKE, need, None) == INVALID   # no router weights
    assert fw(*([ctypes.byref(P(cn=5, cd=4))] + args[1:]), FAKE, 1 << 30, None) == UNSUPPORTED
    assert fw(*([ctypes.byref(P(N=1 << 20, D=4096))] + args[1:]), FAKE, 1 << 62, None) \
        == UNSUPPORTED                                                # x of 8 GiB
    assert fw(*([ctypes.byref(P(N=0))] + args[1:]), None, 0, None) == OK
    n = ctypes.c_size_t()
    assert L.moe_fused_error_offset(bp, 0, ctypes.byref(n)) == OK
    n1 = ctypes.c_size_t()
    assert L.moe_fused_error_offset(bp, 1, ctypes.byref(n1)) == OK
    assert n.value % 4 == 0 and n1.value > n.value and n1.value + 4 <= need
    assert L.moe_fused_error_offset(bp, 0, None) == INVALID



def forward_static_status(p, x=FAKE, w=FAKE, y=FAKE):
    return moe.lib.moe_forward_static(ctypes.byref(p), x, w, None, w, w, w, y, None, None, None,
                                      None, None, None)


def test_forward_static_host_checks():
    """moe_forward_static: the problem, the pointers and the scratch size are
    checked on the host; a problem whose workspace exceeds the static scratch
    is refused before any HIP call (nothing here touches a GPU)."""
    assert moe.STATIC_SCRATCH_BYTES == 64 << 20
    assert forward_static_status(P(K=0)) == INVALID
    assert forward_static_status(P(D=100)) == UNSUPPORTED
    assert forward_static_status(P(), x=None) == INVALID
    assert forward_static_status(P(), y=None) == INVALID
    assert forward_static_status(P(N=0)) == OK
    big = P(N=8192, D=7168, F=2048, E=256, K=8, g=1)      # a DeepSeek-V3-shape prefill batch
    assert moe.workspace_size(big) > moe.STATIC_SCRATCH_BYTES
    assert forward_static_status(big) == WORKSPACE
    dec = P(N=64, D=2048, F=768, E=128, K=8)               # a Qwen3-30B-A3B-shape decode step
    assert moe.workspace_size(dec) <= moe.STATIC_SCRATCH_BYTES
