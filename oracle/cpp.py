"""ctypes binding of the C++ oracle (oracle/liboracle.so, built by oracle/build.py).

TEST INFRASTRUCTURE, like the numpy oracle: only the test suite, the smoke
check and the benchmark's CPU-baseline leg may use it.  The functions take
and return numpy arrays with the names and conventions of
``oracle.moe_oracle`` (bf16 tensors as raw uint16 bit patterns on input; h,
out_perm and y returned as float64 arrays holding bf16 values), so the same
pins can be run against both oracles.  The arithmetic is all in the C++
source; this module only marshals arguments.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

_lib = None


def lib():
    """The loaded C++ oracle; builds it first if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = ctypes.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


P = ctypes.c_void_p
I64, I32 = ctypes.c_int64, ctypes.c_int


def _declare(L):
    L.oracle_version.restype = I32
    L.oracle_threads.restype = I32
    L.oracle_capacity.argtypes = [I64, I32, I32, I64, I64]
    L.oracle_capacity.restype = I64
    L.oracle_router_logits.argtypes = [I64, I32, I32, P, P, P]
    L.oracle_route.argtypes = [I64, I32, I32, I32, P, P, P, P]
    L.oracle_permute.argtypes = [I64, I32, I32, I64, P, P, P, P, P]
    L.oracle_ffn_rows.argtypes = [I64, P, P, P, I32, I32, I32, P, P, P, P, P]
    L.oracle_expert_ffn.argtypes = [I64, I32, I32, I32, P, P, P, P, P, P, P]
    L.oracle_combine.argtypes = [I64, I32, I32, P, P, P, P]
    L.oracle_forward.argtypes = [I64, I32, I32, I32, I32, I32, I64, P, P, P, P, P, P, I32,
                                 P, P, P, P, P, P, P, P, P, P]
    L.oracle_quantize_fp8.argtypes = [I64, I32, P, P, P]
    L.oracle_dequantize_fp8.argtypes = [I64, I32, P, P, P]
    for f in ("oracle_quantize_fp8", "oracle_dequantize_fp8", "oracle_router_logits", "oracle_route", "oracle_permute", "oracle_ffn_rows",
              "oracle_expert_ffn", "oracle_combine", "oracle_forward"):
        getattr(L, f).restype = None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a):
    return None if a is None else a.ctypes.data_as(P)


def _gating(g) -> int:
    return {"softmax": 0, "sigmoid": 1}[g] if isinstance(g, str) else int(g)


def _bf16_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def threads() -> int:
    return int(lib().oracle_threads())


def capacity(N: int, K: int, E: int, num: int, den: int) -> int:
    return int(lib().oracle_capacity(N, K, E, num, den))


def quantize_fp8(w_bits):
    """bf16 weights [..., cols] -> (codes uint8 [..., cols], scales uint8 [..., cols/32])."""
    w = _c(w_bits, np.uint16)
    cols = w.shape[-1]
    rows = w.size // cols
    codes = np.empty(w.shape, dtype=np.uint8)
    scales = np.empty(w.shape[:-1] + (cols // 32,), dtype=np.uint8)
    lib().oracle_quantize_fp8(rows, cols, _p(w), _p(codes), _p(scales))
    return codes, scales


def dequantize_fp8_bits(codes, scales):
    """(codes, scales) -> bf16 bit patterns of the dequantised weights."""
    c = _c(codes, np.uint8)
    s = _c(scales, np.uint8)
    cols = c.shape[-1]
    out = np.empty(c.shape, dtype=np.uint16)
    lib().oracle_dequantize_fp8(c.size // cols, cols, _p(c), _p(s), _p(out))
    return out


def router_logits(x_bits, w_router):
    x = _c(x_bits, np.uint16)
    w = _c(w_router, np.float32)
    N, D = x.shape
    E = w.shape[0]
    out = np.empty((N, E), dtype=np.float32)
    lib().oracle_router_logits(N, D, E, _p(x), _p(w), _p(out))
    return out


def route_from_logits(logits, bias, K: int, gating):
    lg = _c(logits, np.float32)
    N, E = lg.shape
    b = None if bias is None else _c(bias, np.float32)
    ids = np.empty((N, K), dtype=np.int32)
    w = np.empty((N, K), dtype=np.float32)
    lib().oracle_route(N, E, K, _gating(gating), _p(lg), _p(b), _p(ids), _p(w))
    return ids, w


def route(x_bits, w_router, bias, K: int, gating):
    logits = router_logits(x_bits, w_router)
    ids, w = route_from_logits(logits, bias, K, gating)
    return logits, ids, w


def permute(topk_ids, E: int, cap=None):
    ids = _c(topk_ids, np.int32)
    N, K = ids.shape
    R = N * K if cap is None else E * cap
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    row_token = np.empty(R, dtype=np.int32)
    slot_row = np.empty(N * K, dtype=np.int32)
    lib().oracle_permute(N, K, E, 0 if cap is None else int(cap), _p(ids), _p(counts),
                         _p(offsets), _p(row_token), _p(slot_row))
    return counts, offsets, row_token, slot_row


def ffn_rows(row_expert, row_token, x_bits, w_gate_bits, w_up_bits, w_down_bits,
             want_h: bool = True):
    """FFN of given rows: row i is x[row_token[i]] run through expert
    row_expert[i] (row_token < 0: a zero row).  Returns (h, out) as float64
    arrays of bf16 values (h None unless want_h)."""
    re = _c(row_expert, np.int32)
    rt = _c(row_token, np.int32)
    x = _c(x_bits, np.uint16)
    wg, wu, wd = (_c(w, np.uint16) for w in (w_gate_bits, w_up_bits, w_down_bits))
    E, F, D = wg.shape
    n = re.shape[0]
    h = np.empty((n, F), dtype=np.uint16) if want_h else None
    out = np.empty((n, D), dtype=np.uint16)
    lib().oracle_ffn_rows(n, _p(re), _p(rt), _p(x), D, F, E, _p(wg), _p(wu), _p(wd), _p(h),
                          _p(out))
    return (None if h is None else _bf16_f64(h)), _bf16_f64(out)


def expert_ffn(x_perm_bits, offsets, w_gate_bits, w_up_bits, w_down_bits):
    xp = _c(x_perm_bits, np.uint16)
    off = _c(offsets, np.int32)
    wg, wu, wd = (_c(w, np.uint16) for w in (w_gate_bits, w_up_bits, w_down_bits))
    E, F, D = wg.shape
    R = xp.shape[0]
    h = np.zeros((R, F), dtype=np.uint16)
    out = np.zeros((R, D), dtype=np.uint16)
    lib().oracle_expert_ffn(R, D, F, E, _p(xp), _p(off), _p(wg), _p(wu), _p(wd), _p(h), _p(out))
    return _bf16_f64(h), _bf16_f64(out)


def combine(out_perm, slot_row, topk_w):
    """out_perm as float64 values of bf16 numbers (as the numpy oracle takes it)."""
    op = np.asarray(out_perm, dtype=np.float64).astype(np.float32)   # exact: bf16 values
    opb = _c((op.view(np.uint32) >> np.uint32(16)).astype(np.uint16), np.uint16)
    w = _c(topk_w, np.float32)
    N, K = w.shape
    D = opb.shape[1]
    sr = _c(slot_row, np.int32)
    y = np.empty((N, D), dtype=np.uint16)
    lib().oracle_combine(N, K, D, _p(opb), _p(sr), _p(w), _p(y))
    return _bf16_f64(y)


def forward(x_bits, w_router, bias, w_gate_bits, w_up_bits, w_down_bits, K: int, gating,
            cap=None, logits=None, want_h: bool = True) -> dict:
    """The whole layer (as oracle.moe_oracle.forward; x_perm is not built)."""
    x = _c(x_bits, np.uint16)
    wr = _c(w_router, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    wg, wu, wd = (_c(w, np.uint16) for w in (w_gate_bits, w_up_bits, w_down_bits))
    N, D = x.shape
    E, F = wr.shape[0], wg.shape[1]
    R = N * K if cap is None else E * cap
    lg = np.empty((N, E), dtype=np.float32) if logits is None else _c(logits, np.float32)
    ids = np.empty((N, K), dtype=np.int32)
    w = np.empty((N, K), dtype=np.float32)
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    row_token = np.empty(R, dtype=np.int32)
    slot_row = np.empty(N * K, dtype=np.int32)
    h = np.zeros((R, F), dtype=np.uint16) if want_h else None
    out = np.zeros((R, D), dtype=np.uint16)
    y = np.empty((N, D), dtype=np.uint16)
    lib().oracle_forward(N, D, E, K, F, _gating(gating), 0 if cap is None else int(cap), _p(x),
                         _p(wr), _p(b), _p(wg), _p(wu), _p(wd), 0 if logits is None else 1,
                         _p(lg), _p(ids), _p(w), _p(counts), _p(offsets), _p(row_token),
                         _p(slot_row), _p(h), _p(out), _p(y))
    return dict(logits=lg, topk_ids=ids, topk_weights=w, expert_counts=counts,
                expert_offsets=offsets, row_token=row_token, slot_row=slot_row,
                h=None if h is None else _bf16_f64(h), out_perm=_bf16_f64(out),
                y=_bf16_f64(y))
