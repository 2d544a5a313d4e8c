"""ctypes binding of libmoe (include/moe.h): argument marshalling only."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(HERE, "libmoe.so")

MOE_OK = 0
GATING_SOFTMAX_TOPK = 0
GATING_SIGMOID_RENORM = 1

_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape or alignment",
           3: "workspace missing or too small", 4: "HIP launch failed"}


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str = ""):
        msg = f"{fn}: status {status} ({_STATUS.get(status, 'unknown')})"
        super().__init__(msg + (f": {detail}" if detail else ""))
        self.status = status


class MoEProblem(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int64), ("hidden", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("gating", ctypes.c_int32),
                ("capacity_num", ctypes.c_int32), ("capacity_den", ctypes.c_int32)]


def _load():
    # torch first: its bundled HIP runtime (soname libamdhip64.so.7) is then the
    # one libmoe binds to, so both share one runtime, one device context and
    # the same streams.  Loading libmoe first would pull in a second runtime.
    import torch  # noqa: F401
    if not os.path.exists(library_path):
        raise ImportError(f"{library_path} is not built; run __graft_entry__.build() "
                          f"(hipcc for gfx950) first")
    L = ctypes.CDLL(library_path)
    P = ctypes.POINTER(MoEProblem)
    vp = ctypes.c_void_p
    sz = ctypes.c_size_t
    L.moe_abi_version.restype = ctypes.c_int
    L.moe_abi_version.argtypes = []
    L.moe_status_str.restype = ctypes.c_char_p
    L.moe_status_str.argtypes = [ctypes.c_int]
    L.moe_last_hip_error.restype = ctypes.c_char_p
    L.moe_last_hip_error.argtypes = []
    L.moe_permuted_rows.restype = ctypes.c_int
    L.moe_permuted_rows.argtypes = [P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
    L.moe_workspace_size.restype = ctypes.c_int
    L.moe_workspace_size.argtypes = [P, ctypes.POINTER(sz)]
    L.moe_route.restype = ctypes.c_int
    L.moe_route.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_permute.restype = ctypes.c_int
    L.moe_permute.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_routing_stats.restype = ctypes.c_int
    L.moe_routing_stats.argtypes = [ctypes.c_int32, vp, vp, vp, ctypes.c_float, ctypes.c_float, vp]
    L.moe_grouped_ffn.restype = ctypes.c_int
    L.moe_grouped_ffn.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_expert_gateup.restype = ctypes.c_int
    L.moe_expert_gateup.argtypes = [P, vp, vp, vp, vp, vp, vp]
    L.moe_expert_gateup_gathered.restype = ctypes.c_int
    L.moe_expert_gateup_gathered.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    L.moe_expert_down.restype = ctypes.c_int
    L.moe_expert_down.argtypes = [P, vp, vp, vp, vp, vp]
    L.moe_unpermute_combine.restype = ctypes.c_int
    L.moe_unpermute_combine.argtypes = [P, vp, vp, vp, vp, vp]
    L.moe_forward.restype = ctypes.c_int
    L.moe_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_forward_static.restype = ctypes.c_int
    L.moe_forward_static.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_fused_ffn.restype = ctypes.c_int
    L.moe_fused_ffn.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_forward_fused.restype = ctypes.c_int
    L.moe_forward_fused.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_fused_error_offset.restype = ctypes.c_int
    L.moe_fused_error_offset.argtypes = [P, ctypes.c_int32, ctypes.POINTER(sz)]
    L.moe_route_mlp.restype = ctypes.c_int
    L.moe_route_mlp.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_expert_up_gelu_gathered.restype = ctypes.c_int
    L.moe_expert_up_gelu_gathered.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    L.moe_expert_up_gelu.restype = ctypes.c_int
    L.moe_expert_up_gelu.argtypes = [P, vp, vp, vp, vp, vp, vp]
    L.moe_expert_down_bias.restype = ctypes.c_int
    L.moe_expert_down_bias.argtypes = [P, vp, vp, vp, vp, vp, vp]
    L.moe_grouped_ffn_gelu.restype = ctypes.c_int
    L.moe_grouped_ffn_gelu.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_forward_gelu.restype = ctypes.c_int
    L.moe_forward_gelu.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                   vp, vp, sz, vp]
    L.moe_quantize_fp8.restype = ctypes.c_int
    L.moe_quantize_fp8.argtypes = [ctypes.c_int64, ctypes.c_int32, vp, vp, vp, vp]
    L.moe_expert_gateup_fp8.restype = ctypes.c_int
    L.moe_expert_gateup_fp8.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_expert_gateup_fp8_gathered.restype = ctypes.c_int
    L.moe_expert_gateup_fp8_gathered.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_expert_down_fp8.restype = ctypes.c_int
    L.moe_expert_down_fp8.argtypes = [P, vp, vp, vp, vp, vp, vp]
    L.moe_grouped_ffn_fp8.restype = ctypes.c_int
    L.moe_grouped_ffn_fp8.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_forward_fp8.restype = ctypes.c_int
    L.moe_forward_fp8.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                  vp, sz, vp]
    L.moe_packed_weight_size.restype = ctypes.c_int
    L.moe_packed_weight_size.argtypes = [P, ctypes.c_int32, ctypes.POINTER(sz)]
    L.moe_pack_weights.restype = ctypes.c_int
    L.moe_pack_weights.argtypes = [P, ctypes.c_int32, vp, vp, vp, vp]
    L.moe_expert_gateup_packed.restype = ctypes.c_int
    L.moe_expert_gateup_packed.argtypes = [P, vp, vp, vp, vp, vp]
    L.moe_expert_gateup_packed_gathered.restype = ctypes.c_int
    L.moe_expert_gateup_packed_gathered.argtypes = [P, vp, vp, vp, vp, vp, vp]
    L.moe_expert_down_packed.restype = ctypes.c_int
    L.moe_expert_down_packed.argtypes = [P, vp, vp, vp, vp, vp]
    L.moe_forward_packed.restype = ctypes.c_int
    L.moe_forward_packed.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_pack_weights_fp8.restype = ctypes.c_int
    L.moe_pack_weights_fp8.argtypes = [P, ctypes.c_int32, vp, vp, vp, vp]
    L.moe_expert_gateup_fp8_packed.restype = ctypes.c_int
    L.moe_expert_gateup_fp8_packed.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    L.moe_expert_gateup_fp8_packed_gathered.restype = ctypes.c_int
    L.moe_expert_gateup_fp8_packed_gathered.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_expert_down_fp8_packed.restype = ctypes.c_int
    L.moe_expert_down_fp8_packed.argtypes = [P, vp, vp, vp, vp, vp, vp]
    L.moe_forward_fp8_packed.restype = ctypes.c_int
    L.moe_forward_fp8_packed.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         vp, vp, sz, vp]
    return L


lib = _load()


def abi_version() -> int:
    return lib.moe_abi_version()


def status_str(s: int) -> str:
    return lib.moe_status_str(s).decode()


def problem(N: int, D: int, F: int, E: int, K: int, gating="softmax",
            capacity: Optional[tuple] = None) -> MoEProblem:
    g = {"softmax": GATING_SOFTMAX_TOPK, "sigmoid": GATING_SIGMOID_RENORM}.get(gating, gating)
    num, den = capacity if capacity else (0, 1)
    return MoEProblem(N, D, F, E, K, g, num, den)


def _ptr(t):
    """Device address of a tensor (or an int address, or None for NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t) -> int:
    if t is None or isinstance(t, int):
        return 0
    return t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, st: int):
    if st != MOE_OK:
        detail = lib.moe_last_hip_error().decode() if st == 4 else ""
        raise MoEError(fn, st, detail)


def permuted_rows(p: MoEProblem):
    rows = ctypes.c_int64()
    cap = ctypes.c_int64()
    _check("moe_permuted_rows", lib.moe_permuted_rows(ctypes.byref(p), ctypes.byref(rows),
                                                      ctypes.byref(cap)))
    return rows.value, cap.value


def workspace_size(p: MoEProblem) -> int:
    n = ctypes.c_size_t()
    _check("moe_workspace_size", lib.moe_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def route(p, x, w_router, bias, logits, topk_ids, topk_weights, ws=None, stream=None):
    _check("moe_route", lib.moe_route(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(bias),
                                      _ptr(logits), _ptr(topk_ids), _ptr(topk_weights),
                                      _ptr(ws), _nbytes(ws), _stream(stream)))


def permute(p, x, topk_ids, counts, offsets, row_token, slot_row, x_perm, ws, stream=None):
    _check("moe_permute", lib.moe_permute(ctypes.byref(p), _ptr(x), _ptr(topk_ids), _ptr(counts),
                                          _ptr(offsets), _ptr(row_token), _ptr(slot_row),
                                          _ptr(x_perm), _ptr(ws), _nbytes(ws), _stream(stream)))


def grouped_ffn(p, x_perm, offsets, w_gate, w_up, w_down, out_perm, h, ws, stream=None):
    _check("moe_grouped_ffn", lib.moe_grouped_ffn(ctypes.byref(p), _ptr(x_perm), _ptr(offsets),
                                                  _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                                  _ptr(out_perm), _ptr(h), _ptr(ws), _nbytes(ws),
                                                  _stream(stream)))


def expert_gateup(p, x_perm, offsets, w_gate, w_up, h, stream=None):
    _check("moe_expert_gateup", lib.moe_expert_gateup(ctypes.byref(p), _ptr(x_perm), _ptr(offsets),
                                                      _ptr(w_gate), _ptr(w_up), _ptr(h),
                                                      _stream(stream)))


def expert_gateup_gathered(p, x, row_token, offsets, w_gate, w_up, h, stream=None):
    _check("moe_expert_gateup_gathered",
           lib.moe_expert_gateup_gathered(ctypes.byref(p), _ptr(x), _ptr(row_token), _ptr(offsets),
                                          _ptr(w_gate), _ptr(w_up), _ptr(h), _stream(stream)))


def expert_down(p, h, offsets, w_down, out_perm, stream=None):
    _check("moe_expert_down", lib.moe_expert_down(ctypes.byref(p), _ptr(h), _ptr(offsets),
                                                  _ptr(w_down), _ptr(out_perm), _stream(stream)))


def unpermute_combine(p, out_perm, slot_row, topk_weights, y, stream=None):
    _check("moe_unpermute_combine",
           lib.moe_unpermute_combine(ctypes.byref(p), _ptr(out_perm), _ptr(slot_row),
                                     _ptr(topk_weights), _ptr(y), _stream(stream)))


def forward(p, x, w_router, bias, w_gate, w_up, w_down, y, ws, logits=None, topk_ids=None,
            topk_weights=None, counts=None, offsets=None, stream=None):
    _check("moe_forward", lib.moe_forward(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(bias),
                                          _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(y),
                                          _ptr(logits), _ptr(topk_ids), _ptr(topk_weights),
                                          _ptr(counts), _ptr(offsets), _ptr(ws), _nbytes(ws),
                                          _stream(stream)))


STATIC_SCRATCH_BYTES = 64 << 20     # MOE_STATIC_SCRATCH_BYTES


def forward_static(p, x, w_router, bias, w_gate, w_up, w_down, y, logits=None, topk_ids=None,
                   topk_weights=None, counts=None, offsets=None, stream=None):
    """moe_forward_static: moe_forward with the library's static scratch (no workspace)."""
    _check("moe_forward_static",
           lib.moe_forward_static(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(bias),
                                  _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(y), _ptr(logits),
                                  _ptr(topk_ids), _ptr(topk_weights), _ptr(counts),
                                  _ptr(offsets), _stream(stream)))


def routing_stats(num_experts, expert_counts, ema, expert_bias, decay=0.99, step=0.1, stream=None):
    _check("moe_routing_stats", lib.moe_routing_stats(int(num_experts), _ptr(expert_counts),
                                                      _ptr(ema), _ptr(expert_bias), float(decay),
                                                      float(step), _stream(stream)))


# Block-scaled FP8 weights: each weight argument below is a (codes, scales)
# pair as written by quantize_fp8.

def quantize_fp8(rows, cols, w, codes, scales, stream=None):
    _check("moe_quantize_fp8", lib.moe_quantize_fp8(int(rows), int(cols), _ptr(w), _ptr(codes),
                                                    _ptr(scales), _stream(stream)))


def expert_gateup_fp8(p, x_perm, offsets, w_gate, w_up, h, stream=None):
    _check("moe_expert_gateup_fp8",
           lib.moe_expert_gateup_fp8(ctypes.byref(p), _ptr(x_perm), _ptr(offsets), _ptr(w_gate[0]),
                                     _ptr(w_gate[1]), _ptr(w_up[0]), _ptr(w_up[1]), _ptr(h),
                                     _stream(stream)))


def expert_gateup_fp8_gathered(p, x, row_token, offsets, w_gate, w_up, h, stream=None):
    _check("moe_expert_gateup_fp8_gathered",
           lib.moe_expert_gateup_fp8_gathered(ctypes.byref(p), _ptr(x), _ptr(row_token),
                                              _ptr(offsets), _ptr(w_gate[0]), _ptr(w_gate[1]),
                                              _ptr(w_up[0]), _ptr(w_up[1]), _ptr(h),
                                              _stream(stream)))


def expert_down_fp8(p, h, offsets, w_down, out_perm, stream=None):
    _check("moe_expert_down_fp8",
           lib.moe_expert_down_fp8(ctypes.byref(p), _ptr(h), _ptr(offsets), _ptr(w_down[0]),
                                   _ptr(w_down[1]), _ptr(out_perm), _stream(stream)))


def grouped_ffn_fp8(p, x_perm, offsets, w_gate, w_up, w_down, out_perm, h, ws, stream=None):
    _check("moe_grouped_ffn_fp8",
           lib.moe_grouped_ffn_fp8(ctypes.byref(p), _ptr(x_perm), _ptr(offsets), _ptr(w_gate[0]),
                                   _ptr(w_gate[1]), _ptr(w_up[0]), _ptr(w_up[1]), _ptr(w_down[0]),
                                   _ptr(w_down[1]), _ptr(out_perm), _ptr(h), _ptr(ws),
                                   _nbytes(ws), _stream(stream)))


def forward_fp8(p, x, w_router, bias, w_gate, w_up, w_down, y, ws, logits=None, topk_ids=None,
                topk_weights=None, counts=None, offsets=None, stream=None):
    _check("moe_forward_fp8",
           lib.moe_forward_fp8(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(bias),
                               _ptr(w_gate[0]), _ptr(w_gate[1]), _ptr(w_up[0]), _ptr(w_up[1]),
                               _ptr(w_down[0]), _ptr(w_down[1]), _ptr(y), _ptr(logits),
                               _ptr(topk_ids), _ptr(topk_weights), _ptr(counts), _ptr(offsets),
                               _ptr(ws), _nbytes(ws), _stream(stream)))


# Packed bf16 weights (moe_pack_weights): the same values in the kernels'
# stage-image order; kind PACK_GATEUP (gate and up) or PACK_DOWN.

PACK_GATEUP, PACK_DOWN, PACK_GATEUP_FP8, PACK_DOWN_FP8 = 0, 1, 2, 3   # moe_pack_kind


def packed_weight_size(p, kind) -> int:
    n = ctypes.c_size_t()
    _check("moe_packed_weight_size",
           lib.moe_packed_weight_size(ctypes.byref(p), int(kind), ctypes.byref(n)))
    return n.value


def pack_weights(p, kind, w0, w1, packed, stream=None):
    _check("moe_pack_weights", lib.moe_pack_weights(ctypes.byref(p), int(kind), _ptr(w0), _ptr(w1),
                                                    _ptr(packed), _stream(stream)))


def expert_gateup_packed(p, x_perm, offsets, w_gateup, h, stream=None):
    _check("moe_expert_gateup_packed",
           lib.moe_expert_gateup_packed(ctypes.byref(p), _ptr(x_perm), _ptr(offsets),
                                        _ptr(w_gateup), _ptr(h), _stream(stream)))


def expert_gateup_packed_gathered(p, x, row_token, offsets, w_gateup, h, stream=None):
    _check("moe_expert_gateup_packed_gathered",
           lib.moe_expert_gateup_packed_gathered(ctypes.byref(p), _ptr(x), _ptr(row_token),
                                                 _ptr(offsets), _ptr(w_gateup), _ptr(h),
                                                 _stream(stream)))


def expert_down_packed(p, h, offsets, w_down, out_perm, stream=None):
    _check("moe_expert_down_packed",
           lib.moe_expert_down_packed(ctypes.byref(p), _ptr(h), _ptr(offsets), _ptr(w_down),
                                      _ptr(out_perm), _stream(stream)))


def forward_packed(p, x, w_router, bias, w_gateup, w_down, y, ws, logits=None, topk_ids=None,
                   topk_weights=None, counts=None, offsets=None, stream=None):
    _check("moe_forward_packed",
           lib.moe_forward_packed(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(bias),
                                  _ptr(w_gateup), _ptr(w_down), _ptr(y), _ptr(logits),
                                  _ptr(topk_ids), _ptr(topk_weights), _ptr(counts),
                                  _ptr(offsets), _ptr(ws), _nbytes(ws), _stream(stream)))


# Packed FP8 codes (moe_pack_weights_fp8): the codes of an FP8 stack in the
# same stage-image order, 128 codes deep; the scales stay as quantize_fp8
# wrote them and are passed beside the packed codes.

def pack_weights_fp8(p, kind, c0, c1, packed, stream=None):
    _check("moe_pack_weights_fp8",
           lib.moe_pack_weights_fp8(ctypes.byref(p), int(kind), _ptr(c0), _ptr(c1), _ptr(packed),
                                    _stream(stream)))


def expert_gateup_fp8_packed(p, x_perm, offsets, w_gateup, gate_scales, up_scales, h,
                             stream=None):
    _check("moe_expert_gateup_fp8_packed",
           lib.moe_expert_gateup_fp8_packed(ctypes.byref(p), _ptr(x_perm), _ptr(offsets),
                                            _ptr(w_gateup), _ptr(gate_scales), _ptr(up_scales),
                                            _ptr(h), _stream(stream)))


def expert_gateup_fp8_packed_gathered(p, x, row_token, offsets, w_gateup, gate_scales,
                                      up_scales, h, stream=None):
    _check("moe_expert_gateup_fp8_packed_gathered",
           lib.moe_expert_gateup_fp8_packed_gathered(ctypes.byref(p), _ptr(x), _ptr(row_token),
                                                     _ptr(offsets), _ptr(w_gateup),
                                                     _ptr(gate_scales), _ptr(up_scales), _ptr(h),
                                                     _stream(stream)))


def expert_down_fp8_packed(p, h, offsets, w_down, down_scales, out_perm, stream=None):
    _check("moe_expert_down_fp8_packed",
           lib.moe_expert_down_fp8_packed(ctypes.byref(p), _ptr(h), _ptr(offsets), _ptr(w_down),
                                          _ptr(down_scales), _ptr(out_perm), _stream(stream)))


def forward_fp8_packed(p, x, w_router, bias, w_gateup, gate_scales, up_scales, w_down,
                       down_scales, y, ws, logits=None, topk_ids=None, topk_weights=None,
                       counts=None, offsets=None, stream=None):
    _check("moe_forward_fp8_packed",
           lib.moe_forward_fp8_packed(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(bias),
                                      _ptr(w_gateup), _ptr(gate_scales), _ptr(up_scales),
                                      _ptr(w_down), _ptr(down_scales), _ptr(y), _ptr(logits),
                                      _ptr(topk_ids), _ptr(topk_weights), _ptr(counts),
                                      _ptr(offsets), _ptr(ws), _nbytes(ws), _stream(stream)))


# GELU experts and the MLP router.

def route_mlp(p, x, w_proj, b_proj, w_out, b_out, logits, topk_ids, topk_weights, ws,
              features=None, stream=None):
    _check("moe_route_mlp", lib.moe_route_mlp(ctypes.byref(p), _ptr(x), _ptr(w_proj),
                                              _ptr(b_proj), _ptr(w_out), _ptr(b_out),
                                              _ptr(features), _ptr(logits), _ptr(topk_ids),
                                              _ptr(topk_weights), _ptr(ws), _nbytes(ws),
                                              _stream(stream)))


def expert_up_gelu(p, x_perm, offsets, w1, b1, h, stream=None):
    _check("moe_expert_up_gelu", lib.moe_expert_up_gelu(ctypes.byref(p), _ptr(x_perm),
                                                        _ptr(offsets), _ptr(w1), _ptr(b1),
                                                        _ptr(h), _stream(stream)))


def expert_up_gelu_gathered(p, x, row_token, offsets, w1, b1, h, stream=None):
    _check("moe_expert_up_gelu_gathered",
           lib.moe_expert_up_gelu_gathered(ctypes.byref(p), _ptr(x), _ptr(row_token),
                                           _ptr(offsets), _ptr(w1), _ptr(b1), _ptr(h),
                                           _stream(stream)))


def expert_down_bias(p, h, offsets, w2, b2, out_perm, stream=None):
    _check("moe_expert_down_bias", lib.moe_expert_down_bias(ctypes.byref(p), _ptr(h),
                                                            _ptr(offsets), _ptr(w2), _ptr(b2),
                                                            _ptr(out_perm), _stream(stream)))


def grouped_ffn_gelu(p, x_perm, offsets, w1, b1, w2, b2, out_perm, h, ws, stream=None):
    _check("moe_grouped_ffn_gelu",
           lib.moe_grouped_ffn_gelu(ctypes.byref(p), _ptr(x_perm), _ptr(offsets), _ptr(w1),
                                    _ptr(b1), _ptr(w2), _ptr(b2), _ptr(out_perm), _ptr(h),
                                    _ptr(ws), _nbytes(ws), _stream(stream)))


def forward_gelu(p, x, w_proj, b_proj, w_out, b_out, w1, b1, w2, b2, y, ws, logits=None,
                 topk_ids=None, topk_weights=None, counts=None, offsets=None, stream=None):
    _check("moe_forward_gelu",
           lib.moe_forward_gelu(ctypes.byref(p), _ptr(x), _ptr(w_proj), _ptr(b_proj),
                                _ptr(w_out), _ptr(b_out), _ptr(w1), _ptr(b1), _ptr(w2),
                                _ptr(b2), _ptr(y), _ptr(logits), _ptr(topk_ids),
                                _ptr(topk_weights), _ptr(counts), _ptr(offsets), _ptr(ws),
                                _nbytes(ws), _stream(stream)))


# The fused FFN (one persistent launch, rows gathered from x).

def fused_ffn(p, x, row_token, offsets, w_gate, w_up, w_down, out_perm, ws, stream=None):
    _check("moe_fused_ffn", lib.moe_fused_ffn(ctypes.byref(p), _ptr(x), _ptr(row_token),
                                              _ptr(offsets), _ptr(w_gate), _ptr(w_up),
                                              _ptr(w_down), _ptr(out_perm), _ptr(ws), _nbytes(ws),
                                              _stream(stream)))


def forward_fused(p, x, w_router, bias, w_gate, w_up, w_down, y, ws, logits=None, topk_ids=None,
                  topk_weights=None, counts=None, offsets=None, stream=None):
    _check("moe_forward_fused",
           lib.moe_forward_fused(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(bias),
                                 _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(y), _ptr(logits),
                                 _ptr(topk_ids), _ptr(topk_weights), _ptr(counts), _ptr(offsets),
                                 _ptr(ws), _nbytes(ws), _stream(stream)))


def fused_error_offset(p, whole_layer: bool) -> int:
    n = ctypes.c_size_t()
    _check("moe_fused_error_offset", lib.moe_fused_error_offset(ctypes.byref(p),
                                                                1 if whole_layer else 0,
                                                                ctypes.byref(n)))
    return n.value
