"""Single-GPU MoE-layer forward pass for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libmoe.so`` (hand-written HIP
kernels, declared in ``include/moe.h``).  This package only marshals
arguments: it turns torch tensors into device pointers and the current HIP
stream into a handle, calls the library and raises on a non-OK status.
PyTorch supplies device memory and streams and nothing else; there is no
fallback path, and a missing library is an error.
"""
from ._lib import (  # noqa: F401
    GATING_SIGMOID_RENORM,
    GATING_SOFTMAX_TOPK,
    MoEError,
    MoEProblem,
    abi_version,
    expert_down,
    expert_down_bias,
    expert_down_fp8,
    expert_down_packed,
    expert_gateup,
    expert_gateup_gathered,
    expert_gateup_fp8,
    expert_gateup_fp8_gathered,
    expert_gateup_packed,
    expert_gateup_packed_gathered,
    expert_up_gelu,
    expert_up_gelu_gathered,
    forward,
    forward_fp8,
    forward_fused,
    forward_packed,
    forward_static,
    forward_gelu,
    fused_error_offset,
    fused_ffn,
    grouped_ffn,
    grouped_ffn_fp8,
    grouped_ffn_gelu,
    lib,
    library_path,
    pack_weights,
    packed_weight_size,
    PACK_DOWN,
    PACK_GATEUP,
    permute,
    permuted_rows,
    problem,
    quantize_fp8,
    STATIC_SCRATCH_BYTES,
    route,
    route_mlp,
    routing_stats,
    status_str,
    unpermute_combine,
    workspace_size,
)
