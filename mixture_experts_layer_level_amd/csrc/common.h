// Internal definitions shared by the libmoe HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// Validated problem shape, derived sizes included.
struct Dims {
  int64_t N;     // tokens
  int64_t S;     // slots N*K
  int64_t R;     // permuted rows: S (contiguous) or E*cap (padded)
  int64_t cap;   // capacity per expert, 0 when contiguous
  int D, F, E, K, gating;
  bool padded;
};

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Permutation kernels: slots handled per workgroup.
constexpr int kPermChunk = 1024;

// ---------------------------------------------------------------- device helpers

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ---------------------------------------------------------------- launchers

// route.hip.  With a partials buffer of router_ws_bytes(d) (when nonzero) the
// router runs in its split form and writes partial logits there; launch_topk
// with the same buffer then sums them into logits before selecting (the
// logits are bit-identical to the unsplit router's).  partials NULL: the
// router writes logits and launch_topk reads them.
size_t router_ws_bytes(const Dims& d);
hipError_t launch_router_gemm(const Dims& d, const uint16_t* x, const float* w, float* logits,
                              float* partials, hipStream_t s);
hipError_t launch_topk(const Dims& d, float* logits, const float* bias, int32_t* ids,
                       float* weights, const float* partials, hipStream_t s);

// permute.hip (x_perm NULL: the routing tables only, no row copy)
size_t permute_ws_bytes(const Dims& d);
hipError_t launch_permute(const Dims& d, const uint16_t* x, const int32_t* ids, int32_t* counts,
                          int32_t* offsets, int32_t* row_token, int32_t* slot_row,
                          uint16_t* x_perm, void* ws, hipStream_t s);

// grouped_gemm.hip.  packed: wg (gate/up) or wd (down) is a packed stack
// from launch_pack_weights (wu unused).
size_t ffn_ws_bytes(const Dims& d);  // h when the caller gives none
hipError_t launch_expert_gateup(const Dims& d, const uint16_t* x_perm, const int32_t* offsets,
                                const uint16_t* wg, const uint16_t* wu, uint16_t* h,
                                hipStream_t s, bool packed = false);
hipError_t launch_expert_down(const Dims& d, const uint16_t* h, const int32_t* offsets,
                              const uint16_t* wd, uint16_t* out_perm, hipStream_t s,
                              bool packed = false);
// fp8 / packed: FP8 weight stacks, packed ones (which the 128- and 64-deep
// rings read at any D that is a multiple of 128)
bool gateup_gather_supported(const Dims& d, bool fp8 = false, bool packed = false);
hipError_t launch_expert_gateup_gathered(const Dims& d, const uint16_t* x,
                                         const int32_t* row_token, const int32_t* offsets,
                                         const uint16_t* wg, const uint16_t* wu, uint16_t* h,
                                         hipStream_t s, bool packed = false);
hipError_t launch_grouped_ffn(const Dims& d, const uint16_t* x_perm, const int32_t* offsets,
                              const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                              uint16_t* out_perm, uint16_t* h, void* ws, hipStream_t s,
                              bool packed = false);
// Packed weight stacks: gate/up (w0 = W_gate, w1 = W_up, [E, F, D]) or
// down (w0 = W_down [E, D, F]) as the 32 KB LDS images of their 256-row
// weight stages, in (expert, column tile, stage) order: stages of 64 bf16
// values, or (fp8) of 128 FP8 codes, passed here as pairs of codes.
size_t packed_weight_bytes(const Dims& d, bool gateup, bool fp8 = false);
hipError_t launch_pack_weights(const Dims& d, bool gateup, const uint16_t* w0, const uint16_t* w1,
                               uint16_t* out, hipStream_t s, bool fp8 = false);

// Block-scaled FP8 weights of one matrix stack [E, rows, cols]: E4M3 codes
// [E, rows, cols] and scale bytes [E, rows/32, cols/32, 32].
struct Fp8Weight {
  const uint8_t* codes;
  const uint8_t* scales;
};
// packed: wg.codes (gate/up) or wd.codes (down) is a packed FP8 stack (its
// D, resp. F, a multiple of 128; wu.codes unused); the scales stay in place.
hipError_t launch_expert_gateup_fp8(const Dims& d, const uint16_t* x_perm, const int32_t* offsets,
                                    const Fp8Weight& wg, const Fp8Weight& wu, uint16_t* h,
                                    hipStream_t s, bool packed = false);
hipError_t launch_expert_gateup_fp8_gathered(const Dims& d, const uint16_t* x,
                                             const int32_t* row_token, const int32_t* offsets,
                                             const Fp8Weight& wg, const Fp8Weight& wu,
                                             uint16_t* h, hipStream_t s, bool packed = false);
hipError_t launch_expert_down_fp8(const Dims& d, const uint16_t* h, const int32_t* offsets,
                                  const Fp8Weight& wd, uint16_t* out_perm, hipStream_t s,
                                  bool packed = false);
hipError_t launch_grouped_ffn_fp8(const Dims& d, const uint16_t* x_perm, const int32_t* offsets,
                                  const Fp8Weight& wg, const Fp8Weight& wu, const Fp8Weight& wd,
                                  uint16_t* out_perm, uint16_t* h, void* ws, hipStream_t s,
                                  bool packed = false);

// GELU-expert layer: up GEMM with bias + GELU epilogue, down GEMM with bias,
// and the router's compression GEMM (one group of N rows).
hipError_t launch_expert_up_gelu(const Dims& d, const uint16_t* x_perm, const int32_t* offsets,
                                 const uint16_t* w1, const float* b1, uint16_t* h,
                                 hipStream_t s);
hipError_t launch_expert_up_gelu_gathered(const Dims& d, const uint16_t* x,
                                          const int32_t* row_token, const int32_t* offsets,
                                          const uint16_t* w1, const float* b1, uint16_t* h,
                                          hipStream_t s);
hipError_t launch_expert_down_bias(const Dims& d, const uint16_t* h, const int32_t* offsets,
                                   const uint16_t* w2, const float* b2, uint16_t* out_perm,
                                   hipStream_t s);
hipError_t launch_grouped_ffn_gelu(const Dims& d, const uint16_t* x_perm, const int32_t* offsets,
                                   const uint16_t* w1, const float* b1, const uint16_t* w2,
                                   const float* b2, uint16_t* out_perm, uint16_t* h, void* ws,
                                   hipStream_t s);
// C[N, Nout] = bf16(GELU(A W^T + bias)); offsets2: 2 int32 of device scratch.
hipError_t launch_dense_gelu(int64_t N, int Kd, int Nout, const uint16_t* A, const uint16_t* W,
                             const float* bias, uint16_t* C, int32_t* offsets2, hipStream_t s);

// The fused FFN: one persistent launch for gate/up, SwiGLU and down, A rows of
// gate/up gathered from x by row_token (contiguous layout).  Workspace: h and
// the launch's counters; *err receives the device address of its error word.
size_t fused_ws_bytes(const Dims& d);
size_t fused_err_offset(const Dims& d);
hipError_t launch_fused_ffn(const Dims& d, const uint16_t* x, const int32_t* row_token,
                            const int32_t* offsets, const uint16_t* wg, const uint16_t* wu,
                            const uint16_t* wd, uint16_t* out_perm, void* ws, hipStream_t s);

// quant.hip
hipError_t launch_quantize_fp8(int64_t rows, int cols, const uint16_t* w, uint8_t* codes,
                               uint8_t* scales, hipStream_t s);

// combine.hip
hipError_t launch_combine(const Dims& d, const uint16_t* out_perm, const int32_t* slot_row,
                          const float* weights, uint16_t* y, hipStream_t s);

// stats.hip
hipError_t launch_routing_stats(int E, const int32_t* counts, float* ema, float* bias, float decay,
                                float step, hipStream_t s);

// Compute units of the current device (cached per device).
int device_cu_count();

}  // namespace moe
