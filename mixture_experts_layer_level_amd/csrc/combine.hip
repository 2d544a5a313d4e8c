// Un-permutation and router-weighted combine.
//
// "MoE 推理完整机制" (zoe.im), 第二层 范式 A Step 3: the expert outputs are put
// back in token order and multiplied by the router weights; the opening
// dataflow then sums a token's K weighted rows.  Slots dropped by the
// capacity (slot_row < 0) contribute nothing.
//
// Each work item is one 16-byte chunk (8 bf16) of one token's output row: it
// gathers that chunk from the token's K expert rows, accumulates w * value in
// fp32 in k order and writes the bf16 result.  HBM-bound: every kept out_perm
// row is read once and every y row written once.  Grid-stride over the
// N * D / 8 items, blocks of 256.
#include <algorithm>

#include "common.h"

namespace moe {
namespace {

// y chunk c (8 bf16) of token n: the K slot rows and weights of the token are
// read first (the same addresses for every thread of the token), then up to 8
// gathers are in flight before the first is used; the sum runs in k order.
__device__ __forceinline__ void combine_chunk(int64_t n, int c, int D, int K,
                                              const uint16_t* __restrict__ out_perm,
                                              const int32_t* __restrict__ slot_row,
                                              const float* __restrict__ w,
                                              uint16_t* __restrict__ y) {
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int k0 = 0; k0 < K; k0 += 8) {
    int32_t r[8];
    float wk[8];
    uint4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool in = k0 + j < K;
      r[j] = in ? slot_row[n * K + k0 + j] : -1;
      wk[j] = in ? w[n * K + k0 + j] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = r[j] >= 0 ? reinterpret_cast<const uint4*>(out_perm + (int64_t)r[j] * D)[c]
                       : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (r[j] < 0) continue;
      const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = __builtin_fmaf(wk[j], bf16_bits_to_f32(u[i] & 0xffffu), acc[2 * i]);
        acc[2 * i + 1] = __builtin_fmaf(wk[j], bf16_bits_to_f32(u[i] >> 16), acc[2 * i + 1]);
      }
    }
  }
  uint4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  reinterpret_cast<uint4*>(y + n * D)[c] = o;
}

// One thread per (token, 16-byte chunk), grid-stride.
__global__ void __launch_bounds__(256)
combine_kernel(int64_t N, int D, int K, const uint16_t* __restrict__ out_perm,
               const int32_t* __restrict__ slot_row, const float* __restrict__ w,
               uint16_t* __restrict__ y) {
  const int cpr = D / 8;
  const int64_t items = N * cpr;
  for (int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x; item < items;
       item += (int64_t)gridDim.x * 256)
    combine_chunk(item / cpr, (int)(item % cpr), D, K, out_perm, slot_row, w, y);
}

// Many tokens with wide rows: one workgroup per token (grid-stride over
// tokens), as many threads as the row has chunks rounded up to a wave (at most
// 1024).  The token's K slot rows and weights are then
// wave-uniform and come through scalar loads, so the vector-memory path
// carries only the gathered rows: with a thread per chunk, the 2K metadata
// loads of each thread were two thirds of its vector-memory instructions.
// Same sums in the same order as combine_chunk: the results are identical.
__global__ void __launch_bounds__(1024)
combine_token_kernel(int64_t N, int D, int K, const uint16_t* __restrict__ out_perm,
                     const int32_t* __restrict__ slot_row, const float* __restrict__ w,
                     uint16_t* __restrict__ y) {
  const int cpr = D / 8;
  for (int64_t n = blockIdx.x; n < N; n += gridDim.x) {
    for (int c = threadIdx.x; c < cpr; c += blockDim.x) {
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
      for (int k0 = 0; k0 < K; k0 += 8) {
        int32_t r[8];
        float wk[8];
        uint4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bool in = k0 + j < K;
          r[j] = in ? slot_row[n * K + k0 + j] : -1;
          wk[j] = in ? w[n * K + k0 + j] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
          v[j] = r[j] >= 0 ? reinterpret_cast<const uint4*>(out_perm + (int64_t)r[j] * D)[c]
                           : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (r[j] < 0) continue;
          const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] = __builtin_fmaf(wk[j], bf16_bits_to_f32(u[i] & 0xffffu), acc[2 * i]);
            acc[2 * i + 1] = __builtin_fmaf(wk[j], bf16_bits_to_f32(u[i] >> 16), acc[2 * i + 1]);
          }
        }
      }
      uint4 o;
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      o.z = pack_bf16x2(acc[4], acc[5]);
      o.w = pack_bf16x2(acc[6], acc[7]);
      reinterpret_cast<uint4*>(y + n * D)[c] = o;
    }
  }
}

}  // namespace

hipError_t launch_combine(const Dims& d, const uint16_t* out_perm, const int32_t* slot_row,
                          const float* weights, uint16_t* y, hipStream_t s) {
  if (d.N >= 1024 && d.D >= 1024) {
    const int cpr = d.D / 8;
    const int threads = std::min(1024, (cpr + 63) / 64 * 64);
    const int64_t blocks = std::min<int64_t>(d.N, 1 << 20);
    hipLaunchKernelGGL(combine_token_kernel, dim3((unsigned)blocks), dim3(threads), 0, s, d.N, d.D,
                       d.K, out_perm, slot_row, weights, y);
    return hipGetLastError();
  }
  const int64_t items = d.N * (d.D / 8);
  const int64_t blocks = std::min<int64_t>((items + 255) / 256, 1 << 20);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, s, d.N,
                     d.D, d.K, out_perm, slot_row, weights, y);
  return hipGetLastError();
}

}  // namespace moe
