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
// row is read once and every y row written once.
#include "common.h"

namespace moe {
namespace {

__global__ void __launch_bounds__(256)
combine_kernel(int64_t N, int D, int K, int tpb, const uint16_t* __restrict__ out_perm,
               const int32_t* __restrict__ slot_row, const float* __restrict__ w,
               uint16_t* __restrict__ y) {
  const int cpr = D / 8;
  const int64_t t0 = (int64_t)blockIdx.x * tpb;
  for (int wi = threadIdx.x; wi < tpb * cpr; wi += 256) {
    const int64_t n = t0 + wi / cpr;
    if (n >= N) break;
    const int c = wi % cpr;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int k = 0; k < K; ++k) {
      const int32_t r = slot_row[n * K + k];
      if (r < 0) continue;
      const float wk = w[n * K + k];
      const uint4 v = reinterpret_cast<const uint4*>(out_perm + (int64_t)r * D)[c];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = __builtin_fmaf(wk, bf16_bits_to_f32(u[i] & 0xffffu), acc[2 * i]);
        acc[2 * i + 1] = __builtin_fmaf(wk, bf16_bits_to_f32(u[i] >> 16), acc[2 * i + 1]);
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

}  // namespace

hipError_t launch_combine(const Dims& d, const uint16_t* out_perm, const int32_t* slot_row,
                          const float* weights, uint16_t* y, hipStream_t s) {
  const int cpr = d.D / 8;
  const int tpb = cpr >= 2048 ? 1 : 2048 / cpr;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((d.N + tpb - 1) / tpb)), dim3(256), 0, s,
                     d.N, d.D, d.K, tpb, out_perm, slot_row, weights, y);
  return hipGetLastError();
}

}  // namespace moe
