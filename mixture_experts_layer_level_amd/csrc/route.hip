// Router GEMM and top-K gating.
//
// Router: logits = x . W_gate^T, a bias-free Linear(D -> E) ("MoE 推理完整机制",
// zoe.im, 第一层: Router 与 Top-K 的算法细节; gate Linear of "MoE 大规模分布式
// 推理工程实战", ybb.press, 4.1).  Gating: top-K on key = logit + bias, then
// softmax over the K selected keys, or sigmoid of the K keys renormalised by
// their sum (zoe.im 第一层, "DeepSeek 的 sigmoid + norm 变体").
#include "common.h"

namespace moe {
namespace {

// ------------------------------------------------------------------ router GEMM
// fp32 FMA tiles of 64 tokens x 64 experts, 32-deep K steps staged through LDS.
// Thread (ty, tx) owns tokens ty + 16*i and experts tx + 16*j (i, j < 4), so a
// wave reads 4 broadcast token values and 16 consecutive expert values per k.
constexpr int RT_TM = 64, RT_TE = 64, RT_BK = 32;

__global__ void __launch_bounds__(256)
router_gemm_kernel(int64_t N, int D, int E, const uint16_t* __restrict__ x,
                   const float* __restrict__ w, float* __restrict__ logits) {
  __shared__ float xs[RT_BK][RT_TM + 4];
  __shared__ float ws[RT_BK][RT_TE + 4];
  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;
  const int64_t n0 = (int64_t)blockIdx.y * RT_TM;
  const int e0 = blockIdx.x * RT_TE;

  // loader mapping: 64 rows x 4 chunks of 8 elements
  const int lrow = tid >> 2, lchunk = tid & 3;
  const int64_t xrow = min<int64_t>(n0 + lrow, N - 1);
  const int wrow = min(e0 + lrow, E - 1);
  const uint16_t* xp = x + xrow * D + lchunk * 8;
  const float* wp = w + (int64_t)wrow * D + lchunk * 8;

  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  for (int k0 = 0; k0 < D; k0 += RT_BK) {
    uint4 xv = *reinterpret_cast<const uint4*>(xp + k0);
    float4 w0 = *reinterpret_cast<const float4*>(wp + k0);
    float4 w1 = *reinterpret_cast<const float4*>(wp + k0 + 4);
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xs[lchunk * 8 + 2 * i][lrow] = bf16_bits_to_f32(xw[i] & 0xffffu);
      xs[lchunk * 8 + 2 * i + 1][lrow] = bf16_bits_to_f32(xw[i] >> 16);
    }
    ws[lchunk * 8 + 0][lrow] = w0.x;
    ws[lchunk * 8 + 1][lrow] = w0.y;
    ws[lchunk * 8 + 2][lrow] = w0.z;
    ws[lchunk * 8 + 3][lrow] = w0.w;
    ws[lchunk * 8 + 4][lrow] = w1.x;
    ws[lchunk * 8 + 5][lrow] = w1.y;
    ws[lchunk * 8 + 6][lrow] = w1.z;
    ws[lchunk * 8 + 7][lrow] = w1.w;
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < RT_BK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[k][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = ws[k][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t n = n0 + ty + 16 * i;
    if (n >= N) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx + 16 * j;
      if (e < E) logits[n * E + e] = acc[i][j];
    }
  }
}

// ------------------------------------------------------------------ top-K
// One wave per token.  Lane l holds the keys of experts l, l+64, ... packed as
// (orderable(key) << 32) | (0xffffffff - e): the unsigned maximum is the
// largest key and, among equal keys, the lowest expert id.  K rounds of a
// wave-wide max each remove one winner.  Packed value 0 never encodes a real
// key (orderable() is 0 only for a negative-NaN pattern, canonicalised away).

__device__ __forceinline__ uint32_t orderable(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float from_orderable(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

template <int EPL>
__global__ void __launch_bounds__(256)
topk_kernel(int64_t N, int E, int K, int gating, const float* __restrict__ logits,
            const float* __restrict__ bias, int32_t* __restrict__ ids,
            float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const float* row = logits + n * E;
  uint64_t pk[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    pk[j] = 0;
    if (e < E) {
      float key = row[e];
      if (bias) key = key + bias[e];
      if (key == 0.f) key = 0.f;                  // -0.0 -> +0.0
      if (key != key) key = -__builtin_inff();    // NaN ranks last
      pk[j] = ((uint64_t)orderable(key) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
    }
  }
  float my_key = 0.f;
  int my_id = 0;
  for (int r = 0; r < K; ++r) {
    uint64_t best = pk[0];
#pragma unroll
    for (int j = 1; j < EPL; ++j) best = pk[j] > best ? pk[j] : best;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const uint64_t o = __shfl_xor(best, off, 64);
      best = o > best ? o : best;
    }
    const int e = (int)(0xffffffffu - (uint32_t)best);
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (lane + 64 * j == e) pk[j] = 0;
    if (lane == r) {
      my_id = e;
      my_key = from_orderable((uint32_t)(best >> 32));
    }
  }
  // weights over the K selected keys (lanes 0..K-1)
  const bool sel = lane < K;
  const float kmax = __shfl(my_key, 0, 64);
  float z = 0.f;
  if (gating == MOE_GATING_SOFTMAX_TOPK) {
    if (sel && kmax != -__builtin_inff()) z = expf(my_key - kmax);
  } else {
    if (sel) z = 1.f / (1.f + expf(-my_key));
  }
  float tot = z;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off, 64);
  if (sel) {
    ids[n * K + lane] = my_id;
    weights[n * K + lane] = tot > 0.f ? z / tot : 1.f / (float)K;
  }
}

}  // namespace

hipError_t launch_router_gemm(const Dims& d, const uint16_t* x, const float* w, float* logits,
                              hipStream_t s) {
  dim3 grid((d.E + RT_TE - 1) / RT_TE, (unsigned)((d.N + RT_TM - 1) / RT_TM));
  hipLaunchKernelGGL(router_gemm_kernel, grid, dim3(256), 0, s, d.N, d.D, d.E, x, w, logits);
  return hipGetLastError();
}

hipError_t launch_topk(const Dims& d, const float* logits, const float* bias, int32_t* ids,
                       float* weights, hipStream_t s) {
  dim3 grid((unsigned)((d.N + 3) / 4));
  const int epl = (d.E + 63) / 64;
#define MOE_TOPK_CASE(V)                                                                   \
  hipLaunchKernelGGL(topk_kernel<V>, grid, dim3(256), 0, s, d.N, d.E, d.K, d.gating, logits, \
                     bias, ids, weights)
  if (epl <= 1) MOE_TOPK_CASE(1);
  else if (epl <= 2) MOE_TOPK_CASE(2);
  else if (epl <= 4) MOE_TOPK_CASE(4);
  else if (epl <= 8) MOE_TOPK_CASE(8);
  else MOE_TOPK_CASE(16);
#undef MOE_TOPK_CASE
  return hipGetLastError();
}

}  // namespace moe
