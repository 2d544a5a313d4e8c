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
// bf16 MFMA with an exact three-way split of the fp32 router weights.
//
// Every fp32 weight w is split as w = hi + mid + lo with hi = bf16(w),
// mid = bf16(w - hi), lo = w - hi - mid; all three are exact bf16 values (a
// 24-bit significand cut into three 8-bit pieces), so the layer's x.w is
// the sum of 3*D exact bf16 x bf16 products, accumulated in fp32 by
// v_mfma_f32_32x32x16_bf16.  hi products go to one accumulator and the much
// smaller mid + lo products to another; the two are added once.  The result
// is an fp32 sum of exact products, so it obeys the usual fp32 dot-product
// error bound (relative to sum |x.w|), at bf16 MFMA speed instead of fp32
// vector-FMA speed.
//
// Workgroup = S waves on one tile of WT tokens x WT experts; wave s takes the
// 64-deep k blocks s, s+S, s+2S, ...  Operands go straight from global memory
// into MFMA registers (lane l reads a contiguous run of row l % 32), so there
// is no LDS staging; the S partial tiles are summed through LDS in
// wave order, so the result does not depend on scheduling.

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t rne_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Split 8 fp32 weights into the hi / mid / lo bf16 vectors.
__device__ __forceinline__ void split3(const float4& a, const float4& b, bf16x8_t& hi,
                                       bf16x8_t& mid, bf16x8_t& lo) {
  const float w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t h[4], m[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t hb[2], mb[2], lb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float v = w[2 * i + j];
      hb[j] = rne_bf16(v);
      const float r1 = v - __uint_as_float(hb[j] << 16);      // exact
      mb[j] = rne_bf16(r1);
      const float r2 = r1 - __uint_as_float(mb[j] << 16);     // exact, fits bf16
      lb[j] = __float_as_uint(r2) >> 16;
    }
    h[i] = hb[0] | (hb[1] << 16);
    m[i] = mb[0] | (mb[1] << 16);
    l[i] = lb[0] | (lb[1] << 16);
  }
  hi = __builtin_bit_cast(bf16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
  mid = __builtin_bit_cast(bf16x8_t, make_uint4(m[0], m[1], m[2], m[3]));
  lo = __builtin_bit_cast(bf16x8_t, make_uint4(l[0], l[1], l[2], l[3]));
}

// Launch bounds follow the largest workgroup the launcher uses for each tile
// size (4 waves at 64x64, 8 at 32x32), which sets the register budget.
template <int WT>
__global__ void __launch_bounds__(WT == 64 ? 256 : 512)
router_mfma_kernel(int64_t N, int D, int E, int vec4, const uint16_t* __restrict__ x,
                   const float* __restrict__ w, float* __restrict__ logits) {
  constexpr int TB = WT / 32;                   // 32-row blocks per tile side
  constexpr int LD = WT + 4;                    // LDS row stride (floats)
  extern __shared__ float red[];                // [S-1][WT][LD] partial tiles
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int S = blockDim.x >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * WT;
  const int e0 = blockIdx.y * WT;
  const int r = lane & 31, kh = lane >> 5;

  // k order inside a 64-deep block: MFMA step ks takes, in lane half kh,
  // k = 32*kh + 8*ks .. +7.  Both operands use the same order, so the MFMA
  // still pairs equal k; a lane then reads one contiguous 32-element run of
  // its row per block (64 bytes of x, one 128-byte line of w).
  const uint16_t* xr[TB];
  const float* wr[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    xr[b] = x + min<int64_t>(n0 + b * 32 + r, N - 1) * D + kh * 32;
    wr[b] = w + (int64_t)min(e0 + b * 32 + r, E - 1) * D + kh * 32;
  }
  f32x16_t acc_hi[TB][TB], acc_lo[TB][TB];      // [expert block][token block]
#pragma unroll
  for (int i = 0; i < TB; ++i)
#pragma unroll
    for (int j = 0; j < TB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc_hi[i][j][v] = acc_lo[i][j][v] = 0.f;

  // One 64-deep k block of raw operands.  With 32x32 tiles the next block is
  // loaded while the MFMAs of the current one run (two register sets,
  // alternating).
  struct Blk {
    uint4 x[4][TB];
    float4 wa[4][TB], wb[4][TB];
  };
  auto load = [&](Blk& b, int kb) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int k = kb * 64 + ks * 8;
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        b.x[ks][t] = *reinterpret_cast<const uint4*>(xr[t] + k);
        b.wa[ks][t] = *reinterpret_cast<const float4*>(wr[t] + k);
        b.wb[ks][t] = *reinterpret_cast<const float4*>(wr[t] + k + 4);
      }
    }
  };
  auto compute = [&](const Blk& b) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int i = 0; i < TB; ++i) {
        bf16x8_t hi, mid, lo;
        split3(b.wa[ks][i], b.wb[ks][i], hi, mid, lo);
#pragma unroll
        for (int j = 0; j < TB; ++j) {
          const bf16x8_t xa = __builtin_bit_cast(bf16x8_t, b.x[ks][j]);
          acc_hi[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, xa, acc_hi[i][j], 0, 0, 0);
          acc_lo[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mid, xa, acc_lo[i][j], 0, 0, 0);
          acc_lo[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, xa, acc_lo[i][j], 0, 0, 0);
        }
      }
  };
  const int nkb = D / 64;
  if constexpr (WT == 64) {
    // 64x64 tiles are issued when the grid already fills the chip: one
    // register set, no look-ahead (two sets would spill).
    Blk b0;
    for (int kb = wave; kb < nkb; kb += S) {
      load(b0, kb);
      compute(b0);
    }
  } else {
    Blk b0, b1;
    int kb = wave;
    if (kb < nkb) load(b0, kb);
    while (kb < nkb) {
      if (kb + S < nkb) load(b1, kb + S);
      compute(b0);
      kb += S;
      if (kb >= nkb) break;
      if (kb + S < nkb) load(b0, kb + S);
      compute(b1);
      kb += S;
    }
  }
  // Block (i, j): lane l, register v holds expert 8*(v/4) + 4*(l/32) + v%4 of
  // expert block i and token l%32 of token block j; four consecutive
  // registers are four consecutive experts.  Waves 1..S-1 leave their partial
  // tiles in LDS; wave 0 adds them to its own in wave order and stores.
  if (wave > 0) {
    float* mine = red + (size_t)(wave - 1) * WT * LD;
#pragma unroll
    for (int i = 0; i < TB; ++i)
#pragma unroll
      for (int j = 0; j < TB; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float4 v;
          v.x = acc_hi[i][j][4 * g + 0] + acc_lo[i][j][4 * g + 0];
          v.y = acc_hi[i][j][4 * g + 1] + acc_lo[i][j][4 * g + 1];
          v.z = acc_hi[i][j][4 * g + 2] + acc_lo[i][j][4 * g + 2];
          v.w = acc_hi[i][j][4 * g + 3] + acc_lo[i][j][4 * g + 3];
          *reinterpret_cast<float4*>(mine + (j * 32 + r) * LD + i * 32 + 8 * g + 4 * kh) = v;
        }
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int i = 0; i < TB; ++i)
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      const int64_t n = n0 + j * 32 + r;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int el = i * 32 + 8 * g + 4 * kh;
        float4 v;
        v.x = acc_hi[i][j][4 * g + 0] + acc_lo[i][j][4 * g + 0];
        v.y = acc_hi[i][j][4 * g + 1] + acc_lo[i][j][4 * g + 1];
        v.z = acc_hi[i][j][4 * g + 2] + acc_lo[i][j][4 * g + 2];
        v.w = acc_hi[i][j][4 * g + 3] + acc_lo[i][j][4 * g + 3];
        for (int q = 0; q + 1 < S; ++q) {
          const float4 o = *reinterpret_cast<const float4*>(red + ((size_t)q * WT + j * 32 + r) * LD + el);
          v.x += o.x;
          v.y += o.y;
          v.z += o.z;
          v.w += o.w;
        }
        if (n >= N) continue;
        float* dst = logits + n * E + e0 + el;
        if (vec4 && e0 + el + 3 < E) {
          *reinterpret_cast<float4*>(dst) = v;
        } else {
          const float vv[4] = {v.x, v.y, v.z, v.w};
          for (int c = 0; c < 4; ++c)
            if (e0 + el + c < E) dst[c] = vv[c];
        }
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
  // 64x64 tiles with 4 waves when they alone give the chip at least one
  // workgroup per CU; otherwise 32x32 tiles and as many waves per tile
  // (up to 8, at most one per 64-deep k block) as bring the grid to about
  // 512 waves.  LDS: (S-1) partial tiles, at most 52 KB.
  const int nkb = d.D / 64;
  // 16-byte stores of four logits when every row start is 16-byte aligned
  const int vec4 = (d.E % 4 == 0) && ((reinterpret_cast<uintptr_t>(logits) & 15u) == 0);
  const int64_t t64 = ((d.N + 63) / 64) * ((d.E + 63) / 64);
  if (t64 >= device_cu_count()) {
    const int S = nkb < 4 ? nkb : 4;
    dim3 grid((unsigned)((d.N + 63) / 64), (unsigned)((d.E + 63) / 64));
    hipLaunchKernelGGL(router_mfma_kernel<64>, grid, dim3(64 * S),
                       (S - 1) * 64 * 68 * sizeof(float), s, d.N, d.D, d.E, vec4, x, w,
                       logits);
    return hipGetLastError();
  }
  const int64_t t32 = ((d.N + 31) / 32) * ((d.E + 31) / 32);
  int S = (int)((512 + t32 - 1) / t32);
  if (S > 8) S = 8;
  if (S > nkb) S = nkb;
  if (S < 1) S = 1;
  dim3 grid((unsigned)((d.N + 31) / 32), (unsigned)((d.E + 31) / 32));
  hipLaunchKernelGGL(router_mfma_kernel<32>, grid, dim3(64 * S), (S - 1) * 32 * 36 * sizeof(float), s,
                     d.N, d.D, d.E, vec4, x, w, logits);
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
