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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values to packed bf16, round to nearest even (one
// v_cvt_pk_bf16_f32), and the bf16 values back as fp32.
__device__ __forceinline__ uint32_t rne_pk(f32x2_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ f32x2_t unpk(uint32_t b) {
  return f32x2_t{__uint_as_float(b << 16), __uint_as_float(b & 0xffff0000u)};
}

// Split 8 fp32 weights into the hi / mid / lo bf16 vectors: hi = bf16(w),
// mid = bf16(w - hi) (w - hi is exact), lo = w - hi - mid (exact, at most 8
// significant bits, so its top 16 bits are the value).
__device__ __forceinline__ void split3(const float4& a, const float4& b, bf16x8_t& hi,
                                       bf16x8_t& mid, bf16x8_t& lo) {
  const f32x2_t w[4] = {{a.x, a.y}, {a.z, a.w}, {b.x, b.y}, {b.z, b.w}};
  uint32_t h[4], m[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = rne_pk(w[i]);
    const f32x2_t r1 = w[i] - unpk(h[i]);
    m[i] = rne_pk(r1);
    const f32x2_t r2 = r1 - unpk(m[i]);
    l[i] = (__float_as_uint(r2.x) >> 16) | (__float_as_uint(r2.y) & 0xffff0000u);
  }
  hi = __builtin_bit_cast(bf16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
  mid = __builtin_bit_cast(bf16x8_t, make_uint4(m[0], m[1], m[2], m[3]));
  lo = __builtin_bit_cast(bf16x8_t, make_uint4(l[0], l[1], l[2], l[3]));
}

// Launch bounds follow the largest workgroup the launcher uses for each tile
// size (4 waves at 64x64, 8 at 32x32), which sets the register budget.
//
// Split form (partials != NULL, 32x32 tiles only): the S waves of a tile run
// as S one-wave workgroups, wave s of tile t in workgroup t * S + s, each
// writing its partial tile to partials[s] ([S][N][E] fp32); the top-K kernel
// then adds the partials in wave order, the order of the LDS reduction here.
// Every logit is the same sum of the same terms in the same order: the two
// forms give bit-identical logits, the split one on S times as many compute
// units (a decode-sized router has only a few tiles).
template <int WT>
__global__ void __launch_bounds__(WT == 64 ? 256 : 512)
router_mfma_kernel(int64_t N, int D, int E, int vec4, const uint16_t* __restrict__ x,
                   const float* __restrict__ w, float* __restrict__ logits, int split_waves,
                   float* __restrict__ partials) {
  constexpr int TB = WT / 32;                   // 32-row blocks per tile side
  constexpr int LD = WT + 4;                    // LDS row stride (floats)
  extern __shared__ float red[];                // [S-1][WT][LD] partial tiles
  const int lane = threadIdx.x & 63;
  const bool split = partials != nullptr;
  const int S = split ? split_waves : (int)(blockDim.x >> 6);
  // This workgroup's tile.  Tiles are numbered token tile by token tile (the
  // expert tiles of one token tile are consecutive) and cut into eight
  // contiguous parts, one per XCD (workgroup b runs on XCD b % 8), so the
  // workgroups that read the same x rows run together and share them in one
  // L2.  The grid is a multiple of 8; workgroups past the last tile leave.
  const int ne = (E + WT - 1) / WT;
  const int64_t total = ((N + WT - 1) / WT) * ne * (split ? S : 1);
  int64_t v = (int64_t)(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  if (v >= total) return;
  int wave = threadIdx.x >> 6;
  if (split) {   // workgroup = (tile, wave)
    wave = (int)(v % S);
    v /= S;
  }
  const int64_t n0 = (v / ne) * WT;
  const int e0 = (int)(v % ne) * WT;
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
    // 64x64 tiles: two full register sets would spill, so the look-ahead is
    // by half blocks (k-steps 0-1, then 2-3): the next half loads while the
    // MFMAs of the current one run, in the registers of one block.  Same k
    // order as above, so the same sums.
    struct Half {
      uint4 x[2][TB];
      float4 wa[2][TB], wb[2][TB];
    };
    auto load_half = [&](Half& h, int kb, int part) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int k = kb * 64 + (2 * part + q) * 8;
#pragma unroll
        for (int t = 0; t < TB; ++t) {
          h.x[q][t] = *reinterpret_cast<const uint4*>(xr[t] + k);
          h.wa[q][t] = *reinterpret_cast<const float4*>(wr[t] + k);
          h.wb[q][t] = *reinterpret_cast<const float4*>(wr[t] + k + 4);
        }
      }
    };
    auto compute_half = [&](const Half& h) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int i = 0; i < TB; ++i) {
          bf16x8_t hi, mid, lo;
          split3(h.wa[q][i], h.wb[q][i], hi, mid, lo);
#pragma unroll
          for (int j = 0; j < TB; ++j) {
            const bf16x8_t xa = __builtin_bit_cast(bf16x8_t, h.x[q][j]);
            acc_hi[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, xa, acc_hi[i][j], 0, 0, 0);
            acc_lo[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mid, xa, acc_lo[i][j], 0, 0, 0);
            acc_lo[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, xa, acc_lo[i][j], 0, 0, 0);
          }
        }
    };
    Half h0, h1;
    int kb = wave;
    if (kb < nkb) load_half(h0, kb, 0);
    while (kb < nkb) {
      load_half(h1, kb, 1);
      compute_half(h0);
      const int kn = kb + S;
      if (kn < nkb) load_half(h0, kn, 0);
      compute_half(h1);
      kb = kn;
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
  // tiles in LDS; wave 0 adds them to its own in wave order and stores.  In
  // the split form every wave stores its partial tile to partials[wave].
  if (split) {
    float* dst0 = partials + (size_t)wave * N * E;
#pragma unroll
    for (int i = 0; i < TB; ++i)
#pragma unroll
      for (int j = 0; j < TB; ++j) {
        const int64_t n = n0 + j * 32 + r;
        if (n >= N) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int el = i * 32 + 8 * g + 4 * kh;
          float4 v4;
          v4.x = acc_hi[i][j][4 * g + 0] + acc_lo[i][j][4 * g + 0];
          v4.y = acc_hi[i][j][4 * g + 1] + acc_lo[i][j][4 * g + 1];
          v4.z = acc_hi[i][j][4 * g + 2] + acc_lo[i][j][4 * g + 2];
          v4.w = acc_hi[i][j][4 * g + 3] + acc_lo[i][j][4 * g + 3];
          float* dst = dst0 + n * E + e0 + el;
          if (vec4 && e0 + el + 3 < E) {
            *reinterpret_cast<float4*>(dst) = v4;
          } else {
            const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
            for (int c = 0; c < 4; ++c)
              if (e0 + el + c < E) dst[c] = vv[c];
          }
        }
      }
    return;
  }
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

// With partials (the split router), each logit is first summed from its
// nparts partials in order and written to logits.
template <int EPL>
__global__ void __launch_bounds__(256)
topk_kernel(int64_t N, int E, int K, int gating, float* __restrict__ logits,
            const float* __restrict__ bias, int32_t* __restrict__ ids,
            float* __restrict__ weights, const float* __restrict__ partials, int nparts) {
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  float* row = logits + n * E;
  uint64_t pk[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    pk[j] = 0;
    if (e < E) {
      if (partials) {
        float lg = partials[n * E + e];
        for (int q = 1; q < nparts; ++q) lg += partials[(size_t)q * N * E + n * E + e];
        row[e] = lg;
      }
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

namespace {

// Router tiling: 64x64 tiles with 4 waves when they alone give the chip at
// least one workgroup per CU; otherwise 32x32 tiles and as many waves per
// tile (up to 8, at most one per 64-deep k block) as bring the grid to about
// 512 waves.  S = waves per tile (0 for the 64x64 tiles, which never split).
// 32x32 tiles: waves per tile.
int router_waves32(const Dims& d) {
  const int nkb = d.D / 64;
  const int64_t t32 = ((d.N + 31) / 32) * ((d.E + 31) / 32);
  if (t32 <= 0) return 1;
  int S = (int)((512 + t32 - 1) / t32);
  if (S > 8) S = 8;
  if (S > nkb) S = nkb;
  if (S < 1) S = 1;
  return S;
}

int router_split_waves(const Dims& d) {
  const int64_t t64 = ((d.N + 63) / 64) * ((d.E + 63) / 64);
  if (t64 >= device_cu_count()) return 0;
  return router_waves32(d);
}

}  // namespace

// Sized without asking the device (workspace sizes are host-only): the 32x32
// tiles are taken only when the 64x64 ones number fewer than the CUs, and no
// device has more than 1024.
size_t router_ws_bytes(const Dims& d) {
  const int64_t t64 = ((d.N + 63) / 64) * ((d.E + 63) / 64);
  const int S = t64 < 1024 ? router_waves32(d) : 1;
  return S > 1 ? align_up((size_t)S * d.N * d.E * sizeof(float)) : 0;
}

hipError_t launch_router_gemm(const Dims& d, const uint16_t* x, const float* w, float* logits,
                              float* partials, hipStream_t s) {
  // LDS: (S-1) partial tiles, at most 52 KB (none in the split form).
  const int nkb = d.D / 64;
  // 16-byte stores of four logits when every row start is 16-byte aligned
  const int vec4 = (d.E % 4 == 0) && ((reinterpret_cast<uintptr_t>(logits) & 15u) == 0) &&
                   ((reinterpret_cast<uintptr_t>(partials) & 15u) == 0);
  const int S = router_split_waves(d);
  if (S == 0) {
    const int64_t t64 = ((d.N + 63) / 64) * ((d.E + 63) / 64);
    const int S64 = nkb < 4 ? nkb : 4;
    dim3 grid((unsigned)((t64 + 7) / 8 * 8));
    hipLaunchKernelGGL(router_mfma_kernel<64>, grid, dim3(64 * S64),
                       (S64 - 1) * 64 * 68 * sizeof(float), s, d.N, d.D, d.E, vec4, x, w,
                       logits, 0, (float*)nullptr);
    return hipGetLastError();
  }
  const int64_t t32 = ((d.N + 31) / 32) * ((d.E + 31) / 32);
  if (partials && S > 1) {
    // split form: one one-wave workgroup per (tile, wave)
    dim3 grid((unsigned)((t32 * S + 7) / 8 * 8));
    hipLaunchKernelGGL(router_mfma_kernel<32>, grid, dim3(64), 0, s, d.N, d.D, d.E, vec4, x, w,
                       logits, S, partials);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((t32 + 7) / 8 * 8));
  hipLaunchKernelGGL(router_mfma_kernel<32>, grid, dim3(64 * S), (S - 1) * 32 * 36 * sizeof(float), s,
                     d.N, d.D, d.E, vec4, x, w, logits, 0, (float*)nullptr);
  return hipGetLastError();
}

hipError_t launch_topk(const Dims& d, float* logits, const float* bias, int32_t* ids,
                       float* weights, const float* partials, hipStream_t s) {
  dim3 grid((unsigned)((d.N + 3) / 4));
  const int epl = (d.E + 63) / 64;
  const int nparts = partials ? router_split_waves(d) : 0;
  if (nparts <= 1) partials = nullptr;
#define MOE_TOPK_CASE(V)                                                                   \
  hipLaunchKernelGGL(topk_kernel<V>, grid, dim3(256), 0, s, d.N, d.E, d.K, d.gating, logits, \
                     bias, ids, weights, partials, nparts)
  if (epl <= 1) MOE_TOPK_CASE(1);
  else if (epl <= 2) MOE_TOPK_CASE(2);
  else if (epl <= 4) MOE_TOPK_CASE(4);
  else if (epl <= 8) MOE_TOPK_CASE(8);
  else MOE_TOPK_CASE(16);
#undef MOE_TOPK_CASE
  return hipGetLastError();
}

}  // namespace moe
