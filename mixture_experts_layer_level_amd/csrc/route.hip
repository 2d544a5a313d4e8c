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

// ------------------------------------------------------------------ router GEMM, LDS-staged
// For many tokens and E a multiple of 256: a workgroup of 8 waves takes 128
// tokens x 256 experts and one part of k, and stages both operands through LDS
// (LDS-DMA, global_load_lds_dwordx4), so each x and weight byte leaves memory
// once per workgroup instead of once per wave: per 64-deep stage 16 KB of x
// (bf16) and 64 KB of weights (fp32) feed 128 x 256 x 64 x 3 MACs.  Wave w
// computes all 128 tokens x experts [32 w, +32) with the same exact three-way
// weight split and the same hi / mid+lo accumulators as the kernel above:
// each weight value is split by one wave only (with 64 x 64 per wave, two
// waves split every weight block, and the split, not the MFMAs, set the
// kernel's pace).  Two LDS slots: stage kt+2 is fetched once every wave is done
// with stage kt.  k is cut into `parts` contiguous parts; a part's partial
// tile is hi + lo of its accumulators.  Split form (partials != NULL): one
// workgroup per (tile, part), partial tiles to partials[part] and summed by
// the top-K kernel in part order.  Otherwise one workgroup per tile runs the
// parts in order and adds each into logits (part 0 writes it): the same sums
// in the same order, so both forms give the same logits bit for bit.
constexpr int kRT = 128, kRE = 256, kRBK = 64;
constexpr int kRXU4 = kRT * kRBK * 2 / 16;   // x stage: 16 KB
constexpr int kRWU4 = kRE * kRBK * 4 / 16;   // weight stage: 64 KB

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// One LDS-DMA instruction: lane i moves 16 bytes from base + voff into LDS at
// lds_addr + 16 i.  Issued through inline asm (the builtin would make the
// compiler wait for every outstanding DMA before each LDS read); completion
// is tracked with explicit vmcnt waits.  base must be wave-uniform.
__device__ __forceinline__ void router_dma16(uint32_t lds_addr, const void* base, uint32_t voff) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  base = reinterpret_cast<const void*>((uint64_t)lo | ((uint64_t)hi << 32));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               ::"s"(lds_addr), "v"(voff), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// XOR swizzles of the 16-byte chunks of an LDS row: x rows are 128 bytes (two
// rows per 256-byte bank window), weight rows 256 bytes; 16 consecutive rows
// read at one logical chunk hit 16 distinct bank groups.
__device__ __forceinline__ int rswz_x(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int rswz_w(int r) { return r & 15; }

__global__ void __launch_bounds__(512)
router_lds_kernel(int64_t N, int D, int E, int parts, int vec4, const uint16_t* __restrict__ x,
                  const float* __restrict__ w, float* __restrict__ logits,
                  float* __restrict__ partials) {
  __shared__ uint4 lx[2][kRXU4];
  __shared__ uint4 lw[2][kRWU4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool split = partials != nullptr;
  const int ne = E / kRE;
  const int64_t tiles = ((N + kRT - 1) / kRT) * ne;
  const int64_t total = tiles * (split ? parts : 1);
  int64_t v = (int64_t)(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  if (v >= total) return;
  int part0 = 0, part1 = parts;
  if (split) {
    part0 = (int)(v % parts);
    part1 = part0 + 1;
    v /= parts;
  }
  const int64_t n0 = (v / ne) * kRT;
  const int e0 = (int)(v % ne) * kRE;
  const int r = lane & 31, kh = lane >> 5;
  const int nkb = D / kRBK;
  const uint32_t ax = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)&lx[0][0];
  const uint32_t aw = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)&lw[0][0];
  const uint16_t* xb = x + n0 * D;          // the tile's first token row
  const float* wb = w + (int64_t)e0 * D;    // the tile's first expert row
  // DMA lanes: x instruction q (2 per wave) moves tile rows 8q .. 8q+7, weight
  // instruction q (8 per wave) rows 4q .. 4q+3; the lane writing LDS chunk p
  // of row rr fetches global chunk p ^ swizzle(rr).  Rows past N or E read
  // the last row (their results are not stored).
  uint32_t offx[2], offw[8];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int q = wave * 2 + j, rr = q * 8 + (lane >> 3), p = lane & 7;
    const int row = (int)min<int64_t>(rr, N - 1 - n0);
    offx[j] = ((uint32_t)row * D + (uint32_t)(p ^ rswz_x(rr)) * 8) * 2u;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = wave * 8 + j, rr = q * 4 + (lane >> 4), p = lane & 15;
    const int row = min(rr, E - 1 - e0);
    offw[j] = ((uint32_t)row * D + (uint32_t)(p ^ rswz_w(rr)) * 4) * 4u;
  }
  auto dma = [&](int slot, int kb) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      router_dma16(ax + (uint32_t)slot * (kRXU4 * 16) + (uint32_t)(wave * 2 + j) * 1024, xb,
                   offx[j] + (uint32_t)kb * (kRBK * 2));
#pragma unroll
    for (int j = 0; j < 8; ++j)
      router_dma16(aw + (uint32_t)slot * (kRWU4 * 16) + (uint32_t)(wave * 8 + j) * 1024, wb,
                   offw[j] + (uint32_t)kb * (kRBK * 4));
  };

  for (int part = part0; part < part1; ++part) {
    const int kb0 = (int)((int64_t)part * nkb / parts), kb1 = (int)((int64_t)(part + 1) * nkb / parts);
    const int nk = kb1 - kb0;
    f32x16_t acc_hi[4], acc_lo[4];   // [token block] of this wave's expert block
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc_hi[j][q] = acc_lo[j][q] = 0.f;
    // every wave is past its LDS reads of the previous part
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    dma(0, kb0);
    if (nk > 1) {
      dma(1, kb0 + 1);
      asm volatile("s_waitcnt vmcnt(10)" ::: "memory");   // stage 0 landed
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    asm volatile("s_barrier" ::: "memory");
    for (int kt = 0; kt < nk; ++kt) {
      const uint4* sx = lx[kt & 1];
      const uint4* sw = lw[kt & 1];
#pragma unroll
      for (int ks = 0; ks < kRBK / 16; ++ks) {
        const int c = 2 * ks + kh;               // this lane's 8 k: chunk c of x, 2c and 2c+1 of w
        bf16x8_t xa[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rr = j * 32 + r;
          xa[j] = __builtin_bit_cast(bf16x8_t, sx[rr * 8 + (c ^ rswz_x(rr))]);
        }
        {
          const int rr = wave * 32 + r;
          const uint4 a = sw[rr * 16 + ((2 * c) ^ rswz_w(rr))];
          const uint4 b = sw[rr * 16 + ((2 * c + 1) ^ rswz_w(rr))];
          bf16x8_t hi, mid, lo;
          split3(__builtin_bit_cast(float4, a), __builtin_bit_cast(float4, b), hi, mid, lo);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc_hi[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, xa[j], acc_hi[j], 0, 0, 0);
            acc_lo[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mid, xa[j], acc_lo[j], 0, 0, 0);
            acc_lo[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, xa[j], acc_lo[j], 0, 0, 0);
          }
        }
      }
      // this wave is done with stage kt, and stage kt+1 has landed (nothing
      // was issued after it)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (kt + 1 < nk) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      asm volatile("s_barrier" ::: "memory");
      if (kt + 2 < nk) dma(kt & 1, kb0 + kt + 2);
    }
    // Block j: lane l, register q holds expert 8*(q/4) + 4*(l/32) + q%4 of
    // this wave's expert block and token l%32 of token block j.
    float* out = split ? partials + (size_t)part * N * E : logits;
    const bool add = !split && part > 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + j * 32 + r;
      if (n >= N) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int el = wave * 32 + 8 * g + 4 * kh;
        float vv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) vv[q] = acc_hi[j][4 * g + q] + acc_lo[j][4 * g + q];
        float* dst = out + n * E + e0 + el;
        if (vec4) {
          float4 o = make_float4(vv[0], vv[1], vv[2], vv[3]);
          if (add) {
            const float4 pv = *reinterpret_cast<const float4*>(dst);
            o = make_float4(pv.x + o.x, pv.y + o.y, pv.z + o.z, pv.w + o.w);
          }
          *reinterpret_cast<float4*>(dst) = o;
        } else {
          for (int q = 0; q < 4; ++q) dst[q] = add ? dst[q] + vv[q] : vv[q];
        }
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

// Parts of a split router: waves per 32x32 tile or k parts of the LDS
// tiles, both capped at 8.
constexpr int kMaxParts = 8;

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
  // Every load of the token goes out before the first use: the partials of
  // all its experts (part index clamped to nparts - 1, so no load sits behind
  // a branch), or its logits, and the bias.  The logit that a split router's
  // partials sum to (in part order) is written out and used as it is.
  // (without a bias the bias loads read the logits row instead, and are not used)
  const float* bsrc = bias ? bias : row;
  float lg[EPL], bv[EPL];
  // (with more than 256 experts, a group of 64 experts at a time: all groups
  // at once would not fit in registers)
  constexpr int JB = EPL <= 4 ? EPL : 1;
  if (partials) {
#pragma unroll
    for (int j0 = 0; j0 < EPL; j0 += JB) {
      float pv[JB][kMaxParts];
#pragma unroll
      for (int j = 0; j < JB; ++j)
#pragma unroll
        for (int q = 0; q < kMaxParts; ++q)
          pv[j][q] = partials[(size_t)min(q, nparts - 1) * N * E + n * E +
                              min(lane + 64 * (j0 + j), E - 1)];
#pragma unroll
      for (int j = 0; j < JB; ++j) bv[j0 + j] = bsrc[min(lane + 64 * (j0 + j), E - 1)];
#pragma unroll
      for (int j = 0; j < JB; ++j) {
        float v = pv[j][0];
#pragma unroll
        for (int q = 1; q < kMaxParts; ++q)
          if (q < nparts) v += pv[j][q];
        lg[j0 + j] = v;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      lg[j] = row[min(lane + 64 * j, E - 1)];
      bv[j] = bsrc[min(lane + 64 * j, E - 1)];
    }
  }
  uint64_t pk[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    pk[j] = 0;
    if (e < E) {
      if (partials) row[e] = lg[j];
      float key = lg[j];
      if (bias) key = key + bv[j];
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

// Router tiling.
//  - E a multiple of 256 and at least 1024 tokens: the LDS-staged kernel, 128
//    tokens x 256 experts per workgroup, k cut into `parts` parts so that the
//    launch has about one workgroup per CU of a 256-CU device (the part count
//    depends on the shape only, so the logits do too).
//  - else 64x64 tiles with 4 waves when they alone give the chip at least one
//    workgroup per CU; otherwise 32x32 tiles and as many waves per tile (up to
//    8, at most one per 64-deep k block) as bring the grid to about 512 waves.
struct RouterPlan {
  int kind;    // 0: 64x64 tiles, 1: 32x32 tiles, 2: LDS-staged 128 x 256 tiles
  int parts;   // kind 1: waves per tile; kind 2: k parts
};

bool router_lds_ok(const Dims& d) {
  return d.E % kRE == 0 && d.N >= 1024 && (uint64_t)d.E * d.D * 4 < (1ull << 32);
}

int router_lds_parts(const Dims& d) {
  const int nkb = d.D / kRBK;
  const int64_t tiles = ((d.N + kRT - 1) / kRT) * (d.E / kRE);
  int p = (int)((256 + tiles - 1) / tiles);
  if (p > kMaxParts) p = kMaxParts;
  if (p > nkb) p = nkb;
  if (p < 1) p = 1;
  return p;
}

// 32x32 tiles: waves per tile.
int router_waves32(const Dims& d) {
  const int nkb = d.D / 64;
  const int64_t t32 = ((d.N + 31) / 32) * ((d.E + 31) / 32);
  if (t32 <= 0) return 1;
  int S = (int)((512 + t32 - 1) / t32);
  if (S > kMaxParts) S = kMaxParts;
  if (S > nkb) S = nkb;
  if (S < 1) S = 1;
  return S;
}

RouterPlan router_plan(const Dims& d) {
  if (router_lds_ok(d)) return {2, router_lds_parts(d)};
  const int64_t t64 = ((d.N + 63) / 64) * ((d.E + 63) / 64);
  if (t64 >= device_cu_count()) return {0, 1};
  return {1, router_waves32(d)};
}

}  // namespace

// Sized without asking the device (workspace sizes are host-only): the 32x32
// tiles are taken only when the 64x64 ones number fewer than the CUs, and no
// device has more than 1024.
size_t router_ws_bytes(const Dims& d) {
  int S = 1;
  if (router_lds_ok(d)) {
    S = router_lds_parts(d);
  } else {
    const int64_t t64 = ((d.N + 63) / 64) * ((d.E + 63) / 64);
    if (t64 < 1024) S = router_waves32(d);
  }
  return S > 1 ? align_up((size_t)S * d.N * d.E * sizeof(float)) : 0;
}

hipError_t launch_router_gemm(const Dims& d, const uint16_t* x, const float* w, float* logits,
                              float* partials, hipStream_t s) {
  const int nkb = d.D / 64;
  // 16-byte stores of four logits when every row start is 16-byte aligned
  const int vec4 = (d.E % 4 == 0) && ((reinterpret_cast<uintptr_t>(logits) & 15u) == 0) &&
                   ((reinterpret_cast<uintptr_t>(partials) & 15u) == 0);
  const RouterPlan plan = router_plan(d);
  if (plan.kind == 2) {
    const int64_t tiles = ((d.N + kRT - 1) / kRT) * (d.E / kRE);
    const bool split = partials && plan.parts > 1;
    const int64_t wgs = tiles * (split ? plan.parts : 1);
    hipLaunchKernelGGL(router_lds_kernel, dim3((unsigned)((wgs + 7) / 8 * 8)), dim3(512), 0, s,
                       d.N, d.D, d.E, plan.parts, vec4, x, w, logits,
                       split ? partials : (float*)nullptr);
    return hipGetLastError();
  }
  if (plan.kind == 0) {
    // LDS: (S-1) partial tiles, at most 52 KB
    const int64_t t64 = ((d.N + 63) / 64) * ((d.E + 63) / 64);
    const int S64 = nkb < 4 ? nkb : 4;
    dim3 grid((unsigned)((t64 + 7) / 8 * 8));
    hipLaunchKernelGGL(router_mfma_kernel<64>, grid, dim3(64 * S64),
                       (S64 - 1) * 64 * 68 * sizeof(float), s, d.N, d.D, d.E, vec4, x, w,
                       logits, 0, (float*)nullptr);
    return hipGetLastError();
  }
  const int S = plan.parts;
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
  const RouterPlan plan = router_plan(d);
  const int nparts = partials && plan.kind != 0 ? plan.parts : 0;
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
