// Grouped SwiGLU expert FFN on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16).
//
// "MoE 推理完整机制" (zoe.im), 第二层 范式 A Step 2 and "关键 kernel: Grouped
// GEMM": every expert runs (m_e, D) -> (m_e, F) -> (m_e, D) and all experts'
// GEMMs of different sizes go through one launch, with compute units handed
// to experts dynamically (a hot expert simply owns more tiles).
//
// Two launches per layer, both of this kernel template:
//   gate/up : C = h [R, F],        A = x_perm [R, D], B = Wg[e], Wu[e] [F, D];
//             the tile holds matching gate and up columns, the epilogue
//             writes h = bf16(silu(g) * u).
//   down    : C = out_perm [R, D], A = h [R, F],      B = Wd[e] [D, F].
//
// Work list: expert e contributes ceil(m_e / BM) row tiles (m_e from
// expert_offsets, read on the device); every workgroup prefix-sums them into
// LDS at start-up, so no host synchronisation and no plan pass are needed.
// Tiles are ordered expert-major, then column panel, then row tile, so
// consecutive tiles share a weight panel.  The grid is
// persistent (a multiple of 8 workgroups); workgroup b runs on XCD b % 8 and
// each XCD walks its own contiguous eighth of the list, so the row tiles that
// share a weight panel hit the same L2.
//
// Tile: BM x BN x 64 (bf16), operands double-buffered in LDS with a 16-byte
// XOR swizzle (see swz) so the MFMA operand reads spread over all banks.
#include "common.h"

namespace moe {
namespace {

constexpr int BK = 64;           // k depth of one LDS stage (bf16)
constexpr int CHUNKS = BK / 8;   // 16-byte chunks per tile row

// LDS swizzle: chunk c of tile row r is stored at position c ^ swz(r).  A
// 128-byte tile row covers half of gfx950's 64 four-byte banks, so two
// consecutive rows share one 16-chunk bank window; swz(r) = (r >> 1) & 7 gives
// the 16 rows that one MFMA operand read touches per LDS cycle 16 distinct
// (row parity, chunk position) pairs, i.e. all 64 banks once.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

struct GemmArgs {
  const uint16_t* A;        // [rows, Kd]
  const uint16_t* B0;       // [E, NB0rows, Kd]  (gate or down weights)
  const uint16_t* B1;       // [E, NB0rows, Kd]  (up weights; gate/up only)
  uint16_t* C;              // [rows, Nout]
  const int32_t* offsets;   // [E+1]
  int E, Kd, Nout, n_tiles;
};

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.f + expf(-g)) * u;
}

// Global -> register loads of one stage: A rows, then B rows (gate or up matrix).
template <int NA, int NB_>
__device__ __forceinline__ void stage_gload(uint4 (&ra)[NA], uint4 (&rb)[NB_],
                                            const uint16_t* a_base, const uint32_t (&a_off)[NA],
                                            const uint16_t* b0_base, const uint16_t* b1_base,
                                            const uint32_t (&b_off)[NB_], uint32_t b_up, int k0) {
#pragma unroll
  for (int i = 0; i < NA; ++i) ra[i] = *reinterpret_cast<const uint4*>(a_base + a_off[i] + k0);
#pragma unroll
  for (int i = 0; i < NB_; ++i)
    rb[i] = *reinterpret_cast<const uint4*>(((b_up >> i) & 1 ? b1_base : b0_base) + b_off[i] + k0);
}

// Register -> LDS stores of one stage with the XOR swizzle.
template <int NA, int NB_, int RPP, int BM>
__device__ __forceinline__ void stage_lstore(uint4* st, const uint4 (&ra)[NA],
                                             const uint4 (&rb)[NB_], int lrow, int lchunk) {
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int r = lrow + i * RPP;
    st[r * CHUNKS + (lchunk ^ swz(r))] = ra[i];
  }
#pragma unroll
  for (int i = 0; i < NB_; ++i) {
    const int r = lrow + i * RPP;
    st[(BM + r) * CHUNKS + (lchunk ^ swz(r))] = rb[i];
  }
}

// MFMA over one LDS stage: BK/16 steps of 32x32x16 per (mb, nb) block.
template <int MB, int NB, int TM, int TN, int BM>
__device__ __forceinline__ void stage_mfma(f32x16_t (&acc)[MB][NB], const uint4* st, int wm,
                                           int wn, int lane) {
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    const int kc = ks * 2 + (lane >> 5);
    bf16x8_t af[MB], bfr[NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = wm * TM + mb * 32 + (lane & 31);
      af[mb] = __builtin_bit_cast(bf16x8_t, st[r * CHUNKS + (kc ^ swz(r))]);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int r = wn * TN + nb * 32 + (lane & 31);
      bfr[nb] = __builtin_bit_cast(bf16x8_t, st[(BM + r) * CHUNKS + (kc ^ swz(r))]);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[nb], af[mb], acc[mb][nb], 0, 0, 0);
  }
}

template <int BM, int BN, int WM, int WN, bool GATEUP>
__global__ void __launch_bounds__(64 * WM * WN)
grouped_gemm_kernel(GemmArgs p) {
  constexpr int NT = 64 * WM * WN;                // threads
  constexpr int TM = BM / WM, TN = BN / WN;       // wave tile
  constexpr int MB = TM / 32, NB = TN / 32;       // 32x32 MFMA blocks per wave
  static_assert(!GATEUP || NB % 2 == 0, "gate/up pairs");
  constexpr int RPP = NT / CHUNKS;                // tile rows loaded per pass
  constexpr int A_LD = BM / RPP;                  // 16-byte loads per thread per stage
  constexpr int B_LD = BN / RPP;
  static_assert(A_LD >= 1 && B_LD >= 1 && BM % RPP == 0 && BN % RPP == 0, "loader shape");

  __shared__ uint4 lds[2][(BM + BN) * CHUNKS];
  __shared__ int32_t mstart[1025];   // prefix sums of row tiles per expert

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lrow = tid / CHUNKS, lchunk = tid % CHUNKS;   // loader mapping

  // ---- work list: row tiles per expert from the offsets, prefix-summed by wave 0
  if (wave == 0) {
    const int per = (p.E + 63) / 64;
    const int e0 = lane * per;
    int local = 0;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < p.E) {
        const int m = p.offsets[e + 1] - p.offsets[e];
        local += m > 0 ? (m + BM - 1) / BM : 0;
      }
    }
    int incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(incl, d, 64);
      if (lane >= d) incl += t;
    }
    int run = incl - local;
    for (int i = 0; i < per; ++i) {
      const int e = e0 + i;
      if (e < p.E) {
        mstart[e] = run;
        const int m = p.offsets[e + 1] - p.offsets[e];
        run += m > 0 ? (m + BM - 1) / BM : 0;
      }
    }
    if (lane == 63) mstart[p.E] = incl;
  }
  __syncthreads();
  const int total = p.n_tiles * mstart[p.E];
  const int xcd = blockIdx.x & 7, P8 = gridDim.x >> 3, j = blockIdx.x >> 3;
  const int begin = (int)((int64_t)total * xcd / 8);
  const int end = (int)((int64_t)total * (xcd + 1) / 8);

  for (int l = begin + j; l < end; l += P8) {
    // ---- decode tile l -> (expert, row tile, column panel)
    int lo = 0, hi = p.E - 1;
    while (lo < hi) {            // last e with n_tiles * mstart[e] <= l
      const int mid = (lo + hi + 1) >> 1;
      if (p.n_tiles * mstart[mid] <= l) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int mt_e = mstart[e + 1] - mstart[e];
    const int idx = l - p.n_tiles * mstart[e];
    const int nt = idx / mt_e, mt = idx % mt_e;
    const int64_t row0 = (int64_t)p.offsets[e] + (int64_t)mt * BM;
    const int rows = min(BM, (int)(p.offsets[e + 1] - row0));

    // ---- this thread's load sources: 32-bit element offsets from per-tile bases
    const uint16_t* a_base = p.A + row0 * p.Kd + lchunk * 8;
    const size_t wmat = (size_t)p.Nout * p.Kd;      // elements of one expert's matrix
    const uint16_t* b0_base = p.B0 + (size_t)e * wmat + lchunk * 8;
    const uint16_t* b1_base = GATEUP ? p.B1 + (size_t)e * wmat + lchunk * 8 : b0_base;
    uint32_t a_off[A_LD], b_off[B_LD];
    uint32_t b_up = 0;                               // bit i: load i reads the up matrix
#pragma unroll
    for (int i = 0; i < A_LD; ++i) a_off[i] = (uint32_t)min(lrow + i * RPP, rows - 1) * p.Kd;
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int r = lrow + i * RPP;                  // tile row in [0, BN)
      int wrow;
      if (GATEUP) {
        const int q = r >> 5;                        // 32-row block: even = gate, odd = up
        wrow = nt * (BN / 2) + (q >> 1) * 32 + (r & 31);
        b_up |= (uint32_t)(q & 1) << i;
      } else {
        wrow = nt * BN + r;
      }
      b_off[i] = (uint32_t)min(wrow, p.Nout - 1) * p.Kd;
    }

    f32x16_t acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[mb][nb][v] = 0.f;

    uint4 ra[A_LD], rb[B_LD];
    const int nk = p.Kd / BK;
    // Stage 0 is rewritten below: wait until every wave is done with the
    // previous tile's last stage.
    __syncthreads();
    stage_gload(ra, rb, a_base, a_off, b0_base, b1_base, b_off, b_up, 0);
    stage_lstore<A_LD, B_LD, RPP, BM>(lds[0], ra, rb, lrow, lchunk);
    __syncthreads();
    for (int kt = 0; kt + 1 < nk; ++kt) {
      stage_gload(ra, rb, a_base, a_off, b0_base, b1_base, b_off, b_up, (kt + 1) * BK);
      stage_mfma<MB, NB, TM, TN, BM>(acc, lds[kt & 1], wm, wn, lane);
      stage_lstore<A_LD, B_LD, RPP, BM>(lds[(kt & 1) ^ 1], ra, rb, lrow, lchunk);
      __syncthreads();
    }
    stage_mfma<MB, NB, TM, TN, BM>(acc, lds[(nk - 1) & 1], wm, wn, lane);

    // ---- epilogue.  The MFMA ran with the weight tile as its first operand,
    //      so a 32x32 block holds C^T: lane l, register v has C row (l % 32)
    //      and C column 8*(v/4) + 4*(l/32) + v%4.  Four consecutive registers
    //      are four consecutive columns of one row: one 8-byte store.
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = wm * TM + mb * 32 + (lane & 31);
      if (r >= rows) continue;
      uint16_t* crow = p.C + (row0 + r) * p.Nout;
      if (GATEUP) {
#pragma unroll
        for (int pr = 0; pr < NB / 2; ++pr)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int f = nt * (BN / 2) + wn * (TN / 2) + pr * 32 + 8 * g + 4 * (lane >> 5);
            if (f >= p.Nout) continue;
            float hv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
              hv[q] = silu_mul(acc[mb][2 * pr][4 * g + q], acc[mb][2 * pr + 1][4 * g + q]);
            uint2 o;
            o.x = pack_bf16x2(hv[0], hv[1]);
            o.y = pack_bf16x2(hv[2], hv[3]);
            *reinterpret_cast<uint2*>(crow + f) = o;
          }
      } else {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = nt * BN + wn * TN + nb * 32 + 8 * g + 4 * (lane >> 5);
            if (n >= p.Nout) continue;
            uint2 o;
            o.x = pack_bf16x2(acc[mb][nb][4 * g + 0], acc[mb][nb][4 * g + 1]);
            o.y = pack_bf16x2(acc[mb][nb][4 * g + 2], acc[mb][nb][4 * g + 3]);
            *reinterpret_cast<uint2*>(crow + n) = o;
          }
      }
    }
  }
}

// Persistent grid: one workgroup per CU (two for the small-row tile), never
// more than the upper bound of tiles, rounded to a multiple of the 8 XCDs.
template <int BM, int BN, int WM, int WN, bool GATEUP>
hipError_t launch_one(const Dims& d, const GemmArgs& a, int occupancy, hipStream_t s) {
  const int64_t mt_max = d.padded ? (int64_t)d.E * ((d.cap + BM - 1) / BM)
                                  : (d.R + BM - 1) / BM + d.E;
  int64_t g = (int64_t)device_cu_count() * occupancy;
  const int64_t work = mt_max * a.n_tiles;
  if (g > work) g = work;
  g = (g + 7) / 8 * 8;
  hipLaunchKernelGGL((grouped_gemm_kernel<BM, BN, WM, WN, GATEUP>), dim3((unsigned)g),
                     dim3(64 * WM * WN), 0, s, a);
  return hipGetLastError();
}

// Row-tile height: 32 rows when experts average at most 48 rows (decode-like
// batches: the weight stream dominates), else 256.
inline bool small_rows(const Dims& d) { return (double)d.R / d.E <= 48.0; }

}  // namespace

size_t ffn_ws_bytes(const Dims& d) { return align_up((size_t)d.R * d.F * 2); }

hipError_t launch_expert_gateup(const Dims& d, const uint16_t* x_perm, const int32_t* offsets,
                                const uint16_t* wg, const uint16_t* wu, uint16_t* h,
                                hipStream_t s) {
  if (small_rows(d)) {
    GemmArgs a{x_perm, wg, wu, h, offsets, d.E, d.D, d.F, (d.F + 127) / 128};
    return launch_one<32, 256, 1, 4, true>(d, a, 2, s);
  }
  GemmArgs a{x_perm, wg, wu, h, offsets, d.E, d.D, d.F, (d.F + 127) / 128};
  return launch_one<256, 256, 2, 2, true>(d, a, 1, s);
}

hipError_t launch_expert_down(const Dims& d, const uint16_t* h, const int32_t* offsets,
                              const uint16_t* wd, uint16_t* out_perm, hipStream_t s) {
  GemmArgs a{h, wd, nullptr, out_perm, offsets, d.E, d.F, d.D, (d.D + 255) / 256};
  if (small_rows(d)) return launch_one<32, 256, 1, 4, false>(d, a, 2, s);
  return launch_one<256, 256, 2, 2, false>(d, a, 1, s);
}

hipError_t launch_grouped_ffn(const Dims& d, const uint16_t* x_perm, const int32_t* offsets,
                              const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                              uint16_t* out_perm, uint16_t* h, void* ws, hipStream_t s) {
  if (!h) h = static_cast<uint16_t*>(ws);
  hipError_t e = launch_expert_gateup(d, x_perm, offsets, wg, wu, h, s);
  if (e != hipSuccess) return e;
  return launch_expert_down(d, h, offsets, wd, out_perm, s);
}

}  // namespace moe
