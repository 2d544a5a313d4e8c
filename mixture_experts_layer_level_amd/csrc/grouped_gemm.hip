// Grouped SwiGLU expert FFN on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16).
//
// "MoE 推理完整机制" (zoe.im), 第二层 范式 A Step 2 and "关键 kernel: Grouped
// GEMM": every expert runs (m_e, D) -> (m_e, F) -> (m_e, D) and all experts'
// GEMMs of different sizes go through one launch, with compute units handed
// to experts dynamically (a hot expert simply owns more tiles).
//
// Two launches per layer, both of one kernel family:
//   gate/up : C = h [R, F],        A = x_perm [R, D], B = Wg[e], Wu[e] [F, D];
//             the tile holds matching gate and up columns, the epilogue
//             writes h = bf16(silu(g) * u).
//   down    : C = out_perm [R, D], A = h [R, F],      B = Wd[e] [D, F].
//
// Work list: expert e contributes ceil(m_e / BM) row tiles (m_e from
// expert_offsets, read on the device); every workgroup prefix-sums them into
// LDS at start-up, so no host synchronisation and no plan pass are needed.
// Tiles are ordered expert-major, then column panel, then row tile, so
// consecutive tiles share a weight panel.  The grid is persistent (a multiple
// of 8 workgroups); workgroup b runs on XCD b % 8 and each XCD walks its own
// contiguous eighth of the list, so the row tiles that share a weight panel
// meet in the same L2.
//
// Two kernels:
//   grouped_gemm_ring  (prefill-sized experts): operands go straight from
//     global memory into an S-stage LDS ring with LDS-DMA
//     (global_load_lds_dwordx4), BK-deep stages, one barrier per stage.  The
//     DMA for stage kt+S is issued right after the barrier of stage kt, when
//     every wave has read all of stage kt, behind the last MFMAs of stage kt;
//     the fragments of the first k-step of stage kt+1 are read from LDS while
//     those MFMAs run.
//   grouped_gemm_regs  (decode-sized experts, 32-row tiles): operands staged
//     through registers into a double-buffered LDS tile.
// Both accumulate k in the same order (ascending, 16 at a time), so they give
// bit-identical results.
#include "common.h"

namespace moe {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

struct GemmArgs {
  const uint16_t* A;        // [rows, Kd]
  const uint16_t* B0;       // [E, Nout, Kd]  (gate or down weights)
  const uint16_t* B1;       // [E, Nout, Kd]  (up weights; gate/up only)
  uint16_t* C;              // [rows, Nout]
  const int32_t* offsets;   // [E+1]
  int E, Kd, Nout, n_tiles;
};

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.f + expf(-g)) * u;
}

// LDS swizzle for BK-deep tile rows: 16-byte chunk c of row r is stored at
// c ^ swz(r).  A BK*2-byte row covers BK/2 of the 64 four-byte banks, so
// 128/BK consecutive rows share one bank window; consecutive windows get
// distinct XOR masks, so the 16 rows that one MFMA operand read serves per LDS
// cycle land on distinct banks.
template <int BK>
__device__ __forceinline__ int swz(int r) {
  return (r / (128 / BK)) % (BK / 8);
}

// Work list prologue (wave 0): mstart[e] = row tiles of experts before e,
// mstart[E] = all row tiles.
template <int BM>
__device__ __forceinline__ void build_work_list(const GemmArgs& p, int32_t* mstart, int lane) {
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

// Tile l -> (expert, column panel, first row, valid rows); all
// workgroup-uniform, kept in scalar registers.
struct Tile {
  int e, nt;
  int64_t row0;
  int rows;
};
template <int BM>
__device__ __forceinline__ Tile decode_tile(const GemmArgs& p, const int32_t* mstart, int l) {
  int lo = 0, hi = p.E - 1;
  while (lo < hi) {  // last e with n_tiles * mstart[e] <= l
    const int mid = (lo + hi + 1) >> 1;
    if (p.n_tiles * mstart[mid] <= l) lo = mid; else hi = mid - 1;
  }
  Tile t;
  t.e = __builtin_amdgcn_readfirstlane(lo);
  const int mt_e = __builtin_amdgcn_readfirstlane(mstart[t.e + 1] - mstart[t.e]);
  const int idx = l - p.n_tiles * __builtin_amdgcn_readfirstlane(mstart[t.e]);
  t.nt = idx / mt_e;
  const int mt = idx % mt_e;
  const int seg0 = __builtin_amdgcn_readfirstlane(p.offsets[t.e]);
  const int seg1 = __builtin_amdgcn_readfirstlane(p.offsets[t.e + 1]);
  t.row0 = (int64_t)seg0 + (int64_t)mt * BM;
  t.rows = min(BM, (int)(seg1 - t.row0));
  return t;
}

// Weight row of tile row r (r in [0, BN)) and whether it is an up row.  In
// gate/up tiles, 32-row block q holds gate rows for even q and the matching
// up rows for odd q, so each wave's pair of blocks covers the same 32 columns
// of h.
template <int BN, bool GATEUP>
__device__ __forceinline__ int weight_row(int nt, int r, bool& up) {
  if (GATEUP) {
    const int q = r >> 5;
    up = q & 1;
    return nt * (BN / 2) + (q >> 1) * 32 + (r & 31);
  }
  up = false;
  return nt * BN + r;
}

// Epilogue.  The MFMA ran with the weight tile as its first operand, so a
// 32x32 block holds C^T: lane l, register v has C row (l % 32) and C column
// 8*(v/4) + 4*(l/32) + v%4; four consecutive registers are four consecutive
// columns of one row, stored as one 8-byte write.
template <int MB, int NB, int TM, int TN, int BN, bool GATEUP>
__device__ __forceinline__ void store_tile(const GemmArgs& p, const Tile& t,
                                           const f32x16_t (&acc)[MB][NB], int wm, int wn,
                                           int lane) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = wm * TM + mb * 32 + (lane & 31);
    if (r >= t.rows) continue;
    uint16_t* crow = p.C + (t.row0 + r) * p.Nout;
    if (GATEUP) {
#pragma unroll
      for (int pr = 0; pr < NB / 2; ++pr)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int f = t.nt * (BN / 2) + wn * (TN / 2) + pr * 32 + 8 * g + 4 * (lane >> 5);
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
          const int n = t.nt * BN + wn * TN + nb * 32 + 8 * g + 4 * (lane >> 5);
          if (n >= p.Nout) continue;
          uint2 o;
          o.x = pack_bf16x2(acc[mb][nb][4 * g + 0], acc[mb][nb][4 * g + 1]);
          o.y = pack_bf16x2(acc[mb][nb][4 * g + 2], acc[mb][nb][4 * g + 3]);
          *reinterpret_cast<uint2*>(crow + n) = o;
        }
    }
  }
}

// MFMA fragments of one 16-deep k-step from an LDS stage of BM A rows
// followed by BN B rows, CH 16-byte chunks per row.
template <int MB, int NB, int TM, int TN, int BM, int BK>
__device__ __forceinline__ void read_frags(bf16x8_t (&af)[MB], bf16x8_t (&bfr)[NB],
                                           const uint4* st, int ks, int wm, int wn, int lane) {
  constexpr int CH = BK / 8;
  const int kc = ks * 2 + (lane >> 5);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = wm * TM + mb * 32 + (lane & 31);
    af[mb] = __builtin_bit_cast(bf16x8_t, st[r * CH + (kc ^ swz<BK>(r))]);
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int r = wn * TN + nb * 32 + (lane & 31);
    bfr[nb] = __builtin_bit_cast(bf16x8_t, st[(BM + r) * CH + (kc ^ swz<BK>(r))]);
  }
}

template <int MB, int NB>
__device__ __forceinline__ void mfma_step(f32x16_t (&acc)[MB][NB], const bf16x8_t (&af)[MB],
                                          const bf16x8_t (&bfr)[NB]) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[nb], af[mb], acc[mb][nb], 0, 0, 0);
}

template <int MB, int NB>
__device__ __forceinline__ void zero(f32x16_t (&acc)[MB][NB]) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][nb][v] = 0.f;
}

// ------------------------------------------------------------ LDS-DMA ring

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// One LDS-DMA instruction: each lane moves 16 bytes from base + voff into
// LDS at lds_addr + 16 * lane.  Issued through inline asm so that the
// compiler does not treat the in-flight LDS writes as aliasing every later
// LDS read (it would otherwise wait for all outstanding DMA before each
// ds_read); completion is tracked with the explicit vmcnt waits below.
// M0 is a reserved register (the compiler ignores it in a clobber list, hence
// the pragma); nothing else in these kernels reads or writes it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(uint32_t lds_addr, const uint16_t* base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               ::"s"(lds_addr), "v"(voff), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int BM, int BN, int WM, int WN, int BK, int S>
struct Ring {
  static constexpr int NW = WM * WN;
  static constexpr int TM = BM / WM, TN = BN / WN, MB = TM / 32, NB = TN / 32;
  static constexpr int CH = BK / 8;          // 16-byte chunks per tile row
  static constexpr int RPI = 64 / CH;        // tile rows per DMA instruction
  static constexpr int ROWS = BM + BN;
  static constexpr int PW = ROWS / RPI / NW; // DMA instructions per wave per stage
  static constexpr int KS = BK / 16;         // MFMA k-steps per stage
  static_assert(ROWS % (RPI * NW) == 0 && BM % RPI == 0 && 32 % RPI == 0, "DMA split");
  static_assert(PW * (S - 1) <= 63, "vmcnt range");
  static_assert((size_t)S * ROWS * BK * 2 + 4100 <= 160 * 1024, "LDS budget");
};

// Wait until at most n stages of this wave's DMA are still outstanding
// (n is clamped to the supported values; waiting for more is always safe).
template <int PW, int S>
__device__ __forceinline__ void wait_stages(int n) {
  if constexpr (S >= 4) {
    if (n >= 3) { wait_vmcnt<3 * PW>(); return; }
  }
  if constexpr (S >= 3) {
    if (n >= 2) { wait_vmcnt<2 * PW>(); return; }
  }
  if (n >= 1) { wait_vmcnt<PW>(); return; }
  wait_vmcnt<0>();
}

template <int BM, int BN, int WM, int WN, int BK, int S, bool GATEUP>
__global__ void __launch_bounds__(64 * WM * WN)
grouped_gemm_ring(GemmArgs p) {
  using R = Ring<BM, BN, WM, WN, BK, S>;
  constexpr int MB = R::MB, NB = R::NB, TM = R::TM, TN = R::TN;
  constexpr int CH = R::CH, RPI = R::RPI, PW = R::PW, KS = R::KS;
  __shared__ uint4 lds[S][R::ROWS * CH];
  __shared__ int32_t mstart[1025];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane / CH, lc = lane % CH;   // DMA: lane -> (row in group, LDS chunk)

  if (wave == 0) build_work_list<BM>(p, mstart, lane);
  __syncthreads();
  const int total = p.n_tiles * mstart[p.E];
  const int xcd = blockIdx.x & 7, P8 = gridDim.x >> 3, j0 = blockIdx.x >> 3;
  const int begin = (int)((int64_t)total * xcd / 8);
  const int end = (int)((int64_t)total * (xcd + 1) / 8);
  const int nk = p.Kd / BK;
  const size_t wmat = (size_t)p.Nout * p.Kd;     // elements of one expert's matrix

  for (int l = begin + j0; l < end; l += P8) {
    const Tile t = decode_tile<BM>(p, mstart, l);
    // DMA sources: instruction j of this wave moves tile rows g0..g0+RPI-1
    // (g0 wave-uniform) from base[j] + off[j]; the lane reading LDS chunk lc
    // of a row fetches global chunk lc ^ swz(row), which realises the swizzle.
    const uint16_t* base[PW];
    uint32_t off[PW];
#pragma unroll
    for (int j = 0; j < PW; ++j) {
      const int g0 = (wave * PW + j) * RPI;
      const int trow = (g0 < BM ? g0 : g0 - BM) + lr;
      const uint32_t gc = (uint32_t)(lc ^ swz<BK>(trow));
      if (g0 < BM) {
        base[j] = p.A + t.row0 * p.Kd;
        off[j] = (uint32_t)min(trow, t.rows - 1) * p.Kd + gc * 8;
      } else {
        bool up;
        const int wrow = weight_row<BN, GATEUP>(t.nt, g0 - BM, up) + lr;  // block of g0 holds all RPI rows
        base[j] = (up ? p.B1 : p.B0) + (size_t)t.e * wmat;
        off[j] = (uint32_t)min(wrow, p.Nout - 1) * p.Kd + gc * 8;
      }
    }
    auto dma = [&](int s, int kt) {
      const uint32_t l0 = (uint32_t)(uintptr_t)(lds_void_t*)&lds[s][0];
#pragma unroll
      for (int j = 0; j < PW; ++j)
        lds_dma16(__builtin_amdgcn_readfirstlane(l0 + (wave * PW + j) * 1024), base[j],
                  (off[j] + (uint32_t)(kt * BK)) * 2u);
    };

    f32x16_t acc[MB][NB];
    zero(acc);
    // every wave is past its last LDS read of the previous tile
    wait_lgkmcnt0();
    barrier();
#pragma unroll
    for (int s = 0; s < S; ++s)
      if (s < nk) dma(s, s);
    wait_stages<PW, S>(min(S - 1, nk - 1));
    barrier();
    bf16x8_t fa[2][MB], fb[2][NB];
    read_frags<MB, NB, TM, TN, BM, BK>(fa[0], fb[0], lds[0], 0, wm, wn, lane);
    for (int kt = 0; kt < nk; ++kt) {
      const uint4* cur = lds[kt % S];
#pragma unroll
      for (int ks = 0; ks + 1 < KS; ++ks) {
        read_frags<MB, NB, TM, TN, BM, BK>(fa[(ks + 1) & 1], fb[(ks + 1) & 1], cur, ks + 1, wm,
                                           wn, lane);
        mfma_step(acc, fa[ks & 1], fb[ks & 1]);
      }
      // this wave has read all of stage kt and its part of stage kt+1 landed
      wait_lgkmcnt0();
      if (kt + 1 < nk) wait_stages<PW, S>(min(S - 2, nk - 2 - kt));
      barrier();
      // The last k-step's MFMAs go first (their fragments are already in
      // registers), so the MFMA pipe does not idle while the DMA and the next
      // stage's fragment reads are issued; sched_barrier keeps that order.
      __builtin_amdgcn_sched_barrier(0);
      mfma_step(acc, fa[(KS - 1) & 1], fb[(KS - 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + S < nk) dma(kt % S, kt + S);
      if (kt + 1 < nk)
        read_frags<MB, NB, TM, TN, BM, BK>(fa[KS & 1], fb[KS & 1], lds[(kt + 1) % S], 0, wm, wn,
                                           lane);
    }
    store_tile<MB, NB, TM, TN, BN, GATEUP>(p, t, acc, wm, wn, lane);
  }
}

// ------------------------------------------------------------ register-staged

constexpr int RBK = 64;            // k depth of one LDS stage
constexpr int RCH = RBK / 8;       // 16-byte chunks per tile row

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

template <int NA, int NB_, int RPP, int BM>
__device__ __forceinline__ void stage_lstore(uint4* st, const uint4 (&ra)[NA],
                                             const uint4 (&rb)[NB_], int lrow, int lchunk) {
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int r = lrow + i * RPP;
    st[r * RCH + (lchunk ^ swz<RBK>(r))] = ra[i];
  }
#pragma unroll
  for (int i = 0; i < NB_; ++i) {
    const int r = lrow + i * RPP;
    st[(BM + r) * RCH + (lchunk ^ swz<RBK>(r))] = rb[i];
  }
}

template <int BM, int BN, int WM, int WN, bool GATEUP>
__global__ void __launch_bounds__(64 * WM * WN)
grouped_gemm_regs(GemmArgs p) {
  constexpr int NT = 64 * WM * WN;                // threads
  constexpr int TM = BM / WM, TN = BN / WN;       // wave tile
  constexpr int MB = TM / 32, NB = TN / 32;       // 32x32 MFMA blocks per wave
  static_assert(!GATEUP || NB % 2 == 0, "gate/up pairs");
  constexpr int RPP = NT / RCH;                   // tile rows loaded per pass
  constexpr int A_LD = BM / RPP;                  // 16-byte loads per thread per stage
  constexpr int B_LD = BN / RPP;
  static_assert(A_LD >= 1 && B_LD >= 1 && BM % RPP == 0 && BN % RPP == 0, "loader shape");

  __shared__ uint4 lds[2][(BM + BN) * RCH];
  __shared__ int32_t mstart[1025];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lrow = tid / RCH, lchunk = tid % RCH;   // loader mapping

  if (wave == 0) build_work_list<BM>(p, mstart, lane);
  __syncthreads();
  const int total = p.n_tiles * mstart[p.E];
  const int xcd = blockIdx.x & 7, P8 = gridDim.x >> 3, j0 = blockIdx.x >> 3;
  const int begin = (int)((int64_t)total * xcd / 8);
  const int end = (int)((int64_t)total * (xcd + 1) / 8);
  const size_t wmat = (size_t)p.Nout * p.Kd;

  for (int l = begin + j0; l < end; l += P8) {
    const Tile t = decode_tile<BM>(p, mstart, l);
    const uint16_t* a_base = p.A + t.row0 * p.Kd + lchunk * 8;
    const uint16_t* b0_base = p.B0 + (size_t)t.e * wmat + lchunk * 8;
    const uint16_t* b1_base = GATEUP ? p.B1 + (size_t)t.e * wmat + lchunk * 8 : b0_base;
    uint32_t a_off[A_LD], b_off[B_LD];
    uint32_t b_up = 0;                               // bit i: load i reads the up matrix
#pragma unroll
    for (int i = 0; i < A_LD; ++i) a_off[i] = (uint32_t)min(lrow + i * RPP, t.rows - 1) * p.Kd;
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      bool up;
      const int wrow = weight_row<BN, GATEUP>(t.nt, lrow + i * RPP, up);
      b_up |= (uint32_t)up << i;
      b_off[i] = (uint32_t)min(wrow, p.Nout - 1) * p.Kd;
    }

    f32x16_t acc[MB][NB];
    zero(acc);
    uint4 ra[A_LD], rb[B_LD];
    const int nk = p.Kd / RBK;
    // Stage 0 is rewritten below: wait until every wave is done with the
    // previous tile's last stage.
    __syncthreads();
    stage_gload(ra, rb, a_base, a_off, b0_base, b1_base, b_off, b_up, 0);
    stage_lstore<A_LD, B_LD, RPP, BM>(lds[0], ra, rb, lrow, lchunk);
    __syncthreads();
    for (int kt = 0; kt + 1 < nk; ++kt) {
      stage_gload(ra, rb, a_base, a_off, b0_base, b1_base, b_off, b_up, (kt + 1) * RBK);
      bf16x8_t af[MB], bfr[NB];
#pragma unroll
      for (int ks = 0; ks < RBK / 16; ++ks) {
        read_frags<MB, NB, TM, TN, BM, RBK>(af, bfr, lds[kt & 1], ks, wm, wn, lane);
        mfma_step(acc, af, bfr);
      }
      stage_lstore<A_LD, B_LD, RPP, BM>(lds[(kt & 1) ^ 1], ra, rb, lrow, lchunk);
      __syncthreads();
    }
    {
      bf16x8_t af[MB], bfr[NB];
#pragma unroll
      for (int ks = 0; ks < RBK / 16; ++ks) {
        read_frags<MB, NB, TM, TN, BM, RBK>(af, bfr, lds[(nk - 1) & 1], ks, wm, wn, lane);
        mfma_step(acc, af, bfr);
      }
    }
    store_tile<MB, NB, TM, TN, BN, GATEUP>(p, t, acc, wm, wn, lane);
  }
}

// ------------------------------------------------------------ launch

// Persistent grid: `occupancy` workgroups per CU, never more than the upper
// bound of tiles, rounded to a multiple of the 8 XCDs.
template <int BM>
int64_t grid_size(const Dims& d, int n_tiles, int occupancy) {
  const int64_t mt_max = d.padded ? (int64_t)d.E * ((d.cap + BM - 1) / BM)
                                  : (d.R + BM - 1) / BM + d.E;
  int64_t g = (int64_t)device_cu_count() * occupancy;
  const int64_t work = mt_max * n_tiles;
  if (g > work) g = work;
  return (g + 7) / 8 * 8;
}

template <int BM, int BN, int WM, int WN, int BK, int S, bool GATEUP>
hipError_t launch_ring(const Dims& d, const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((grouped_gemm_ring<BM, BN, WM, WN, BK, S, GATEUP>),
                     dim3((unsigned)grid_size<BM>(d, a.n_tiles, 1)), dim3(64 * WM * WN), 0, s, a);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, bool GATEUP>
hipError_t launch_regs(const Dims& d, const GemmArgs& a, int occupancy, hipStream_t s) {
  hipLaunchKernelGGL((grouped_gemm_regs<BM, BN, WM, WN, GATEUP>),
                     dim3((unsigned)grid_size<BM>(d, a.n_tiles, occupancy)), dim3(64 * WM * WN),
                     0, s, a);
  return hipGetLastError();
}

// Tile shape by the average number of rows per expert (R / E):
//   <= 48  : 32 x 256 register-staged tiles (decode: the weight stream rules)
//   <= 384 : 128 x 256 tiles, 4 waves, 64-deep stages, 3-stage ring
//   else   : 256 x 256 tiles, 8 waves, 32-deep stages, 4-stage ring
enum class Shape { Small, Mid, Large };
inline Shape pick(const Dims& d) {
  const double avg = (double)d.R / d.E;
  if (avg <= 48.0) return Shape::Small;
  if (avg <= 384.0) return Shape::Mid;
  return Shape::Large;
}

}  // namespace

size_t ffn_ws_bytes(const Dims& d) { return align_up((size_t)d.R * d.F * 2); }

hipError_t launch_expert_gateup(const Dims& d, const uint16_t* x_perm, const int32_t* offsets,
                                const uint16_t* wg, const uint16_t* wu, uint16_t* h,
                                hipStream_t s) {
  // every tile covers 128 columns of h (256 weight rows: 128 gate + 128 up)
  GemmArgs a{x_perm, wg, wu, h, offsets, d.E, d.D, d.F, (d.F + 127) / 128};
  switch (pick(d)) {
    case Shape::Small: return launch_regs<32, 256, 1, 4, true>(d, a, 2, s);
    case Shape::Mid: return launch_ring<128, 256, 2, 2, 64, 3, true>(d, a, s);
    default: return launch_ring<256, 256, 2, 4, 32, 4, true>(d, a, s);
  }
}

hipError_t launch_expert_down(const Dims& d, const uint16_t* h, const int32_t* offsets,
                              const uint16_t* wd, uint16_t* out_perm, hipStream_t s) {
  GemmArgs a{h, wd, nullptr, out_perm, offsets, d.E, d.F, d.D, (d.D + 255) / 256};
  switch (pick(d)) {
    case Shape::Small: return launch_regs<32, 256, 1, 4, false>(d, a, 2, s);
    case Shape::Mid: return launch_ring<128, 256, 2, 2, 64, 3, false>(d, a, s);
    default: return launch_ring<256, 256, 2, 4, 32, 4, false>(d, a, s);
  }
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
