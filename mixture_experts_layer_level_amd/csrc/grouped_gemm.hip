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
// Tiles are ordered expert-major; within an expert, row tiles go in bands of
// up to eight, and a band runs panel by panel with the row tile fastest, so
// consecutive tiles share a weight panel and nearby ones share A rows.  The
// grid is persistent (a multiple of 8 workgroups); workgroup b runs on XCD
// b % 8 and each XCD walks its own contiguous part of the list (of equal
// modelled cost, in whole rounds, for the 128- and 256-row tiles; of equal
// tile counts for the 32-row ones), so the row tiles that share a weight
// panel meet in the same L2.
//
// Three kernels:
//   grouped_gemm_split (256 x 256 tiles, bf16 weights, E <= 256): separate
//     LDS rings for the A rows (2 slots, one stage ahead) and the weight rows
//     (3 slots, two stages ahead), filled by LDS-DMA (global_load_lds_dwordx4)
//     whose instructions are spread over the stage's MFMAs; one barrier per
//     64-deep stage.
//   grouped_gemm_ring  (other prefill-sized tiles, FP8 weights): A and weight
//     rows of a stage share one slot of an S-stage LDS ring.  The DMA for
//     stage kt+S is issued right after the barrier of stage kt, when every
//     wave has read all of stage kt, behind the last MFMAs of stage kt; the
//     fragments of the first k-step of stage kt+1 are read from LDS while
//     those MFMAs run.
//   grouped_gemm_regs  (decode-sized experts, 32-row tiles): operands staged
//     through registers into a double-buffered LDS tile.
// All accumulate k in the same order (kchunk below), so they give
// bit-identical results.
//
// Block-scaled FP8 weights (FP8 = true; the FP8 weights of 第四层 DeepGEMM &
// MegaMoE Kernel): the weight operand arrives as E4M3 codes plus one E8M0
// scale byte per 32 k of a weight row and is dequantised on the way into the
// MFMA with v_cvt_scalef32_pk_bf16_fp8.  code * 2^s is exact in bf16, so the
// MFMAs see exactly the dequantised weights and the result is bit-identical to
// the bf16 kernel run on them; only the weight bytes read from memory halve.
// The register-staged kernel converts while staging into its bf16 LDS tile;
// the ring kernel moves codes and scales by LDS-DMA and converts each fragment
// after its LDS read.
//
// Scale layout: for weight rows [32 g, 32 g + 32) and k-block kb, the 32 scale
// bytes are contiguous at ((g * (Kd / 32)) + kb) * 32, so the scales of one
// 32-row group for consecutive k-blocks are one contiguous run.
#include "common.h"

namespace moe {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

struct GemmArgs {
  const uint16_t* A;        // [rows, Kd]
  const void* B0;           // [E, Nout, Kd] bf16 or E4M3 codes (gate or down weights)
  const void* B1;           // [E, Nout, Kd] (up weights; gate/up only)
  uint16_t* C;              // [rows, Nout]
  const int32_t* offsets;   // [E+1]
  int E, Kd, Nout, n_tiles;  // n_tiles: column tiles per expert (set by the launcher)
  const uint8_t* S0;        // FP8 only: scales of B0, [E, Nout/32, Kd/32, 32]
  const uint8_t* S1;        // FP8 only: scales of B1
  const float* bias;        // bias epilogues: [E, Nout] fp32
  const int32_t* gather;    // ring kernels: A row r is A[gather[r]] (NULL: A[r])
  int wpack;                // bf16 only: B0 holds the packed weight panels (B1 unused)
};

// Packed bf16 weights: for each expert e, column tile nt and 64-deep stage kt
// (in that order) the 32 KB image that a 256-row weight stage has in LDS.
// Byte 1024 q + 16 l of a stage image holds tile row 8 q + l / 8, chunk
// (l % 8) ^ swz(row) of its 64 k values, so every LDS-DMA instruction of a
// stage reads 1 KB of contiguous memory and a stage 32 KB: HBM streams long
// runs at a higher rate than 128-byte pieces of rows 2D bytes apart (on one
// MI355X: 4.83 TB/s for 128-byte pieces of 256 rows, 6.13 for 512-byte
// pieces, 6.35 for whole rows).  Gate/up panels hold the interleaved gate
// and up rows of weight_row.  Rows past Nout repeat the last row, as the
// unpacked DMA clamps them.
constexpr uint32_t kPackStage = 32768;   // bytes of one stage image (256 rows x 64 k)
__device__ __forceinline__ size_t packed_panel(const GemmArgs& p, int e, int nt, int nk) {
  return ((size_t)e * p.n_tiles + nt) * (size_t)nk * kPackStage;
}

// Epilogues: what a tile writes to C.
constexpr int kEpiSwiglu = 0;    // gate/up tile (interleaved Wg/Wu rows): bf16(silu(g) * u)
constexpr int kEpiStore = 1;     // bf16(acc)
constexpr int kEpiBiasGelu = 2;  // bf16(GELU(acc + bias)), GELU(v) = v * Phi(v)
constexpr int kEpiBias = 3;      // bf16(acc + bias)

// GELU(v) = v * Phi(v), Phi(v) = erfc(-v / sqrt 2) / 2.  erfc(z) for z >= 0
// by the Chebyshev-fitted formula of Numerical Recipes (Press et al., 2nd ed.,
// section 6.2, "erfcc"): erfc(z) = t exp(-z^2 + P(t)), t = 1 / (1 + z / 2), P
// a degree-9 polynomial, fractional error below 1.2e-7 for every z >= 0.  A
// relative bound keeps the far negative tail (Phi tiny) as accurate as the
// rest; the exponential is the hardware exp2.  For v >= 0, Phi = 1 - erfc/2.
__device__ __forceinline__ float gelu(float v) {
  const float z = fabsf(v) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.5f, z, 1.f));
  float p = 0.17087277f;
  p = __builtin_fmaf(p, t, -0.82215223f);
  p = __builtin_fmaf(p, t, 1.48851587f);
  p = __builtin_fmaf(p, t, -1.13520398f);
  p = __builtin_fmaf(p, t, 0.27886807f);
  p = __builtin_fmaf(p, t, -0.18628806f);
  p = __builtin_fmaf(p, t, 0.09678418f);
  p = __builtin_fmaf(p, t, 0.37409196f);
  p = __builtin_fmaf(p, t, 1.00002368f);
  p = __builtin_fmaf(p, t, -1.26551223f);
  const float half_erfc =
      0.5f * t * __builtin_amdgcn_exp2f((p - z * z) * 1.44269504088896341f);
  return v * (v >= 0.f ? 1.f - half_erfc : half_erfc);
}

// LDS swizzle for rows of RB bytes (16-byte chunks): chunk c of row r is stored
// at c ^ swz_rows<RB>(r).  256 / RB consecutive rows share one 256-byte bank
// window; consecutive windows get distinct XOR masks.
template <int RB>
__device__ __forceinline__ int swz_rows(int r) {
  return (r / (256 / RB)) % (RB / 16);
}

// Eight E4M3 codes (two dwords) times 2^(sbyte - 127) -> eight bf16 values;
// the scale operand of the conversion contributes only its exponent.
__device__ __forceinline__ bf16x8_t dequant8(uint32_t lo, uint32_t hi, float scale) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, true);
  return __builtin_bit_cast(bf16x8_t, make_uint4(__builtin_bit_cast(uint32_t, a),
                                                 __builtin_bit_cast(uint32_t, b),
                                                 __builtin_bit_cast(uint32_t, c),
                                                 __builtin_bit_cast(uint32_t, d)));
}

__device__ __forceinline__ float scale_of(uint32_t sbyte) { return __uint_as_float(sbyte << 23); }

// silu(g) * u = g u / (1 + e^-g), with the hardware exp2 and reciprocal (a
// few ulps of fp32, far below the bf16 rounding of h).  Large -g: e^-g = inf,
// the reciprocal 0, the result 0.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
  return g * u * __builtin_amdgcn_rcpf(1.f + e);
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

// Whether to fill a persistent launch's last round with extra row tiles
// (below): only when that round already holds at least an eighth of a round
// of tiles.  Every extra row tile streams its weight panels once more; with a
// nearly empty last round the extras cost more than the short tail they
// remove (DeepSeek-V3-shape down GEMM: 2.44 ms with them, 2.37 without, its
// last round holding 4 of 256 tiles), with a fuller one they pay (its gate/up
// GEMM, last round 44% full: 4.03 against 4.14 ms; the Mixtral-shape down
// GEMM, 25% full: 0.89 against 1.03 ms).
__device__ __forceinline__ bool fill_last_round(int64_t tiles, int grid) {
  const int64_t last = tiles - (tiles - 1) / grid * grid;   // tiles in the last round
  return last * 8 >= grid;
}

// Work list prologue (wave 0): mstart[e] = row tiles of experts before e,
// mstart[E] = all row tiles.  Expert e gets at least ceil(m_e / BM) row tiles.
// With grid > 0 (a launch of grid workgroups that each take every grid-th
// tile), spare tiles that would leave the last round partly empty are handed
// out as extra row tiles, one at a time, to the expert with the most 32-row
// blocks per row tile (never more row tiles than blocks): every workgroup then
// runs the same number of tiles, each with fewer rows.  A tile's results do
// not depend on its rows, so this changes no bit of the output.
template <int BM>
__device__ __forceinline__ void build_work_list(const GemmArgs& p, int32_t* mstart, int lane,
                                                int grid) {
  const int per = (p.E + 63) / 64;
  const int e0 = lane * per;
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < p.E) {
      const int m = p.offsets[e + 1] - p.offsets[e];
      const int mt = m > 0 ? (m + BM - 1) / BM : 0;
      mstart[e] = mt;
      local += mt;
    }
  }
  if (grid > 0) {
    int total = local;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) total += __shfl_xor(total, d, 64);
    const int64_t t0 = (int64_t)total * p.n_tiles;
    const int64_t rounds = (t0 + grid - 1) / grid;
    for (int64_t extra = fill_last_round(t0, grid) ? (rounds * grid - t0) / p.n_tiles : 0;
         extra > 0; --extra) {
      // this lane's candidate: most blocks per row tile, lower expert on ties
      int bb = 0, bt = 1, be = -1;
      for (int i = 0; i < per; ++i) {
        const int e = e0 + i;
        if (e < p.E) {
          const int nb = (p.offsets[e + 1] - p.offsets[e] + 31) / 32, mt = mstart[e];
          if (mt > 0 && mt < nb && (int64_t)nb * bt > (int64_t)bb * mt) {
            bb = nb;
            bt = mt;
            be = e;
          }
        }
      }
      // the wave's best (a total order: ratio, then expert id)
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) {
        const int ob = __shfl_xor(bb, d, 64), ot = __shfl_xor(bt, d, 64);
        const int oe = __shfl_xor(be, d, 64);
        const int64_t l = (int64_t)ob * bt, r = (int64_t)bb * ot;
        if (oe >= 0 && (be < 0 || l > r || (l == r && oe < be))) {
          bb = ob;
          bt = ot;
          be = oe;
        }
      }
      if (be < 0) break;                       // every expert has one block per tile
      if (be >= e0 && be < e0 + per) mstart[be] += 1;
    }
    local = 0;
    for (int i = 0; i < per; ++i)
      if (e0 + i < p.E) local += mstart[e0 + i];
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
      const int mt = mstart[e];
      mstart[e] = run;
      run += mt;
    }
  }
  if (lane == 63) mstart[p.E] = incl;
}

constexpr int kBand = 8;   // row tiles per band (see decode_tile)

// Tile l -> (expert, column panel, first row, valid rows); all
// workgroup-uniform, kept in scalar registers.
struct Tile {
  int e, nt;
  int64_t row0;
  int rows;
  int mtg;      // row tile over all experts: mstart[e] + row tile within the expert
};
// Tile l of expert e, whose row tiles are [ms_e, ms_e1) of the work list.
template <int BM>
__device__ __forceinline__ Tile tile_of(const GemmArgs& p, int e, int ms_e, int ms_e1, int l) {
  Tile t;
  t.e = e;
  const int mt_e = ms_e1 - ms_e;
  // Within an expert, row tiles go in bands of kBand and each band runs
  // panel by panel: the tiles an XCD runs at once then share both their A
  // rows and their weight panels in its L2 (with one band per expert, an
  // expert of many row tiles ran one panel over all of them and re-read its
  // A rows from HBM for every panel).
  const int idx = l - p.n_tiles * ms_e;
  const int band = idx / (kBand * p.n_tiles), mt0 = band * kBand;
  const int gb = min(kBand, mt_e - mt0), within = idx - band * kBand * p.n_tiles;
  t.nt = within / gb;
  const int mt = mt0 + within % gb;
  const int seg0 = __builtin_amdgcn_readfirstlane(p.offsets[t.e]);
  const int seg1 = __builtin_amdgcn_readfirstlane(p.offsets[t.e + 1]);
  // The expert's ceil(m / 32) row blocks are spread evenly over its mt_e row
  // tiles (each gets at most BM / 32 of them; only the expert's last block is
  // partial), so the row tiles that share a weight panel carry equal work and
  // stay in step through k, and little is computed past the last row.
  const int m = seg1 - seg0, nbk = (m + 31) / 32;
  const int b0 = (int)((int64_t)mt * nbk / mt_e), b1 = (int)((int64_t)(mt + 1) * nbk / mt_e);
  t.row0 = (int64_t)seg0 + 32 * b0;
  t.rows = min(32 * (b1 - b0), m - 32 * b0);
  t.mtg = ms_e + mt;
  return t;
}

template <int BM>
__device__ __forceinline__ Tile decode_tile(const GemmArgs& p, const int32_t* mstart, int l) {
  int lo = 0, hi = p.E - 1;
  while (lo < hi) {  // last e with n_tiles * mstart[e] <= l
    const int mid = (lo + hi + 1) >> 1;
    if (p.n_tiles * mstart[mid] <= l) lo = mid; else hi = mid - 1;
  }
  const int e = __builtin_amdgcn_readfirstlane(lo);
  return tile_of<BM>(p, e, __builtin_amdgcn_readfirstlane(mstart[e]),
                     __builtin_amdgcn_readfirstlane(mstart[e + 1]), l);
}

// The work list of build_work_list kept in registers instead of LDS: lane
// holds ms[i] = mstart[lane * PER + i] for the experts lane * PER + i < E
// (E <= 64 * PER); returns mstart[E], the number of row tiles.  Same row
// tiles, same extra tiles, same order as build_work_list.
template <int BM, int PER>
__device__ __forceinline__ int build_work_list_regs(const GemmArgs& p, int (&ms)[PER], int lane,
                                                    int grid) {
  const int e0 = lane * PER;
  int nbk[PER];      // 32-row blocks of each expert
  int local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = e0 + i;
    int mt = 0, nb = 0;
    if (e < p.E) {
      const int m = p.offsets[e + 1] - p.offsets[e];
      mt = m > 0 ? (m + BM - 1) / BM : 0;
      nb = (m + 31) / 32;
    }
    ms[i] = mt;
    nbk[i] = nb;
    local += mt;
  }
  if (grid > 0) {
    int total = local;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) total += __shfl_xor(total, d, 64);
    const int64_t t0 = (int64_t)total * p.n_tiles;
    const int64_t rounds = (t0 + grid - 1) / grid;
    for (int64_t extra = fill_last_round(t0, grid) ? (rounds * grid - t0) / p.n_tiles : 0;
         extra > 0; --extra) {
      int bb = 0, bt = 1, be = -1;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int nb = nbk[i], mt = ms[i];
        if (mt > 0 && mt < nb && (int64_t)nb * bt > (int64_t)bb * mt) {
          bb = nb;
          bt = mt;
          be = e0 + i;
        }
      }
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) {
        const int ob = __shfl_xor(bb, d, 64), ot = __shfl_xor(bt, d, 64);
        const int oe = __shfl_xor(be, d, 64);
        const int64_t l = (int64_t)ob * bt, r = (int64_t)bb * ot;
        if (oe >= 0 && (be < 0 || l > r || (l == r && oe < be))) {
          bb = ob;
          bt = ot;
          be = oe;
        }
      }
      if (be < 0) break;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (e0 + i == be) ms[i] += 1;
    }
    local = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) local += ms[i];
  }
  int incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(incl, d, 64);
    if (lane >= d) incl += t;
  }
  int run = incl - local;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int mt = ms[i];
    ms[i] = run;
    run += mt;
  }
  return __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
}

// XCD parts of about equal cost, in whole rounds.  A tile costs about
// kTileFixedBlocks 32-row blocks' worth of time whatever its rows plus its
// row blocks; an expert's tiles cost n_tiles * (kTileFixedBlocks * mt + nbk)
// in all.  The list is cut where the running cost crosses x/8 of the total
// (proportionally inside that expert), and each cut is then rounded to a
// multiple of the XCD's workgroup count, so that every workgroup of an XCD
// still runs the same number of tiles.  Which workgroup runs a tile changes
// no result.
constexpr int kTileFixedBlocks = 4;

// The cut for XCD x (x in [0, 8]) from this lane's experts: ms = their first
// row tile, mt = their row tiles, c = their cost, local = sum of c.
template <int N>
__device__ __forceinline__ int xcd_cut(int n_tiles, int total, const int (&ms)[N],
                                       const int (&mt)[N], const int (&c)[N], int64_t local,
                                       int lane, int x, int wgs) {
  int64_t incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t t = __shfl_up(incl, d, 64);
    if (lane >= d) incl += t;
  }
  const int64_t all = __shfl(incl, 63, 64);
  const int tiles = n_tiles * total;
  if (x >= 8 || all == 0) return x >= 8 ? tiles : 0;
  const int64_t T = all * x / 8;
  int64_t run = incl - local;
  int pos = -1;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (c[i] > 0 && run <= T && T < run + c[i])
      pos = n_tiles * ms[i] + (int)((T - run) * (int64_t)(n_tiles * mt[i]) / c[i]);
    run += c[i];
  }
  const uint64_t hit = __ballot(pos >= 0);
  pos = __shfl(pos, __ffsll((unsigned long long)hit) - 1, 64);
  return min(tiles, (pos + wgs / 2) / wgs * wgs);
}

// First tile of XCD x's part (x in [0, 8]) from the LDS work list of
// build_work_list (mstart[e], e <= E <= 1024); wgs: workgroups per XCD.
__device__ __forceinline__ int xcd_begin_lds(const GemmArgs& p, const int32_t* mstart, int lane,
                                             int x, int wgs) {
  constexpr int N = 16;                     // experts per lane, E <= 1024
  const int per = (p.E + 63) / 64;
  int ms[N], mt[N], c[N];
  int64_t local = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int e = lane * per + i;
    ms[i] = mt[i] = c[i] = 0;
    if (i < per && e < p.E) {
      ms[i] = mstart[e];
      mt[i] = mstart[e + 1] - mstart[e];
      c[i] = kTileFixedBlocks * mt[i] + (p.offsets[e + 1] - p.offsets[e] + 31) / 32;
      local += c[i];
    }
  }
  return xcd_cut<N>(p.n_tiles, mstart[p.E], ms, mt, c, local, lane, x, wgs);
}

// First tile of XCD x's part (x in [0, 8]) from the register work list of
// build_work_list_regs; wgs: workgroups per XCD.
template <int BM, int PER>
__device__ __forceinline__ int xcd_begin_regs(const GemmArgs& p, const int (&ms)[PER], int total,
                                              int lane, int x, int wgs) {
  const int e0 = lane * PER;
  const int next = __shfl_down(ms[0], 1, 64);           // mstart of the next lane's first
  int mt[PER], c[PER];
  int64_t local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = e0 + i;
    int nb = 0;
    if (e < p.E) nb = (p.offsets[e + 1] - p.offsets[e] + 31) / 32;
    const int ms1 = i + 1 < PER ? ms[i + 1] : (lane == 63 ? total : next);
    mt[i] = e < p.E ? (e + 1 < p.E ? ms1 : total) - ms[i] : 0;
    c[i] = kTileFixedBlocks * mt[i] + nb;
    local += c[i];
  }
  return xcd_cut<PER>(p.n_tiles, total, ms, mt, c, local, lane, x, wgs);
}

// mstart[e] from the registers of build_work_list_regs (e <= E, uniform).
template <int PER>
__device__ __forceinline__ int mstart_at(const int (&ms)[PER], int e, int E, int total) {
  if (e >= E) return total;
  // read every register of the owning lane, then pick one (selecting on
  // the per-lane array first would index it dynamically, in scratch)
  const int le = e / PER, ie = e % PER;
  int v = __builtin_amdgcn_readlane(ms[0], le);
#pragma unroll
  for (int i = 1; i < PER; ++i) {
    const int w = __builtin_amdgcn_readlane(ms[i], le);
    v = ie == i ? w : v;
  }
  return v;
}

template <int BM, int PER>
__device__ __forceinline__ Tile decode_tile_regs(const GemmArgs& p, const int (&ms)[PER],
                                                 int total, int lane, int l) {
  // experts with n_tiles * mstart[e] <= l; the last of them holds tile l
  int c = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    c += __builtin_popcountll(
        __ballot(lane * PER + i < p.E && p.n_tiles * ms[i] <= l));
  const int e = c - 1;
  return tile_of<BM>(p, e, mstart_at<PER>(ms, e, p.E, total),
                     mstart_at<PER>(ms, e + 1, p.E, total), l);
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
template <int MB, int NB, int TM, int TN, int BN, int EPI>
__device__ __forceinline__ void store_tile(const GemmArgs& p, const Tile& t,
                                           const f32x16_t (&acc)[MB][NB], int wm, int wn,
                                           int lane) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int r = wm * TM + mb * 32 + (lane & 31);
    if (r >= t.rows) continue;
    uint16_t* crow = p.C + (t.row0 + r) * p.Nout;
    if constexpr (EPI == kEpiSwiglu) {
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
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = acc[mb][nb][4 * g + q];
          if constexpr (EPI == kEpiBiasGelu || EPI == kEpiBias) {
            const float4 b = *reinterpret_cast<const float4*>(p.bias + (size_t)t.e * p.Nout + n);
            v[0] += b.x; v[1] += b.y; v[2] += b.z; v[3] += b.w;
          }
          if constexpr (EPI == kEpiBiasGelu) {
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = gelu(v[q]);
          }
          uint2 o;
          o.x = pack_bf16x2(v[0], v[1]);
          o.y = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<uint2*>(crow + n) = o;
        }
    }
  }
}

// k order of the MFMAs.  Each 32-deep k-block b takes two 16-deep k-steps;
// in k-step j the lanes of half h (lane / 32) hold the 8 values at
// 32 b + 16 h + 8 j.  So over the block's two k-steps a lane's values are one
// contiguous run of 16 (one 16-byte read of FP8 codes), and every kernel and
// tile depth accumulates k in this same order.  Returns the 8-value chunk of
// the stage row that a lane reads at k-step ks.
__device__ __forceinline__ int kchunk(int ks, int lane) {
  return 4 * (ks >> 1) + 2 * (lane >> 5) + (ks & 1);
}

// MFMA fragments of one 16-deep k-step from an LDS stage of BM A rows
// followed by BN B rows, CH 16-byte chunks per row.
template <int MB, int NB, int TM, int TN, int BM, int BK>
__device__ __forceinline__ void read_frags(bf16x8_t (&af)[MB], bf16x8_t (&bfr)[NB],
                                           const uint4* st, int ks, int wm, int wn, int lane) {
  constexpr int CH = BK / 8;
  const int kc = kchunk(ks, lane);
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

// One k-step of MFMAs; 32-row blocks mb >= nmb (wholly past the tile's last
// row) are skipped, which frees the SIMD's matrix pipe for the other waves.
template <int MB, int NB>
__device__ __forceinline__ void mfma_step(f32x16_t (&acc)[MB][NB], const bf16x8_t (&af)[MB],
                                          const bf16x8_t (&bfr)[NB], int nmb = MB) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
    if (mb < nmb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[mb][nb] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[nb], af[mb], acc[mb][nb], 0, 0, 0);
    }
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
// UNIFORM: the caller cannot show the compiler that base is wave-uniform
// (it is); read it from the first lane so that it is a scalar operand.
template <bool UNIFORM = false>
__device__ __forceinline__ void lds_dma16(uint32_t lds_addr, const void* base, uint32_t voff) {
  if constexpr (UNIFORM) {
    // readfirstlane returns int: go through uint32_t, which zero-extends
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    base = reinterpret_cast<const void*>((uint64_t)lo | ((uint64_t)hi << 32));
  }
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               ::"s"(lds_addr), "v"(voff), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int BM, int BN, int WM, int WN, int BK, int S_, bool FP8>
struct Ring {
  static constexpr int S = S_;
  static constexpr int NW = WM * WN;
  static constexpr int TM = BM / WM, TN = BN / WN, MB = TM / 32, NB = TN / 32;
  static constexpr int KS = BK / 16;                  // MFMA k-steps per stage
  static constexpr int CHA = BK / 8;                  // 16-byte chunks per A row
  static constexpr int BRB = FP8 ? BK : 2 * BK;       // bytes per B row
  static constexpr int CHB = BRB / 16;                // 16-byte chunks per B row
  static constexpr int RPIA = 64 / CHA, RPIB = 64 / CHB;   // rows per DMA instruction
  static constexpr int PWA = BM / RPIA / NW, PWB = BN / RPIB / NW;
  static constexpr int KB = BK / 32;                  // scale blocks per stage (FP8)
  static constexpr int LS = FP8 ? BN * KB / 16 / NW : 0;   // scale DMA lanes per wave
  static constexpr int GPW = FP8 ? LS / (2 * KB) : 0;      // 32-row groups per wave
  static constexpr int PW = PWA + PWB + (FP8 ? 1 : 0);     // DMA instructions per wave per stage
  static constexpr int A_U4 = BM * CHA, B_U4 = BN * CHB, S_U4 = FP8 ? BN * KB / 16 : 0;
  static constexpr int STAGE_U4 = A_U4 + B_U4 + S_U4;
  static_assert(PWA * RPIA * NW == BM && PWB * RPIB * NW == BN, "DMA split");
  static_assert(32 % RPIA == 0 && 32 % RPIB == 0, "one DMA instruction stays in a 32-row block");
  static_assert(!FP8 || (BK % 32 == 0 && LS * 16 * NW == BN * KB && GPW >= 1 &&
                         GPW * 2 * KB == LS && GPW * NW == BN / 32 && NW % 2 == 0),
                "scale DMA split");
  static_assert(PW * (S_ - 1) <= 63, "vmcnt range");
  static_assert((size_t)S_ * STAGE_U4 * 16 + 4100 <= 160 * 1024, "LDS budget");
};

// Wait until at most n stages of this wave's DMA are still outstanding
// (n is clamped to [0, N]; waiting for more is always safe).
template <int PW, int N>
__device__ __forceinline__ void wait_upto(int n) {
  if constexpr (N == 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= N) { wait_vmcnt<N * PW>(); return; }
    wait_upto<PW, N - 1>(n);
  }
}
template <int PW, int S>
__device__ __forceinline__ void wait_stages(int n) { wait_upto<PW, S - 1>(n); }

// Wait until at most n of this wave's DMA instructions are outstanding
// (n in [0, N]; waiting for fewer is always safe).
template <int N>
__device__ __forceinline__ void wait_vm_le(int n) {
  if constexpr (N == 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= N) { wait_vmcnt<N>(); return; }
    wait_vm_le<N - 1>(n);
  }
}

// FP8 scale area of a stage: wave w fetches LS 16-byte units, unit
// (i * KB + kbl) * 2 + half holding rows 16*half .. 16*half+15 of its i-th
// 32-row group for k-block kbl.  In gate/up tiles the first half of the waves
// fetch the gate groups (even tile groups) and the second half the up groups,
// so that each wave's fetch reads one matrix.  Returns the byte offset, within
// the scale area, of group g's k-block kbl.
template <class R, bool GATEUP>
__device__ __forceinline__ int scale_slot(int g, int kbl) {
  int w, i;
  if (GATEUP) {
    const int m = g & 1, gi = g >> 1;
    w = m * (R::NW / 2) + gi / R::GPW;
    i = gi % R::GPW;
  } else {
    w = g / R::GPW;
    i = g % R::GPW;
  }
  return (w * R::LS + (i * R::KB + kbl) * 2) * 16;
}

// MFMA fragments of k-step ks from a ring stage (A blocks mb >= nmb are not
// read).  bf16: A rows then B rows, swizzled 16-byte chunks.  FP8: on the
// first k-step of a 32-deep block each lane reads its 16 codes of the block
// (qb) and the block's scale of its row (sc); the two k-steps dequantise the
// first and second 8 of them.
template <class R, bool FP8, bool GATEUP>
__device__ __forceinline__ void read_frags_ring(bf16x8_t (&af)[R::MB], bf16x8_t (&bfr)[R::NB],
                                                float (&sc)[R::NB], uint4 (&qb)[R::NB],
                                                const uint4* st, int ks, int wm, int wn,
                                                int lane, int nmb) {
  constexpr int BK = R::CHA * 8;
  const int kc = kchunk(ks, lane);
#pragma unroll
  for (int mb = 0; mb < R::MB; ++mb) {
    const int r = wm * R::TM + mb * 32 + (lane & 31);
    if (mb < nmb) af[mb] = __builtin_bit_cast(bf16x8_t, st[r * R::CHA + (kc ^ swz<BK>(r))]);
  }
  if constexpr (!FP8) {
#pragma unroll
    for (int nb = 0; nb < R::NB; ++nb) {
      const int r = wn * R::TN + nb * 32 + (lane & 31);
      bfr[nb] = __builtin_bit_cast(bf16x8_t, st[R::A_U4 + r * R::CHB + (kc ^ swz<BK>(r))]);
    }
  } else {
    const uint8_t* stb = reinterpret_cast<const uint8_t*>(st + R::A_U4);
    const uint8_t* sts = reinterpret_cast<const uint8_t*>(st + R::A_U4 + R::B_U4);
    if (ks % 2 == 0) {
#pragma unroll
      for (int nb = 0; nb < R::NB; ++nb) {
        const int r = wn * R::TN + nb * 32 + (lane & 31);
        const int c = 2 * (ks >> 1) + (lane >> 5);    // 16-code chunk of this lane's half
        qb[nb] = *reinterpret_cast<const uint4*>(stb + r * R::BRB +
                                                 (c ^ swz_rows<R::BRB>(r)) * 16);
        sc[nb] = scale_of(sts[scale_slot<R, GATEUP>(wn * R::NB + nb, ks / 2) + (lane & 31)]);
      }
    }
#pragma unroll
    for (int nb = 0; nb < R::NB; ++nb)
      bfr[nb] = (ks & 1) ? dequant8(qb[nb].z, qb[nb].w, sc[nb])
                         : dequant8(qb[nb].x, qb[nb].y, sc[nb]);
  }
}

// The k loop of one ring tile, for a wave whose first NMB 32-row blocks hold
// rows of the tile (the MFMAs and A reads of the others are skipped; the
// wave still issues its DMA and meets every barrier).  The tile's first
// stages are already in flight or landed: stage 0 has landed and every wave
// has passed the barrier after it.
template <class R, int NMB, bool FP8, bool GATEUP, class Dma>
__device__ __forceinline__ void ring_kloop(f32x16_t (&acc)[R::MB][R::NB],
                                           uint4 (*lds)[R::STAGE_U4], int nk, int wm, int wn,
                                           int lane, const Dma& dma) {
  constexpr int MB = R::MB, NB = R::NB, PW = R::PW, KS = R::KS, S = R::S;
  bf16x8_t fa[2][MB], fb[2][NB];
  float sc[NB];
  uint4 qb[NB];
  read_frags_ring<R, FP8, GATEUP>(fa[0], fb[0], sc, qb, lds[0], 0, wm, wn, lane, NMB);
  for (int kt = 0; kt < nk; ++kt) {
    const uint4* cur = lds[kt % S];
#pragma unroll
    for (int ks = 0; ks + 1 < KS; ++ks) {
      read_frags_ring<R, FP8, GATEUP>(fa[(ks + 1) & 1], fb[(ks + 1) & 1], sc, qb, cur, ks + 1,
                                      wm, wn, lane, NMB);
      mfma_step(acc, fa[ks & 1], fb[ks & 1], NMB);
    }
    // this wave has read all of stage kt and its part of stage kt+1 landed
    wait_lgkmcnt0();
    if (kt + 1 < nk) wait_stages<PW, S>(min(S - 2, nk - 2 - kt));
    barrier();
    // The last k-step's MFMAs go first (their fragments are already in
    // registers), so the MFMA pipe does not idle while the DMA and the next
    // stage's fragment reads are issued; sched_barrier keeps that order.
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(acc, fa[(KS - 1) & 1], fb[(KS - 1) & 1], NMB);
    __builtin_amdgcn_sched_barrier(0);
    if (kt + S < nk) dma(kt % S, kt + S);
    if (kt + 1 < nk)
      read_frags_ring<R, FP8, GATEUP>(fa[KS & 1], fb[KS & 1], sc, qb, lds[(kt + 1) % S], 0, wm,
                                      wn, lane, NMB);
  }
}

// MFMAs [F, F + C) of one k-step, in mfma_step's (mb, nb) order.
template <int F, int C, int MB, int NB>
__device__ __forceinline__ void mfma_part(f32x16_t (&acc)[MB][NB], const bf16x8_t (&af)[MB],
                                          const bf16x8_t (&bfr)[NB], int nmb) {
#pragma unroll
  for (int i = F; i < F + C; ++i) {
    const int mb = i / NB, nb = i % NB;
    if (mb < nmb)
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[nb], af[mb], acc[mb][nb], 0, 0, 0);
  }
}

// MFMA group J of a k-step (C MFMAs), then DMA instruction J of stage kt
// into slot s (if `an`), in that order.
template <int J, int C, int MB, int NB, class Dma1>
__device__ __forceinline__ void mfma_dma_a(f32x16_t (&acc)[MB][NB], const bf16x8_t (&af)[MB],
                                           const bf16x8_t (&bfr)[NB], int nmb, bool an, int s,
                                           int kt, const Dma1& dma1) {
  mfma_part<J * C, C, MB, NB>(acc, af, bfr, nmb);
  __builtin_amdgcn_sched_barrier(0);
  if (an) dma1(s, kt, J);
  __builtin_amdgcn_sched_barrier(0);
}

// ring_kloop for rings of S >= 3 slots with the DMA spread over the stage
// instead of one burst after the barrier (a wave stalled behind a burst of
// DMA instructions issues no MFMAs).  The DMA of stage kt + S goes out in
// pieces: its first NPOST instructions between the quarters of the last
// k-step's MFMAs of stage kt, the others after the k-steps of stage kt + 1,
// Q per k-step.  Every instruction of stage kt + S is thus issued before the
// barrier that ends stage kt + 1, and when stage kt ends the DMA issued after
// stage kt + 1's is exactly that of stages kt + 2 .. kt + S - 1: the wait is
// ring_kloop's.
template <class R, int NMB, bool FP8, bool GATEUP, class Dma1>
__device__ __forceinline__ void ring_kloop_spread(f32x16_t (&acc)[R::MB][R::NB],
                                                  uint4 (*lds)[R::STAGE_U4], int nk, int wm,
                                                  int wn, int lane, const Dma1& dma1) {
  constexpr int MB = R::MB, NB = R::NB, PW = R::PW, KS = R::KS, S = R::S;
  constexpr int NPOST = 4, C = MB * NB / NPOST, Q = (PW - NPOST + KS - 2) / (KS - 1);
  static_assert(S >= 3 && C * NPOST == MB * NB && PW > NPOST, "DMA spread");
  bf16x8_t fa[2][MB], fb[2][NB];
  float sc[NB];
  uint4 qb[NB];
  read_frags_ring<R, FP8, GATEUP>(fa[0], fb[0], sc, qb, lds[0], 0, wm, wn, lane, NMB);
  int sp = S - 1;   // slot of stage kt + S - 1, whose DMA this step's k-steps finish
  for (int kt = 0; kt < nk; ++kt) {
    const int s0 = kt % S;
    const uint4* cur = lds[s0];
    const bool bdef = kt + S - 1 < nk;
#pragma unroll
    for (int ks = 0; ks + 1 < KS; ++ks) {
      read_frags_ring<R, FP8, GATEUP>(fa[(ks + 1) & 1], fb[(ks + 1) & 1], sc, qb, cur, ks + 1,
                                      wm, wn, lane, NMB);
      mfma_step(acc, fa[ks & 1], fb[ks & 1], NMB);
      if (bdef && NPOST + ks * Q < PW) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < Q; ++q)
          if (NPOST + ks * Q + q < PW) dma1(sp, kt + S - 1, NPOST + ks * Q + q);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // this wave has read all of stage kt and its part of stage kt+1 landed
    wait_lgkmcnt0();
    if (kt + 1 < nk) wait_stages<PW, S>(min(S - 2, nk - 2 - kt));
    barrier();
    __builtin_amdgcn_sched_barrier(0);
    const bool an = kt + S < nk;
    const bf16x8_t(&fl)[MB] = fa[(KS - 1) & 1];
    const bf16x8_t(&gl)[NB] = fb[(KS - 1) & 1];
    mfma_dma_a<0, C>(acc, fl, gl, NMB, an, s0, kt + S, dma1);
    mfma_dma_a<1, C>(acc, fl, gl, NMB, an, s0, kt + S, dma1);
    mfma_dma_a<2, C>(acc, fl, gl, NMB, an, s0, kt + S, dma1);
    mfma_dma_a<3, C>(acc, fl, gl, NMB, an, s0, kt + S, dma1);
    sp = s0;
    if (kt + 1 < nk)
      read_frags_ring<R, FP8, GATEUP>(fa[KS & 1], fb[KS & 1], sc, qb, lds[(kt + 1) % S], 0, wm,
                                      wn, lane, NMB);
  }
}

template <class R, int N, bool FP8, bool GATEUP, class Dma1>
__device__ __forceinline__ void ring_kloop_spread_n(int nmb, f32x16_t (&acc)[R::MB][R::NB],
                                                    uint4 (*lds)[R::STAGE_U4], int nk, int wm,
                                                    int wn, int lane, const Dma1& dma1) {
  if constexpr (N == 0) {
    ring_kloop_spread<R, 0, FP8, GATEUP>(acc, lds, nk, wm, wn, lane, dma1);
  } else {
    if (nmb == N) ring_kloop_spread<R, N, FP8, GATEUP>(acc, lds, nk, wm, wn, lane, dma1);
    else ring_kloop_spread_n<R, N - 1, FP8, GATEUP>(nmb, acc, lds, nk, wm, wn, lane, dma1);
  }
}

// ring_kloop with NMB = nmb, chosen outside the loop so that the loop body
// holds no branch on it.
template <class R, int N, bool FP8, bool GATEUP, class Dma>
__device__ __forceinline__ void ring_kloop_n(int nmb, f32x16_t (&acc)[R::MB][R::NB],
                                             uint4 (*lds)[R::STAGE_U4], int nk, int wm, int wn,
                                             int lane, const Dma& dma) {
  if constexpr (N == 0) {
    ring_kloop<R, 0, FP8, GATEUP>(acc, lds, nk, wm, wn, lane, dma);
  } else {
    if (nmb == N) ring_kloop<R, N, FP8, GATEUP>(acc, lds, nk, wm, wn, lane, dma);
    else ring_kloop_n<R, N - 1, FP8, GATEUP>(nmb, acc, lds, nk, wm, wn, lane, dma);
  }
}

// One tile of the ring kernel: its operands through the LDS ring, the k loop
// and the epilogue.  Every wave of the workgroup takes part; on return each
// wave has issued its stores of the tile.
template <int BM, int BN, int WM, int WN, int BK, int S, int EPI, bool FP8, bool UNIFORM = false,
          bool SPREAD = false>
__device__ __forceinline__ void ring_tile(const GemmArgs& p, const Tile& t,
                                          uint4 (*lds)[Ring<BM, BN, WM, WN, BK, S, FP8>::STAGE_U4],
                                          uint32_t lds_addr, int wave, int lane) {
  constexpr bool GATEUP = EPI == kEpiSwiglu;
  using R = Ring<BM, BN, WM, WN, BK, S, FP8>;
  constexpr int MB = R::MB, NB = R::NB;
  constexpr int PWA = R::PWA, PWB = R::PWB, PW = R::PW;
  const int wm = wave / WN, wn = wave % WN;
  // DMA lane roles: lane -> (row in its instruction's group, LDS chunk)
  const int lra = lane / R::CHA, lca = lane % R::CHA;
  const int lrb = lane / R::CHB, lcb = lane % R::CHB;
  const int nk = p.Kd / BK;
  const size_t wmat = (size_t)p.Nout * p.Kd;     // elements of one expert's matrix
  // DMA sources: instruction j moves 1 KB into LDS at byte ldso[j] of the
  // stage from base[j] + off[j] (+ the per-stage advance); the lane writing
  // LDS chunk c of a row fetches global chunk c ^ swizzle(row), which
  // realises the swizzle.  Instructions [0, PWA) carry A rows, [PWA,
  // PWA + PWB) B rows and, for FP8, the last one (lanes < LS only) scales.
  const void* base[PW];
  uint32_t off[PW], ldso[PW];
  // packed FP8 codes read by 64-deep stages: two stages per 128-deep stage
  // image; dlt = where a lane's piece of an odd stage sits relative to that
  // of the even stage before it
  const bool pk64 = FP8 && BK == 64 && p.wpack;
  uint32_t dlt[PWB];
#pragma unroll
  for (int j = 0; j < PWA; ++j) {
    const int q = wave * PWA + j;
    const int trow = q * R::RPIA + lra;
    const int row = min(trow, t.rows - 1);
    // gathered A: row r of the tile is row gather[row0 + r] of A
    const uint32_t src = p.gather ? (uint32_t)p.gather[t.row0 + row] : (uint32_t)row;
    base[j] = p.gather ? p.A : p.A + t.row0 * p.Kd;
    off[j] = (src * p.Kd + (uint32_t)(lca ^ swz<BK>(trow)) * 8) * 2u;
    ldso[j] = q * 1024;
  }
#pragma unroll
  for (int jb = 0; jb < PWB; ++jb) {
    const int q = wave * PWB + jb;
    const int g0 = q * R::RPIB, trow = g0 + lrb;
    bool up;
    const int wrow = min(weight_row<BN, GATEUP>(t.nt, g0, up) + lrb, p.Nout - 1);
    const char* b = static_cast<const char*>(up ? p.B1 : p.B0);
    if constexpr (!FP8) {
      static_assert(R::B_U4 * 16 == kPackStage && R::RPIB * R::CHB == 64, "packed stage image");
    } else {
      static_assert(BN == 256 && (BK == 64 || BK == 128), "packed FP8 stage image");
    }
    dlt[jb] = 0;
    if (!FP8 && p.wpack) {
      base[PWA + jb] = static_cast<const char*>(p.B0) + packed_panel(p, t.e, t.nt, nk);
      off[PWA + jb] = q * 1024 + lane * 16;
    } else if (FP8 && p.wpack) {
      // stage images of 256 rows x 128 codes: row r at byte 128 r, its
      // 16-byte chunk c at position c ^ ((r / 2) % 8)
      base[PWA + jb] = static_cast<const char*>(p.B0) + packed_panel(p, t.e, t.nt, p.Kd / 128);
      if (BK == 128) {
        off[PWA + jb] = q * 1024 + lane * 16;
      } else {
        // LDS chunk lcb of this 64-code row holds chunk g of the row's 64
        // codes of the stage: chunk g (even stage) or 4 + g (odd stage) of
        // the image row
        const int g = lcb ^ swz_rows<R::BRB>(trow), sw = (trow >> 1) & 7;
        off[PWA + jb] = (uint32_t)(trow * 128 + ((g ^ sw) << 4));
        dlt[jb] = (uint32_t)(trow * 128 + (((4 + g) ^ sw) << 4)) - off[PWA + jb];
      }
    } else if (FP8) {
      base[PWA + jb] = b + (size_t)t.e * wmat;
      off[PWA + jb] = (uint32_t)wrow * p.Kd + (uint32_t)(lcb ^ swz_rows<R::BRB>(trow)) * 16;
    } else {
      base[PWA + jb] = b + (size_t)t.e * wmat * 2;
      off[PWA + jb] = ((uint32_t)wrow * p.Kd + (uint32_t)(lcb ^ swz<BK>(trow)) * 8) * 2u;
    }
    ldso[PWA + jb] = R::A_U4 * 16 + q * 1024;
  }
  if constexpr (FP8) {
    const int lam = min(lane, R::LS - 1);
    const int half = lam & 1, kbl = (lam >> 1) % R::KB, i = (lam >> 1) / R::KB;
    int m = 0, rg;
    if (GATEUP) {
      m = wave / (R::NW / 2);
      rg = t.nt * (BN / 64) + (wave % (R::NW / 2)) * R::GPW + i;
    } else {
      rg = t.nt * (BN / 32) + wave * R::GPW + i;
    }
    rg = min(rg, p.Nout / 32 - 1);
    base[PW - 1] = (m ? p.S1 : p.S0) + (size_t)t.e * (wmat / 32);
    off[PW - 1] = ((uint32_t)rg * (uint32_t)(p.Kd / 32) + kbl) * 32 + half * 16;
    ldso[PW - 1] = (R::A_U4 + R::B_U4) * 16 + wave * R::LS * 16;
  }
  // lds_addr: LDS byte address of lds[0][0] (taken where the array is
  // declared, so no generic-pointer conversion is needed here)
  // per-stage advance of a weight DMA source (a packed stage image, or BRB
  // bytes of a row)
  const uint32_t badv = p.wpack ? kPackStage : R::BRB;
  // source offset of DMA instruction j for stage kt
  auto src_off = [&](int j, int kt) -> uint32_t {
    if (j < PWA) return off[j] + (uint32_t)kt * (BK * 2);
    if (j >= PWA + PWB) return off[j] + (uint32_t)kt * (R::KB * 32);
    if (pk64)
      return off[j] + (uint32_t)(kt >> 1) * kPackStage + ((kt & 1) ? dlt[j - PWA] : 0u);
    return off[j] + (uint32_t)kt * badv;
  };
  auto dma = [&](int s, int kt) {
    const uint32_t l0 = lds_addr + (uint32_t)s * (R::STAGE_U4 * 16);
#pragma unroll
    for (int j = 0; j < PW; ++j) {
      const uint32_t la = __builtin_amdgcn_readfirstlane(l0 + ldso[j]);
      if (FP8 && j == PW - 1) {
        if (lane < R::LS) lds_dma16<UNIFORM>(la, base[j], src_off(j, kt));
      } else {
        lds_dma16<UNIFORM>(la, base[j], src_off(j, kt));
      }
    }
  };

  f32x16_t acc[MB][NB];
  zero(acc);
  // every wave is past its last LDS read of the previous tile
  wait_lgkmcnt0();
  barrier();
  // 32-row blocks of this wave that hold at least one row of the tile
  const int nmb = min(MB, max(0, (t.rows - wm * R::TM + 31) / 32));
  if constexpr (SPREAD) {
    // instruction j of the DMA set alone (the callers pass constants once
    // unrolled)
    auto dma1 = [&](int s, int kt, int j) {
      const uint32_t l0 = lds_addr + (uint32_t)s * (R::STAGE_U4 * 16);
#pragma unroll
      for (int i = 0; i < PW; ++i) {
        if (i != j) continue;
        const uint32_t la = __builtin_amdgcn_readfirstlane(l0 + ldso[i]);
        if (FP8 && i == PW - 1) {
          if (lane < R::LS) lds_dma16<UNIFORM>(la, base[i], src_off(i, kt));
        } else {
          lds_dma16<UNIFORM>(la, base[i], src_off(i, kt));
        }
      }
    };
    // prologue in the loop's issue order: stages 0 .. S-2 whole, stage S-1's
    // first four instructions (step 0's k-steps issue the rest); then stage
    // 0 has landed once at most the later ones are outstanding
#pragma unroll
    for (int s = 0; s + 1 < S; ++s)
      if (s < nk) dma(s, s);
    if (S - 1 < nk)
#pragma unroll
      for (int j = 0; j < 4; ++j) dma1(S - 1, S - 1, j);
    wait_vm_le<(S - 2) * PW + 4>(min(S - 2, nk - 1) * PW + (S - 1 < nk ? 4 : 0));
    barrier();
    ring_kloop_spread_n<R, MB, FP8, GATEUP>(nmb, acc, lds, nk, wm, wn, lane, dma1);
    store_tile<MB, NB, R::TM, R::TN, BN, EPI>(p, t, acc, wm, wn, lane);
    return;
  }
#pragma unroll
  for (int s = 0; s < S; ++s)
    if (s < nk) dma(s, s);
  wait_stages<PW, S>(min(S - 1, nk - 1));
  barrier();
  ring_kloop_n<R, MB, FP8, GATEUP>(nmb, acc, lds, nk, wm, wn, lane, dma);
  store_tile<MB, NB, R::TM, R::TN, BN, EPI>(p, t, acc, wm, wn, lane);
}

template <int BM, int BN, int WM, int WN, int BK, int S, int EPI, bool FP8, bool SPREAD = false>
__global__ void __launch_bounds__(64 * WM * WN)
grouped_gemm_ring(GemmArgs p) {
  using R = Ring<BM, BN, WM, WN, BK, S, FP8>;
  __shared__ uint4 lds[S][R::STAGE_U4];
  __shared__ int32_t mstart[1025];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(lds_void_t*)&lds[0][0];
  if (wave == 0) build_work_list<BM>(p, mstart, lane, gridDim.x);
  __syncthreads();
  const int xcd = blockIdx.x & 7, P8 = gridDim.x >> 3, j0 = blockIdx.x >> 3;
  // Prefill tiles: XCD parts of equal cost in whole rounds (the same value in
  // every lane; readfirstlane lets the compiler see it).  Decode tiles all
  // cost the same and keep parts of equal counts (the cost cut, rounded to
  // whole rounds, put every XCD exactly 16 experts apart and made the decode
  // gate/up GEMM 14% slower).
  int begin, end;
  if constexpr (BM >= 128) {
    begin = __builtin_amdgcn_readfirstlane(xcd_begin_lds(p, mstart, lane, xcd, P8));
    end = __builtin_amdgcn_readfirstlane(xcd_begin_lds(p, mstart, lane, xcd + 1, P8));
  } else {
    const int total = p.n_tiles * __builtin_amdgcn_readfirstlane(mstart[p.E]);
    begin = (int)((int64_t)total * xcd / 8);
    end = (int)((int64_t)total * (xcd + 1) / 8);
  }
  for (int l = begin + j0; l < end; l += P8)
    ring_tile<BM, BN, WM, WN, BK, S, EPI, FP8, false, SPREAD>(p, decode_tile<BM>(p, mstart, l),
                                                              lds, lds_addr, wave, lane);
}

// ------------------------------------------------------------ split ring
//
// In the ring above a stage's A rows and weight rows share one LDS slot; at
// 256 x 256 tiles two slots fill LDS, so the DMA for stage kt+2 has to be
// issued as soon as stage kt's slot frees, in one burst.  The split ring
// keeps two rings: SA = 2 slots of A rows, one stage ahead (A rows are mostly
// L2 hits: every column panel of a row tile reads them), and SB slots of
// weight rows, SB - 1 stages ahead.  The weights' extra stage of slack is
// what lets their DMA be spread over the next stage's k-steps (split_kloop);
// the deeper ring alone gained little.  The rings fill LDS, so the work
// list's row-tile prefix is kept in registers (build_work_list_regs).  Same
// tiles, same MFMAs in the same k order as the ring kernel: the results are
// bit-identical.
template <int BM, int BN, int WM, int WN, int BK, int SB_>
struct Split {
  using R = Ring<BM, BN, WM, WN, BK, 2, false>;   // tile geometry and DMA split
  static constexpr int SA = 2, SB = SB_;
  static constexpr int A_BYTES = R::A_U4 * 16, B_BYTES = R::B_U4 * 16;
  static_assert(SA * A_BYTES + SB * B_BYTES <= 160 * 1024, "LDS budget");
  static_assert(SB >= 3 && 2 * R::PWB + R::PWA <= 63, "vmcnt range");
};

// MFMA fragments of k-step ks from an A slot and a weight slot (bf16; A
// blocks mb >= nmb are not read).
template <class R>
__device__ __forceinline__ void read_frags_split(bf16x8_t (&af)[R::MB], bf16x8_t (&bfr)[R::NB],
                                                 const uint4* sa, const uint4* sb, int ks, int wm,
                                                 int wn, int lane, int nmb) {
  constexpr int BK = R::CHA * 8;
  const int kc = kchunk(ks, lane);
#pragma unroll
  for (int mb = 0; mb < R::MB; ++mb) {
    const int r = wm * R::TM + mb * 32 + (lane & 31);
    if (mb < nmb) af[mb] = __builtin_bit_cast(bf16x8_t, sa[r * R::CHA + (kc ^ swz<BK>(r))]);
  }
#pragma unroll
  for (int nb = 0; nb < R::NB; ++nb) {
    const int r = wn * R::TN + nb * 32 + (lane & 31);
    bfr[nb] = __builtin_bit_cast(bf16x8_t, sb[r * R::CHB + (kc ^ swz<BK>(r))]);
  }
}

// The k loop of a split-ring tile.  Stage kt's A rows are in A slot kt % 2,
// its weight rows in weight slot kt % SB.  The DMA is spread over the stage
// instead of being issued in one burst after the barrier: a CU's texture
// path takes about as long to accept one stage's 64 DMA instructions as the
// matrix cores take to compute half a stage, and a wave stalled behind its
// DMA issues no MFMAs (issued in one burst, a 256 x 256 tile's stage took
// 8-10% longer).
//   - After the barrier that ends stage kt, A slot kt % 2 and weight slot
//     kt % SB are free.  The last k-step's MFMAs of stage kt go first, each
//     quarter followed by one of the wave's PWA A instructions of stage
//     kt + 2 (A rows have one stage to land); then the first weight
//     instruction of stage kt + SB.
//   - In stage kt + 1, k-step ks (ks < KS - 1) is followed by weight
//     instruction ks + 1 of that same stage kt + SB (the weights have
//     SB - 1 stages to land).
// So when stage kt ends, the DMA this wave issued after the A rows of stage
// kt + 1 is exactly the PWB weight instructions of stage kt + SB - 1; the
// weight rows of stage kt + 1 went before them.
template <class SP, int NMB, class DmaA1, class DmaB1>
__device__ __forceinline__ void split_kloop(f32x16_t (&acc)[SP::R::MB][SP::R::NB],
                                            uint4 (*la)[SP::R::A_U4], uint4 (*lb)[SP::R::B_U4],
                                            int nk, int wm, int wn, int lane,
                                            const DmaA1& dma_a1, const DmaB1& dma_b1) {
  using R = typename SP::R;
  constexpr int MB = R::MB, NB = R::NB, KS = R::KS, PWA = R::PWA, PWB = R::PWB, SB = SP::SB;
  constexpr int C = MB * NB / PWA;                   // MFMAs per A instruction
  static_assert(PWB == KS && C * PWA == MB * NB && PWA == 4, "DMA spread");
  bf16x8_t fa[2][MB], fb[2][NB];
  read_frags_split<R>(fa[0], fb[0], la[0], lb[0], 0, wm, wn, lane, NMB);
  int sa = 0, sb = 0, sbp = SB - 1;   // slots of stage kt; weight slot of stage kt - 1
  for (int kt = 0; kt < nk; ++kt) {
    const uint4* ca = la[sa];
    const uint4* cb = lb[sb];
    const bool bdef = kt + SB - 1 < nk;   // stage kt + SB - 1 exists: its DMA goes on here
#pragma unroll
    for (int ks = 0; ks + 1 < KS; ++ks) {
      read_frags_split<R>(fa[(ks + 1) & 1], fb[(ks + 1) & 1], ca, cb, ks + 1, wm, wn, lane, NMB);
      mfma_step(acc, fa[ks & 1], fb[ks & 1], NMB);
      if (bdef) {
        __builtin_amdgcn_sched_barrier(0);
        dma_b1(sbp, kt + SB - 1, ks + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // this wave has read all of stage kt, and its DMA of stage kt+1 landed
    wait_lgkmcnt0();
    if (kt + 1 < nk) {
      if (bdef) wait_vmcnt<PWB>();
      else wait_vmcnt<0>();
    }
    barrier();
    __builtin_amdgcn_sched_barrier(0);
    const bool an = kt + 2 < nk;
    const bf16x8_t(&fl)[MB] = fa[(KS - 1) & 1];
    const bf16x8_t(&gl)[NB] = fb[(KS - 1) & 1];
    const int san = sa ^ 1, sbn = sb + 1 == SB ? 0 : sb + 1;
    mfma_dma_a<0, C>(acc, fl, gl, NMB, an, sa, kt + 2, dma_a1);
    mfma_dma_a<1, C>(acc, fl, gl, NMB, an, sa, kt + 2, dma_a1);
    mfma_dma_a<2, C>(acc, fl, gl, NMB, an, sa, kt + 2, dma_a1);
    mfma_dma_a<3, C>(acc, fl, gl, NMB, an, sa, kt + 2, dma_a1);
    if (kt + SB < nk) dma_b1(sb, kt + SB, 0);
    sbp = sb;
    sa = san;
    sb = sbn;
    if (kt + 1 < nk)
      read_frags_split<R>(fa[KS & 1], fb[KS & 1], la[sa], lb[sb], 0, wm, wn, lane, NMB);
  }
}

template <class SP, int N, class DmaA1, class DmaB1>
__device__ __forceinline__ void split_kloop_n(int nmb, f32x16_t (&acc)[SP::R::MB][SP::R::NB],
                                              uint4 (*la)[SP::R::A_U4],
                                              uint4 (*lb)[SP::R::B_U4], int nk, int wm, int wn,
                                              int lane, const DmaA1& dma_a1, const DmaB1& dma_b1) {
  if constexpr (N == 0) {
    split_kloop<SP, 0>(acc, la, lb, nk, wm, wn, lane, dma_a1, dma_b1);
  } else {
    if (nmb == N) split_kloop<SP, N>(acc, la, lb, nk, wm, wn, lane, dma_a1, dma_b1);
    else split_kloop_n<SP, N - 1>(nmb, acc, la, lb, nk, wm, wn, lane, dma_a1, dma_b1);
  }
}


// One tile of the split-ring kernel (bf16 weights).  A rows are read in
// place, or with p.gather set, row r of the tile is row gather[row0 + r] of A.
template <int BM, int BN, int WM, int WN, int BK, int SB, int EPI, bool UNIFORM = false>
__device__ __forceinline__ void split_tile(const GemmArgs& p, const Tile& t,
                                           uint4 (*la)[Split<BM, BN, WM, WN, BK, SB>::R::A_U4],
                                           uint4 (*lb)[Split<BM, BN, WM, WN, BK, SB>::R::B_U4],
                                           uint32_t addr_a, uint32_t addr_b, int wave, int lane) {
  constexpr bool GATEUP = EPI == kEpiSwiglu;
  using SP = Split<BM, BN, WM, WN, BK, SB>;
  using R = typename SP::R;
  constexpr int MB = R::MB, NB = R::NB, PWA = R::PWA, PWB = R::PWB;
  const int wm = wave / WN, wn = wave % WN;
  const int lra = lane / R::CHA, lca = lane % R::CHA;
  const int lrb = lane / R::CHB, lcb = lane % R::CHB;
  const int nk = p.Kd / BK;
  const size_t wmat = (size_t)p.Nout * p.Kd;
  // DMA sources and LDS offsets within a slot; as in ring_tile, the lane that
  // writes LDS chunk c of a row fetches global chunk c ^ swizzle(row)
  uint32_t offa[PWA], ldsa[PWA], offb[PWB], ldsb[PWB];
  const void* baseb[PWB];
  const uint16_t* basea = p.gather ? p.A : p.A + t.row0 * p.Kd;
#pragma unroll
  for (int j = 0; j < PWA; ++j) {
    const int q = wave * PWA + j;
    const int trow = q * R::RPIA + lra;
    const int row = min(trow, t.rows - 1);
    const uint32_t src = p.gather ? (uint32_t)p.gather[t.row0 + row] : (uint32_t)row;
    offa[j] = (src * p.Kd + (uint32_t)(lca ^ swz<BK>(trow)) * 8) * 2u;
    ldsa[j] = q * 1024;
  }
  static_assert(R::B_U4 * 16 == kPackStage && R::RPIB * R::CHB == 64, "packed stage image");
  // per-stage advance of a weight DMA source: 64 k values of a row, or a
  // packed stage image
  const uint32_t bstep = p.wpack ? kPackStage : BK * 2;
#pragma unroll
  for (int jb = 0; jb < PWB; ++jb) {
    const int q = wave * PWB + jb;
    const int g0 = q * R::RPIB, trow = g0 + lrb;
    if (p.wpack) {
      baseb[jb] = static_cast<const char*>(p.B0) + packed_panel(p, t.e, t.nt, nk);
      offb[jb] = q * 1024 + lane * 16;
    } else {
      bool up;
      const int wrow = min(weight_row<BN, GATEUP>(t.nt, g0, up) + lrb, p.Nout - 1);
      baseb[jb] = static_cast<const char*>(up ? p.B1 : p.B0) + (size_t)t.e * wmat * 2;
      offb[jb] = ((uint32_t)wrow * p.Kd + (uint32_t)(lcb ^ swz<BK>(trow)) * 8) * 2u;
    }
    ldsb[jb] = q * 1024;
  }
  auto dma_a = [&](int s, int kt) {
    const uint32_t l0 = addr_a + (uint32_t)s * SP::A_BYTES;
#pragma unroll
    for (int j = 0; j < PWA; ++j)
      lds_dma16<UNIFORM>(__builtin_amdgcn_readfirstlane(l0 + ldsa[j]), basea,
                offa[j] + (uint32_t)kt * (BK * 2));
  };
  auto dma_b = [&](int s, int kt) {
    const uint32_t l0 = addr_b + (uint32_t)s * SP::B_BYTES;
#pragma unroll
    for (int jb = 0; jb < PWB; ++jb)
      lds_dma16<UNIFORM>(__builtin_amdgcn_readfirstlane(l0 + ldsb[jb]), baseb[jb],
                offb[jb] + (uint32_t)kt * bstep);
  };

  // single instructions: A instruction j, weight instruction jb (the callers
  // pass constants once unrolled; the loops keep the arrays in registers)
  auto dma_a1 = [&](int s, int kt, int j) {
    const uint32_t l0 = addr_a + (uint32_t)s * SP::A_BYTES;
#pragma unroll
    for (int i = 0; i < PWA; ++i)
      if (i == j)
        lds_dma16<UNIFORM>(__builtin_amdgcn_readfirstlane(l0 + ldsa[i]), basea,
                  offa[i] + (uint32_t)kt * (BK * 2));
  };
  auto dma_b1 = [&](int s, int kt, int jb) {
    const uint32_t l0 = addr_b + (uint32_t)s * SP::B_BYTES;
#pragma unroll
    for (int i = 0; i < PWB; ++i)
      if (i == jb)
        lds_dma16<UNIFORM>(__builtin_amdgcn_readfirstlane(l0 + ldsb[i]), baseb[i],
                  offb[i] + (uint32_t)kt * bstep);
  };

  f32x16_t acc[MB][NB];
  zero(acc);
  // every wave is past its last LDS read of the previous tile
  wait_lgkmcnt0();
  barrier();
  // Prologue in the loop's issue order, as if steps -SB .. -1 had run:
  // weight rows of stages 0 .. SB-3, A(0), B(SB-2), A(1), and the first
  // weight instruction of B(SB-1) (step 0's k-steps issue the others).
  for (int j = 0; j + 2 < SB; ++j)
    if (j < nk) dma_b(j, j);
  dma_a(0, 0);
  if (SB - 2 < nk) dma_b(SB - 2, SB - 2);
  if (1 < nk) dma_a(1, 1);
  if (SB - 1 < nk) dma_b1(SB - 1, SB - 1, 0);
  // stage 0 has landed: only B(SB-2), A(1) and B(SB-1)'s first instruction
  // may be outstanding
  wait_vm_le<PWB + PWA + 1>((SB - 2 < nk ? PWB : 0) + (1 < nk ? PWA : 0) +
                            (SB - 1 < nk ? 1 : 0));
  barrier();
  // 32-row blocks of this wave that hold at least one row of the tile
  const int nmb = min(MB, max(0, (t.rows - wm * R::TM + 31) / 32));
  split_kloop_n<SP, MB>(nmb, acc, la, lb, nk, wm, wn, lane, dma_a1, dma_b1);
  store_tile<MB, NB, R::TM, R::TN, BN, EPI>(p, t, acc, wm, wn, lane);
}

template <int BM, int BN, int WM, int WN, int BK, int SB, int EPI, int PER>
__global__ void __launch_bounds__(64 * WM * WN)
grouped_gemm_split(GemmArgs p) {
  using R = typename Split<BM, BN, WM, WN, BK, SB>::R;
  __shared__ uint4 la[2][R::A_U4];
  __shared__ uint4 lb[SB][R::B_U4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t addr_a = (uint32_t)(uintptr_t)(lds_void_t*)&la[0][0];
  const uint32_t addr_b = (uint32_t)(uintptr_t)(lds_void_t*)&lb[0][0];
  int ms[PER];
  const int mt_total = build_work_list_regs<BM, PER>(p, ms, lane, gridDim.x);
  const int xcd = blockIdx.x & 7, P8 = gridDim.x >> 3, j0 = blockIdx.x >> 3;
  // (the same value in every lane; readfirstlane lets the compiler see it)
  const int begin = __builtin_amdgcn_readfirstlane(
      xcd_begin_regs<BM, PER>(p, ms, mt_total, lane, xcd, P8));
  const int end = __builtin_amdgcn_readfirstlane(
      xcd_begin_regs<BM, PER>(p, ms, mt_total, lane, xcd + 1, P8));
  for (int l = begin + j0; l < end; l += P8)
    split_tile<BM, BN, WM, WN, BK, SB, EPI>(p, decode_tile_regs<BM, PER>(p, ms, mt_total, lane, l),
                                            la, lb, addr_a, addr_b, wave, lane);
}

// ------------------------------------------------------------ fused FFN
//
// The whole expert FFN in one persistent launch ("MoE 推理完整机制" (zoe.im),
// 第四层: one kernel, compute units handed to experts dynamically, any number
// of rows per expert).  There are two work lists in the grouped GEMM's tile
// order: every gate/up tile, then every down tile.  Each list is cut into
// eight contiguous parts, one per XCD, each with its own claim counter, so
// that the row tiles sharing a weight panel run on one XCD and meet in its L2
// (as in the grouped GEMM).  A workgroup claims tiles from its XCD's part of
// the gate/up list, then from the other XCDs' parts, and only when every
// gate/up tile is claimed does it turn to the down list (own part first).  A
// gate/up tile gathers its A rows straight from x through row_token (no
// permuted copy of x), writes its h columns and counts itself finished for
// its row tile; a down tile waits until every gate/up tile of its row tile
// has been counted.  Every tile a down tile waits for was claimed before by
// a running workgroup that waits for nothing, so the launch always drains.
// A wait is still bounded: after kWaitTicks of the 100 MHz real-time counter
// it sets the error word and goes on (the results are then wrong, and the
// caller can read the word).
//
// Ordering: every wave of a gate/up tile waits until its h stores have
// completed (they are then in this XCD's L2); after a barrier, wave 0 writes
// the L2 back (agent-scope release fence) and adds 1 to the row tile's count.
// In a down tile, wave 0 polls that count with plain device-coherent loads (an
// acquire per poll would invalidate this XCD's caches over and over, starving
// the tiles being waited for), then acquires once (invalidating this CU's L1
// and this XCD's L2) and waits for that to finish before a barrier releases
// the other waves' loads.  One write-back and one invalidation per tile: done
// by every wave, they took a third of the launch's time.

struct FusedArgs {
  GemmArgs gu;       // gate/up: A = x gathered by row_token, C = h
  GemmArgs dn;       // down: A = h, C = out_perm
  int32_t* claim;    // [16], zero at launch: tiles claimed from each XCD's part of the
                     // gate/up list [0, 8), then of the down list [8, 16)
  int32_t* err;      // [1], zero at launch; nonzero after a wait ran past its bound
  int32_t* done;     // [row tiles], zero at launch: finished gate/up tiles per row tile
};

constexpr int kFusedWords = 17;            // claim counters and the error word
constexpr uint64_t kWaitTicks = 5000000;   // 50 ms of the 100 MHz real-time counter

template <int BM, int BN, int WM, int WN, int BK, int S, bool FP8>
__global__ void __launch_bounds__(64 * WM * WN)
grouped_ffn_fused(FusedArgs f) {
  using R = Ring<BM, BN, WM, WN, BK, S, FP8>;
  __shared__ uint4 lds[S][R::STAGE_U4];
  __shared__ int32_t mstart[1025];
  __shared__ int32_t ticket;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(lds_void_t*)&lds[0][0];
  if (wave == 0) build_work_list<BM>(f.gu, mstart, lane, 0);   // one row split for both lists
  __syncthreads();
  // No branch on the loop's path may depend on the lane (or look as if it
  // did): with an "if (tid == 0)" at the loop head and another after the
  // tile, the compiler merges the two across the back edge, and the lanes
  // other than thread 0 then go round an inner loop that skips the claim
  // while thread 0 waits for them to leave it, so the workgroup repeats one
  // tile for ever.  Hence scalar loop bounds, and atomics that a whole wave
  // executes (lane 0 adds 1, the others 0).
  const int M = __builtin_amdgcn_readfirstlane(mstart[f.gu.E]);
  const int T1 = f.gu.n_tiles * M, T = T1 + f.dn.n_tiles * M;
  const int need = f.gu.n_tiles;               // gate/up tiles per row tile
  const int one = lane == 0 ? 1 : 0;
  const int xcd = blockIdx.x & 7;
  int list = 0, step = 0;                      // wave 0: list and XCD part being claimed from
  for (;;) {
    if (wave == 0) {
      int got = T;
      while (list < 2) {
        const int n = list ? T - T1 : T1, x = (xcd + step) & 7;
        const int b = (int)((int64_t)n * x / 8), e = (int)((int64_t)n * (x + 1) / 8);
        const int c = __builtin_amdgcn_readfirstlane(__hip_atomic_fetch_add(
            f.claim + 8 * list + x, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (b + c < e) {
          got = (list ? T1 : 0) + b + c;
          break;
        }
        if (++step == 8) {
          step = 0;
          ++list;
        }
      }
      ticket = got;
    }
    __syncthreads();
    const int l = __builtin_amdgcn_readfirstlane(ticket);
    __syncthreads();
    if (l >= T) break;
    if (l < T1) {
      const Tile t = decode_tile<BM>(f.gu, mstart, l);
      ring_tile<BM, BN, WM, WN, BK, S, kEpiSwiglu, FP8, true>(f.gu, t, lds, lds_addr, wave,
                                                              lane);
      // every wave's h stores have reached this XCD's L2; wave 0 writes the
      // L2 back (agent-scope release) and counts the tile
      wait_vmcnt<0>();
      __syncthreads();
      if (wave == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_fetch_add(f.done + t.mtg, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      const Tile t = decode_tile<BM>(f.dn, mstart, l - T1);
      // wave 0 waits for the row tile's count, then invalidates this CU's L1
      // and this XCD's L2 (agent-scope acquire) before the other waves load
      if (wave == 0) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        for (;;) {
          const int c = __builtin_amdgcn_readfirstlane(
              __hip_atomic_load(f.done + t.mtg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
          if (c >= need) break;
          if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
            __hip_atomic_fetch_or(f.err, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(4);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        wait_vmcnt<0>();
      }
      __syncthreads();
      ring_tile<BM, BN, WM, WN, BK, S, kEpiStore, FP8, true>(f.dn, t, lds, lds_addr, wave, lane);
    }
  }
}

// The fused FFN on the split rings (256 x 256 tiles, bf16, E <= 64 * PER):
// the same claim loop, dependency counts and ordering as grouped_ffn_fused,
// with split_tile as the tile body and the work list in registers.  The
// rings fill LDS, so the claimed tile goes from wave 0 to the other waves
// through the first word of A slot 0.  That word is free whenever it is
// used: after a tile's last barrier every wave is done with LDS (each waited
// for its own reads before that barrier), and the next tile's DMA goes out
// only after the barriers that follow the read of the word.
template <int BM, int BN, int WM, int WN, int BK, int SB, int PER>
__global__ void __launch_bounds__(64 * WM * WN)
grouped_ffn_fused_split(FusedArgs f) {
  using R = typename Split<BM, BN, WM, WN, BK, SB>::R;
  __shared__ uint4 la[2][R::A_U4];
  __shared__ uint4 lb[SB][R::B_U4];
  volatile int32_t* ticket = reinterpret_cast<volatile int32_t*>(&la[0][0]);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t addr_a = (uint32_t)(uintptr_t)(lds_void_t*)&la[0][0];
  const uint32_t addr_b = (uint32_t)(uintptr_t)(lds_void_t*)&lb[0][0];
  int ms[PER];
  const int M = build_work_list_regs<BM, PER>(f.gu, ms, lane, 0);   // one row split for both
  // (the loop's control flow stays wave-uniform; see grouped_ffn_fused)
  const int T1 = f.gu.n_tiles * M, T = T1 + f.dn.n_tiles * M;
  const int need = f.gu.n_tiles;               // gate/up tiles per row tile
  const int one = lane == 0 ? 1 : 0;
  const int xcd = blockIdx.x & 7;
  int list = 0, step = 0;                      // wave 0: list and XCD part being claimed from
  for (;;) {
    if (wave == 0) {
      int got = T;
      while (list < 2) {
        const int n = list ? T - T1 : T1, x = (xcd + step) & 7;
        const int b = (int)((int64_t)n * x / 8), e = (int)((int64_t)n * (x + 1) / 8);
        const int c = __builtin_amdgcn_readfirstlane(__hip_atomic_fetch_add(
            f.claim + 8 * list + x, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (b + c < e) {
          got = (list ? T1 : 0) + b + c;
          break;
        }
        if (++step == 8) {
          step = 0;
          ++list;
        }
      }
      *ticket = got;
    }
    __syncthreads();
    const int l = __builtin_amdgcn_readfirstlane(*ticket);
    __syncthreads();
    if (l >= T) break;
    if (l < T1) {
      const Tile t = decode_tile_regs<BM, PER>(f.gu, ms, M, lane, l);
      split_tile<BM, BN, WM, WN, BK, SB, kEpiSwiglu, true>(f.gu, t, la, lb, addr_a, addr_b,
                                                           wave, lane);
      // every wave's h stores have reached this XCD's L2; wave 0 writes the
      // L2 back (agent-scope release) and counts the tile
      wait_vmcnt<0>();
      __syncthreads();
      if (wave == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_fetch_add(f.done + t.mtg, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      const Tile t = decode_tile_regs<BM, PER>(f.dn, ms, M, lane, l - T1);
      // wave 0 waits for the row tile's count, then invalidates this CU's L1
      // and this XCD's L2 (agent-scope acquire) before the other waves load
      if (wave == 0) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        for (;;) {
          const int c = __builtin_amdgcn_readfirstlane(
              __hip_atomic_load(f.done + t.mtg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
          if (c >= need) break;
          if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
            __hip_atomic_fetch_or(f.err, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(4);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        wait_vmcnt<0>();
      }
      __syncthreads();
      split_tile<BM, BN, WM, WN, BK, SB, kEpiStore, true>(f.dn, t, la, lb, addr_a, addr_b, wave,
                                                          lane);
    }
  }
}

// Zeroes the fused launch's claim counters, error word and row-tile counters.
__global__ void fused_reset_kernel(int32_t* words, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    words[i] = 0;
}

// ------------------------------------------------------------ register-staged

constexpr int RBK = 64;            // k depth of one LDS stage
constexpr int RCH = RBK / 8;       // 16-byte chunks per tile row (bf16)
constexpr int QCH = RBK / 16;      // 16-byte chunks per weight row (FP8 codes)

// One stage's global loads: A rows (bf16), then the weight rows -- bf16
// chunks, or FP8 code chunks with the scale byte of each chunk's k-block.
template <int NA, int NB_, bool FP8>
__device__ __forceinline__ void stage_gload(uint4 (&ra)[NA], uint4 (&rb)[NB_], uint32_t (&rs)[NB_],
                                            const uint16_t* a_base, const uint32_t (&a_off)[NA],
                                            const char* b0_base, const char* b1_base,
                                            const uint32_t (&b_off)[NB_], const uint8_t* s0_base,
                                            const uint8_t* s1_base, const uint32_t (&s_off)[NB_],
                                            uint32_t b_up, uint32_t bstep, int kt) {
#pragma unroll
  for (int i = 0; i < NA; ++i)
    ra[i] = *reinterpret_cast<const uint4*>(a_base + a_off[i] + kt * RBK);
#pragma unroll
  for (int i = 0; i < NB_; ++i) {
    const bool up = (b_up >> i) & 1;
    if (FP8) {
      rb[i] = *reinterpret_cast<const uint4*>((up ? b1_base : b0_base) + b_off[i] + kt * RBK);
      rs[i] = (up ? s1_base : s0_base)[s_off[i] + kt * (RBK / 32) * 32];
    } else {
      rb[i] = *reinterpret_cast<const uint4*>((up ? b1_base : b0_base) + b_off[i] + kt * bstep);
    }
  }
}

template <int NA, int NB_, int RPP, int QRPP, int BM, bool FP8>
__device__ __forceinline__ void stage_lstore(uint4* st, const uint4 (&ra)[NA],
                                             const uint4 (&rb)[NB_], const uint32_t (&rs)[NB_],
                                             int lrow, int lchunk, int qrow, int qchunk) {
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int r = lrow + i * RPP;
    st[r * RCH + (lchunk ^ swz<RBK>(r))] = ra[i];
  }
#pragma unroll
  for (int i = 0; i < NB_; ++i) {
    if (FP8) {
      // 16 codes = bf16 chunks 2*qchunk and 2*qchunk + 1 of the row
      const int r = qrow + i * QRPP;
      const float sc = scale_of(rs[i]);
      st[(BM + r) * RCH + ((2 * qchunk) ^ swz<RBK>(r))] =
          __builtin_bit_cast(uint4, dequant8(rb[i].x, rb[i].y, sc));
      st[(BM + r) * RCH + ((2 * qchunk + 1) ^ swz<RBK>(r))] =
          __builtin_bit_cast(uint4, dequant8(rb[i].z, rb[i].w, sc));
    } else {
      const int r = lrow + i * RPP;
      st[(BM + r) * RCH + (lchunk ^ swz<RBK>(r))] = rb[i];
    }
  }
}

template <int BM, int BN, int WM, int WN, int EPI, bool FP8>
__global__ void __launch_bounds__(64 * WM * WN)
grouped_gemm_regs(GemmArgs p) {
  constexpr bool GATEUP = EPI == kEpiSwiglu;
  constexpr int NT = 64 * WM * WN;                // threads
  constexpr int TM = BM / WM, TN = BN / WN;       // wave tile
  constexpr int MB = TM / 32, NB = TN / 32;       // 32x32 MFMA blocks per wave
  static_assert(!GATEUP || NB % 2 == 0, "gate/up pairs");
  constexpr int RPP = NT / RCH;                   // bf16 tile rows loaded per pass
  constexpr int QRPP = NT / QCH;                  // FP8 weight rows loaded per pass
  constexpr int A_LD = BM / RPP;                  // 16-byte loads per thread per stage
  constexpr int B_LD = FP8 ? BN / QRPP : BN / RPP;
  static_assert(A_LD >= 1 && B_LD >= 1 && BM % RPP == 0 && BN % (FP8 ? QRPP : RPP) == 0,
                "loader shape");

  __shared__ uint4 lds[2][(BM + BN) * RCH];
  __shared__ int32_t mstart[1025];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lrow = tid / RCH, lchunk = tid % RCH;   // bf16 loader mapping
  const int qrow = tid / QCH, qchunk = tid % QCH;   // FP8 weight loader mapping

  if (wave == 0) build_work_list<BM>(p, mstart, lane, gridDim.x);
  __syncthreads();
  const int total = p.n_tiles * __builtin_amdgcn_readfirstlane(mstart[p.E]);
  const int xcd = blockIdx.x & 7, P8 = gridDim.x >> 3, j0 = blockIdx.x >> 3;
  const int begin = (int)((int64_t)total * xcd / 8);
  const int end = (int)((int64_t)total * (xcd + 1) / 8);
  const size_t wmat = (size_t)p.Nout * p.Kd;
  const int ebytes = FP8 ? 1 : 2;                 // bytes per weight element

  for (int l = begin + j0; l < end; l += P8) {
    const Tile t = decode_tile<BM>(p, mstart, l);
    const uint16_t* a_base = p.A + t.row0 * p.Kd + lchunk * 8;
    const int bcol = FP8 ? qchunk * 16 : lchunk * 16;   // byte column of this thread's chunk
    const char* b0_base = static_cast<const char*>(p.B0) + t.e * wmat * ebytes + bcol;
    const char* b1_base = GATEUP ? static_cast<const char*>(p.B1) + t.e * wmat * ebytes + bcol
                                 : b0_base;
    const uint8_t* s0_base = nullptr;
    const uint8_t* s1_base = nullptr;
    if (FP8) {
      s0_base = p.S0 + t.e * (wmat / 32) + (qchunk >> 1) * 32;
      s1_base = GATEUP ? p.S1 + t.e * (wmat / 32) + (qchunk >> 1) * 32 : s0_base;
    }
    uint32_t a_off[A_LD], b_off[B_LD], s_off[B_LD];
    uint32_t b_up = 0;                               // bit i: load i reads the up matrix
    const int nk = p.Kd / RBK;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) a_off[i] = (uint32_t)min(lrow + i * RPP, t.rows - 1) * p.Kd;
    // per-stage advance of a weight load: 64 k values of a row, or a packed
    // stage image (whose row r holds, at chunk c ^ swz(r), the row's chunk c)
    uint32_t bstep = RBK * 2;
    if constexpr (!FP8) {
      static_assert(BN * RCH * 16 == (int)kPackStage, "packed stage image");
      if (p.wpack) {
        bstep = kPackStage;
        b0_base = static_cast<const char*>(p.B0) + packed_panel(p, t.e, t.nt, nk);
        b1_base = b0_base;
      }
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      bool up;
      const int wrow =
          min(weight_row<BN, GATEUP>(t.nt, (FP8 ? qrow + i * QRPP : lrow + i * RPP), up),
              p.Nout - 1);
      b_up |= (uint32_t)up << i;
      b_off[i] = (uint32_t)wrow * p.Kd * ebytes;
      if (!FP8 && p.wpack) {
        const int r = lrow + i * RPP;
        b_off[i] = (uint32_t)(r * RCH + (lchunk ^ swz<RBK>(r))) * 16;
      }
      s_off[i] = (uint32_t)(wrow >> 5) * (uint32_t)p.Kd + (uint32_t)(wrow & 31);
    }

    f32x16_t acc[MB][NB];
    zero(acc);
    uint4 ra[A_LD], rb[B_LD];
    uint32_t rs[B_LD];
    // Stage 0 is rewritten below: wait until every wave is done with the
    // previous tile's last stage.
    __syncthreads();
    stage_gload<A_LD, B_LD, FP8>(ra, rb, rs, a_base, a_off, b0_base, b1_base, b_off, s0_base,
                                 s1_base, s_off, b_up, bstep, 0);
    stage_lstore<A_LD, B_LD, RPP, QRPP, BM, FP8>(lds[0], ra, rb, rs, lrow, lchunk, qrow, qchunk);
    __syncthreads();
    for (int kt = 0; kt + 1 < nk; ++kt) {
      stage_gload<A_LD, B_LD, FP8>(ra, rb, rs, a_base, a_off, b0_base, b1_base, b_off, s0_base,
                                   s1_base, s_off, b_up, bstep, kt + 1);
      bf16x8_t af[MB], bfr[NB];
#pragma unroll
      for (int ks = 0; ks < RBK / 16; ++ks) {
        read_frags<MB, NB, TM, TN, BM, RBK>(af, bfr, lds[kt & 1], ks, wm, wn, lane);
        mfma_step(acc, af, bfr);
      }
      stage_lstore<A_LD, B_LD, RPP, QRPP, BM, FP8>(lds[(kt & 1) ^ 1], ra, rb, rs, lrow, lchunk,
                                                   qrow, qchunk);
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
    store_tile<MB, NB, TM, TN, BN, EPI>(p, t, acc, wm, wn, lane);
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

// Column tiles per expert: a gate/up tile covers BN / 2 columns of h (BN / 2
// gate rows and the matching up rows), a down tile BN columns of out_perm.
template <int BN, bool GATEUP>
GemmArgs with_tiles(GemmArgs a) {  // (GATEUP: interleaved gate/up tile)
  const int cols = GATEUP ? BN / 2 : BN;
  a.n_tiles = (a.Nout + cols - 1) / cols;
  return a;
}

template <int BM, int BN, int WM, int WN, int BK, int S, int EPI, bool FP8, bool SPREAD = false>
hipError_t launch_ring(const Dims& d, const GemmArgs& a0, hipStream_t s) {
  const GemmArgs a = with_tiles<BN, EPI == kEpiSwiglu>(a0);
  hipLaunchKernelGGL((grouped_gemm_ring<BM, BN, WM, WN, BK, S, EPI, FP8, SPREAD>),
                     dim3((unsigned)grid_size<BM>(d, a.n_tiles, 1)), dim3(64 * WM * WN), 0, s, a);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int BK, int SB, int EPI>
hipError_t launch_split(const Dims& d, const GemmArgs& a0, hipStream_t s) {
  const GemmArgs a = with_tiles<BN, EPI == kEpiSwiglu>(a0);
  const dim3 grid((unsigned)grid_size<BM>(d, a.n_tiles, 1)), block(64 * WM * WN);
  if (a.E <= 64)
    hipLaunchKernelGGL((grouped_gemm_split<BM, BN, WM, WN, BK, SB, EPI, 1>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((grouped_gemm_split<BM, BN, WM, WN, BK, SB, EPI, 4>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int EPI, bool FP8>
hipError_t launch_regs(const Dims& d, const GemmArgs& a0, int occupancy, hipStream_t s) {
  // these tiles read A rows in place: a gathered A would be read as x_perm
  if (a0.gather) return hipErrorNotSupported;
  const GemmArgs a = with_tiles<BN, EPI == kEpiSwiglu>(a0);
  hipLaunchKernelGGL((grouped_gemm_regs<BM, BN, WM, WN, EPI, FP8>),
                     dim3((unsigned)grid_size<BM>(d, a.n_tiles, occupancy)), dim3(64 * WM * WN),
                     0, s, a);
  return hipGetLastError();
}

// Tile shape by the average number of rows per expert (R / E).  Barriers cost
// more than prefetch depth gains, so stages are as deep as LDS allows (FP8
// weight stages are smaller: 128-deep when k is a multiple of 128):
//   <= 48  : 32 x 256 tiles (decode: the weight stream rules), 4 waves; an
//            LDS-DMA ring of 64-deep stages (4) when k >= 1024 (FP8: 3 of
//            128-deep when k >= 512), else register-staged
//   <= 192 : 128 x 256 tiles, 8 waves (64 x 64 each), 64-deep stages, 3-stage ring
//            (FP8: 2 stages of 128-deep)
//   else   : 256 x 256 tiles, 8 waves, 64-deep stages: the split ring with bf16
//            weights and E <= 256 (its work list lives in 4 registers per
//            lane), else a 2-stage ring, or with FP8 weights a 3-stage ring
//            with its DMA spread over the stage; one barrier per 64 k
//            (32-deep stages, twice the barriers, were 5-12% slower)
enum class Shape { Small, Mid, Large };
inline Shape pick(const Dims& d) {
  const double avg = (double)d.R / d.E;
  if (avg <= 48.0) return Shape::Small;
  if (avg <= 192.0) return Shape::Mid;
  return Shape::Large;
}

}  // namespace

size_t ffn_ws_bytes(const Dims& d) { return align_up((size_t)d.R * d.F * 2); }

namespace {

// Tile shape by rows per expert (or as given), for any epilogue.
template <int EPI, bool FP8>
hipError_t launch_gemm(const Dims& d, const GemmArgs& a, hipStream_t s, Shape shape) {
  switch (shape) {
    case Shape::Small:
      // the weight stream rules: a deep LDS-DMA ring (over 100 KB in flight
      // per CU) when k is long enough to fill it, else register staging
      if constexpr (FP8) {
        // (packed FP8 stacks are read by 128- or 64-deep stages only)
        if ((a.Kd >= 512 || a.wpack) && a.Kd % 128 == 0)
          return launch_ring<32, 256, 1, 4, 128, 3, EPI, FP8>(d, a, s);
      }
      if (a.Kd >= 1024) return launch_ring<32, 256, 1, 4, 64, FP8 ? 6 : 4, EPI, FP8>(d, a, s);
      return launch_regs<32, 256, 1, 4, EPI, FP8>(d, a, 2, s);
    case Shape::Mid:
      if constexpr (FP8) {
        if (a.Kd % 128 == 0) return launch_ring<128, 256, 2, 4, 128, 2, EPI, FP8>(d, a, s);
      }
      return launch_ring<128, 256, 2, 4, 64, FP8 ? 4 : 3, EPI, FP8>(d, a, s);
    default:
      if constexpr (!FP8) {
        if (a.E <= 256) return launch_split<256, 256, 2, 4, 64, 3, EPI>(d, a, s);
      }
      if constexpr (FP8) return launch_ring<256, 256, 2, 4, 64, 3, EPI, true, true>(d, a, s);
      return launch_ring<256, 256, 2, 4, 64, 2, EPI, false>(d, a, s);
  }
}

template <int EPI, bool FP8>
hipError_t launch_gemm(const Dims& d, const GemmArgs& a, hipStream_t s) {
  return launch_gemm<EPI, FP8>(d, a, s, pick(d));
}

}  // namespace

hipError_t launch_expert_gateup(const Dims& d, const uint16_t* x_perm, const int32_t* offsets,
                                const uint16_t* wg, const uint16_t* wu, uint16_t* h,
                                hipStream_t s, bool packed) {
  GemmArgs a{x_perm, wg, wu, h, offsets, d.E, d.D, d.F, 0, nullptr, nullptr};
  a.wpack = packed;
  return launch_gemm<kEpiSwiglu, false>(d, a, s);
}

// The LDS-DMA ring and split-ring tiles can read A rows through row_token;
// the register-staged 32-row tiles (few rows per expert, short k) cannot.
// With FP8 weights the 32-row ring also serves k >= 512 in steps of 128.
bool gateup_gather_supported(const Dims& d, bool fp8, bool packed) {
  return pick(d) != Shape::Small || d.D >= 1024 ||
         (fp8 && (d.D >= 512 || packed) && d.D % 128 == 0);
}

hipError_t launch_expert_gateup_gathered(const Dims& d, const uint16_t* x,
                                         const int32_t* row_token, const int32_t* offsets,
                                         const uint16_t* wg, const uint16_t* wu, uint16_t* h,
                                         hipStream_t s, bool packed) {
  if (!gateup_gather_supported(d)) return hipErrorNotSupported;
  GemmArgs a{x, wg, wu, h, offsets, d.E, d.D, d.F, 0, nullptr, nullptr, nullptr, row_token};
  a.wpack = packed;
  return launch_gemm<kEpiSwiglu, false>(d, a, s);
}

hipError_t launch_expert_down(const Dims& d, const uint16_t* h, const int32_t* offsets,
                              const uint16_t* wd, uint16_t* out_perm, hipStream_t s,
                              bool packed) {
  GemmArgs a{h, wd, nullptr, out_perm, offsets, d.E, d.F, d.D, 0, nullptr, nullptr};
  a.wpack = packed;
  return launch_gemm<kEpiStore, false>(d, a, s);
}

hipError_t launch_grouped_ffn(const Dims& d, const uint16_t* x_perm, const int32_t* offsets,
                              const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                              uint16_t* out_perm, uint16_t* h, void* ws, hipStream_t s,
                              bool packed) {
  if (!h) h = static_cast<uint16_t*>(ws);
  hipError_t e = launch_expert_gateup(d, x_perm, offsets, wg, wu, h, s, packed);
  if (e != hipSuccess) return e;
  return launch_expert_down(d, h, offsets, wd, out_perm, s, packed);
}

namespace {
// One 16-byte chunk of the packed image per item, grid-stride: the chunk that
// the unpacked weight DMA fetches for that LDS position (see kPackStage).
template <bool GATEUP>
__global__ void __launch_bounds__(256)
pack_weights_kernel(const uint16_t* __restrict__ w0, const uint16_t* __restrict__ w1, int Nout,
                    int Kd, int n_tiles, int64_t chunks, uint4* __restrict__ out) {
  const int nk = Kd / 64;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < chunks;
       c += (int64_t)gridDim.x * 256) {
    const int64_t stage = c >> 11;                     // 2048 chunks per stage image
    const int w = (int)(c & 2047), q = w >> 6, l = w & 63;
    const int kt = (int)(stage % nk);
    const int64_t panel = stage / nk;
    const int nt = (int)(panel % n_tiles);
    const int64_t e = panel / n_tiles;
    const int trow = q * 8 + (l >> 3);
    bool up;
    const int wrow = min(weight_row<256, GATEUP>(nt, q * 8, up) + (l >> 3), Nout - 1);
    const uint16_t* src = (up ? w1 : w0) + (e * Nout + wrow) * (int64_t)Kd + kt * 64 +
                          ((l & 7) ^ swz<64>(trow)) * 8;
    out[c] = *reinterpret_cast<const uint4*>(src);
  }
}

// Column tiles of a packed stack: 128 columns of h per gate/up panel, 256
// output columns per down panel.
inline int64_t pack_tiles(const Dims& d, bool gateup) {
  return gateup ? (d.F + 127) / 128 : (d.D + 255) / 256;
}
}  // namespace

size_t packed_weight_bytes(const Dims& d, bool gateup, bool fp8) {
  const int64_t kd = gateup ? d.D : d.F;
  return (size_t)d.E * pack_tiles(d, gateup) * (kd / (fp8 ? 128 : 64)) * kPackStage;
}

hipError_t launch_pack_weights(const Dims& d, bool gateup, const uint16_t* w0, const uint16_t* w1,
                               uint16_t* out, hipStream_t s, bool fp8) {
  // FP8 codes are packed as pairs: a 128-code stage is 64 two-byte units
  const int Nout = gateup ? d.F : d.D, Kd = (gateup ? d.D : d.F) / (fp8 ? 2 : 1);
  const int64_t chunks = (int64_t)(packed_weight_bytes(d, gateup, fp8) / 16);
  const int64_t blocks = std::min<int64_t>((chunks + 255) / 256, (int64_t)device_cu_count() * 8);
  if (gateup)
    hipLaunchKernelGGL(pack_weights_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, w0, w1,
                       Nout, Kd, (int)pack_tiles(d, true), chunks, reinterpret_cast<uint4*>(out));
  else
    hipLaunchKernelGGL(pack_weights_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, w0,
                       w0, Nout, Kd, (int)pack_tiles(d, false), chunks,
                       reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}

hipError_t launch_expert_gateup_fp8(const Dims& d, const uint16_t* x_perm, const int32_t* offsets,
                                    const Fp8Weight& wg, const Fp8Weight& wu, uint16_t* h,
                                    hipStream_t s, bool packed) {
  GemmArgs a{x_perm, wg.codes, wu.codes, h, offsets, d.E, d.D, d.F, 0, wg.scales, wu.scales};
  a.wpack = packed;
  return launch_gemm<kEpiSwiglu, true>(d, a, s);
}

hipError_t launch_expert_gateup_fp8_gathered(const Dims& d, const uint16_t* x,
                                             const int32_t* row_token, const int32_t* offsets,
                                             const Fp8Weight& wg, const Fp8Weight& wu,
                                             uint16_t* h, hipStream_t s, bool packed) {
  if (!gateup_gather_supported(d, true, packed)) return hipErrorNotSupported;
  GemmArgs a{x, wg.codes, wu.codes, h, offsets, d.E, d.D, d.F, 0, wg.scales, wu.scales, nullptr,
             row_token};
  a.wpack = packed;
  return launch_gemm<kEpiSwiglu, true>(d, a, s);
}

hipError_t launch_expert_down_fp8(const Dims& d, const uint16_t* h, const int32_t* offsets,
                                  const Fp8Weight& wd, uint16_t* out_perm, hipStream_t s,
                                  bool packed) {
  GemmArgs a{h, wd.codes, nullptr, out_perm, offsets, d.E, d.F, d.D, 0, wd.scales, nullptr};
  a.wpack = packed;
  return launch_gemm<kEpiStore, true>(d, a, s);
}

hipError_t launch_grouped_ffn_fp8(const Dims& d, const uint16_t* x_perm, const int32_t* offsets,
                                  const Fp8Weight& wg, const Fp8Weight& wu, const Fp8Weight& wd,
                                  uint16_t* out_perm, uint16_t* h, void* ws, hipStream_t s,
                                  bool packed) {
  if (!h) h = static_cast<uint16_t*>(ws);
  hipError_t e = launch_expert_gateup_fp8(d, x_perm, offsets, wg, wu, h, s, packed);
  if (e != hipSuccess) return e;
  return launch_expert_down_fp8(d, h, offsets, wd, out_perm, s, packed);
}

hipError_t launch_expert_up_gelu(const Dims& d, const uint16_t* x_perm, const int32_t* offsets,
                                 const uint16_t* w1, const float* b1, uint16_t* h,
                                 hipStream_t s) {
  return launch_gemm<kEpiBiasGelu, false>(
      d, GemmArgs{x_perm, w1, nullptr, h, offsets, d.E, d.D, d.F, 0, nullptr, nullptr, b1}, s);
}

hipError_t launch_expert_up_gelu_gathered(const Dims& d, const uint16_t* x,
                                          const int32_t* row_token, const int32_t* offsets,
                                          const uint16_t* w1, const float* b1, uint16_t* h,
                                          hipStream_t s) {
  if (!gateup_gather_supported(d)) return hipErrorNotSupported;
  return launch_gemm<kEpiBiasGelu, false>(
      d, GemmArgs{x, w1, nullptr, h, offsets, d.E, d.D, d.F, 0, nullptr, nullptr, b1, row_token},
      s);
}

hipError_t launch_expert_down_bias(const Dims& d, const uint16_t* h, const int32_t* offsets,
                                   const uint16_t* w2, const float* b2, uint16_t* out_perm,
                                   hipStream_t s) {
  return launch_gemm<kEpiBias, false>(
      d, GemmArgs{h, w2, nullptr, out_perm, offsets, d.E, d.F, d.D, 0, nullptr, nullptr, b2}, s);
}

hipError_t launch_grouped_ffn_gelu(const Dims& d, const uint16_t* x_perm, const int32_t* offsets,
                                   const uint16_t* w1, const float* b1, const uint16_t* w2,
                                   const float* b2, uint16_t* out_perm, uint16_t* h, void* ws,
                                   hipStream_t s) {
  if (!h) h = static_cast<uint16_t*>(ws);
  hipError_t e = launch_expert_up_gelu(d, x_perm, offsets, w1, b1, h, s);
  if (e != hipSuccess) return e;
  return launch_expert_down_bias(d, h, offsets, w2, b2, out_perm, s);
}

namespace {
__global__ void write_offsets_kernel(int32_t* offsets2, int n) {
  if (threadIdx.x == 0) {
    offsets2[0] = 0;
    offsets2[1] = n;
  }
}
}  // namespace

hipError_t launch_dense_gelu(int64_t N, int Kd, int Nout, const uint16_t* A, const uint16_t* W,
                             const float* bias, uint16_t* C, int32_t* offsets2, hipStream_t s) {
  hipLaunchKernelGGL(write_offsets_kernel, dim3(1), dim3(64), 0, s, offsets2, (int)N);
  Dims d{};
  d.N = N;
  d.S = N;
  d.R = N;
  d.cap = 0;
  d.D = Kd;
  d.F = Nout;
  d.E = 1;
  d.K = 1;
  d.padded = false;
  // One group of N rows: the largest tile that still gives every compute unit
  // a tile (128 x 256 when it gives at least half of them one).
  const int64_t cols = (Nout + 255) / 256, cu = device_cu_count();
  const Shape shape = ((N + 255) / 256) * cols >= cu       ? Shape::Large
                      : ((N + 127) / 128) * cols * 2 >= cu ? Shape::Mid
                                                           : Shape::Small;
  return launch_gemm<kEpiBiasGelu, false>(
      d, GemmArgs{A, W, nullptr, C, offsets2, 1, Kd, Nout, 0, nullptr, nullptr, bias}, s, shape);
}

namespace {

template <int BM, int BN, int WM, int WN, int BK, int S, bool SPLIT = false>
hipError_t launch_fused(const Dims& d, const FusedArgs& f0, hipStream_t s) {
  FusedArgs f = f0;
  f.gu = with_tiles<BN, true>(f.gu);
  f.dn = with_tiles<BN, false>(f.dn);
  const int64_t mt_max = (d.R + BM - 1) / BM + d.E;    // row tiles, upper bound
  const int words = (int)(kFusedWords + mt_max);
  hipLaunchKernelGGL(fused_reset_kernel,
                     dim3((unsigned)((words + 255) / 256 < 64 ? (words + 255) / 256 : 64)),
                     dim3(256), 0, s, f.claim, words);
  int64_t g = device_cu_count();
  const int64_t work = mt_max * (f.gu.n_tiles + f.dn.n_tiles);
  if (g > work) g = work;
  if constexpr (SPLIT) {
    if (d.E <= 64)
      hipLaunchKernelGGL((grouped_ffn_fused_split<BM, BN, WM, WN, BK, S, 1>), dim3((unsigned)g),
                         dim3(64 * WM * WN), 0, s, f);
    else
      hipLaunchKernelGGL((grouped_ffn_fused_split<BM, BN, WM, WN, BK, S, 4>), dim3((unsigned)g),
                         dim3(64 * WM * WN), 0, s, f);
  } else {
    hipLaunchKernelGGL((grouped_ffn_fused<BM, BN, WM, WN, BK, S, false>), dim3((unsigned)g),
                       dim3(64 * WM * WN), 0, s, f);
  }
  return hipGetLastError();
}

}  // namespace

// Workspace of the fused FFN: h [R, F] bf16, then the 16 claim counters, the
// error word and one counter per row tile (row tiles of 32 rows bound those
// of every tile shape).
size_t fused_ws_bytes(const Dims& d) {
  return align_up((size_t)d.R * d.F * 2) +
         align_up((size_t)(kFusedWords + d.R / 32 + 1 + d.E) * 4);
}

size_t fused_err_offset(const Dims& d) { return align_up((size_t)d.R * d.F * 2) + 16 * 4; }

hipError_t launch_fused_ffn(const Dims& d, const uint16_t* x, const int32_t* row_token,
                            const int32_t* offsets, const uint16_t* wg, const uint16_t* wu,
                            const uint16_t* wd, uint16_t* out_perm, void* ws, hipStream_t s) {
  uint16_t* h = static_cast<uint16_t*>(ws);
  int32_t* words = reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                              align_up((size_t)d.R * d.F * 2));
  FusedArgs f;
  f.gu = GemmArgs{x, wg, wu, h, offsets, d.E, d.D, d.F, 0, nullptr, nullptr, nullptr, row_token};
  f.dn = GemmArgs{h, wd, nullptr, out_perm, offsets, d.E, d.F, d.D, 0, nullptr, nullptr, nullptr,
                  nullptr};
  f.claim = words;
  f.err = words + 16;
  f.done = words + kFusedWords;
  switch (pick(d)) {
    case Shape::Small: return launch_fused<32, 256, 1, 4, 64, 4>(d, f, s);
    case Shape::Mid: return launch_fused<128, 256, 2, 4, 64, 3>(d, f, s);
    default:
      // the split rings (three weight slots) when the work list fits in registers
      if (d.E <= 256) return launch_fused<256, 256, 2, 4, 64, 3, true>(d, f, s);
      return launch_fused<256, 256, 2, 4, 64, 2>(d, f, s);
  }
}

}  // namespace moe
