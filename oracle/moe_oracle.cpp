// Plain C++17 CPU oracle of the single-GPU MoE-layer forward pass.
//
// TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
// benchmark's CPU-baseline leg load this library (oracle/liboracle.so, through
// oracle/cpp.py).  The product library never links or calls it, and the two
// share no source: this file includes only the C++ standard library.
//
// What it computes, in the order of the pages ("MoE 推理完整机制：从 Router 到
// Expert Parallelism 的一切", zoe.im, below [zoe]; "MoE 大规模分布式推理工程实战",
// ybb.press, below [ybb]; "MoE工程实战：从门控路由到All-to-All通信的全栈优化",
// jsqmd.com, below [jsq]):
//   1. router logits = W_gate x, a bias-free linear layer        [zoe] 第一层; [ybb] 4.1
//   2. key = logit + per-expert bias (one fp32 add)              [ybb] 4.1
//   3. top-K of the keys, sorted, ties to the lower expert id    [zoe] 第一层
//   4. weights: softmax over the K selected keys, or
//      sigmoid(key) divided by the sum over the K selected       [zoe] 第一层, sigmoid + norm
//   5. counts by histogram, expert_offsets by exclusive prefix   [zoe] 范式 A Step 1; [ybb] 2.2
//   6. every slot n*K+k, in ascending order, takes the next row
//      of its expert's segment                                   [zoe] 范式 A worked example
//   7. capacity-padded variant: cap = ceil(num*N*K/(den*E)),
//      first cap slots of an expert kept, the rest dropped        [zoe] 范式 B; [jsq] 3.2
//   8. per expert, on its rows: g = x Wg^T, u = x Wu^T,
//      h = silu(g) * u, out = h Wd^T (SwiGLU; two GEMMs)          [zoe] 范式 A Step 2
//   9. y[n] = sum_k w[n,k] * out[row of slot n*K+k]               [zoe] 范式 A Step 3
//
// Precision: every sum is a float64 sum (each product of a bf16 and a bf16 or
// fp32 value is exact in float64), taken in index order.  Values are rounded
// where the GPU stores or holds them: logits, g, u, silu(g)*u, the down dot
// and the combine sum to fp32 (IEEE round to nearest even); h, out_perm and y
// then to bf16 (round to nearest even).  The router weights are computed in
// float64 and rounded to fp32.
//
// Readings where the pages are silent (shared with the numpy oracle):
// -0.0 == +0.0 and NaN keys rank below every number; the K outputs are in
// descending key order; sigmoid gating selects on the key itself (sigmoid is
// increasing); a selected set whose weight denominator is zero gets 1/K each;
// ids outside [0, E) mark a dropped slot; dropped slots contribute nothing and
// the kept weights are not renormalised; padding rows are zero rows.
//
// Parallelism: OpenMP over independent outputs only (tokens, or the output
// columns of one expert), each output summed by one thread in index order, so
// the results do not depend on the thread count.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

// ------------------------------------------------------------ number formats

// bf16 bit pattern -> its value (exact: bf16 is the top half of an fp32).
double bf16_value(uint16_t bits) {
  const uint32_t u = static_cast<uint32_t>(bits) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return static_cast<double>(f);
}

// Round a value to bf16, nearest even, and return its bit pattern.  The value
// is written as m * 2^e with 0.5 <= |m| < 1; m * 2^8 rounded to an integer
// (nearbyint: ties to even in the default rounding mode) keeps 8 significant
// bits.  The rounded value is exact in fp32, whose top half is the bf16
// pattern.  Zero keeps its sign; infinities and NaN pass through (a NaN
// becomes the quiet NaN 0x7fc0).
uint16_t bf16_bits(double v) {
  if (std::isnan(v)) return 0x7fc0;
  double r = v;
  if (std::isfinite(v) && v != 0.0) {
    int e = 0;
    const double m = std::frexp(v, &e);
    r = std::ldexp(std::nearbyint(std::ldexp(m, 8)), e - 8);
  }
  const float f = static_cast<float>(r);
  uint32_t u;
  std::memcpy(&u, &f, sizeof u);
  return static_cast<uint16_t>(u >> 16);
}

// fp32 rounding of a float64 value (IEEE conversion, nearest even).
double fl32(double v) { return static_cast<double>(static_cast<float>(v)); }

// The value at bf16 storage: fp32 first (the GPU's arithmetic type), then bf16.
uint16_t store_bf16(double v) { return bf16_bits(fl32(v)); }

// ------------------------------------------------------------ router and gating

// Selection key: fp32 logit + fp32 bias, one fp32 add; -0 -> +0, NaN -> -inf.
float gating_key(float logit, const float* bias, int e) {
  float k = logit;
  if (bias) {
    volatile float b = bias[e];   // one IEEE fp32 addition, as written
    k = logit + b;
  }
  if (k == 0.0f) k = 0.0f;
  if (std::isnan(k)) k = -INFINITY;
  return k;
}

// One token: sort all E keys by (key descending, id ascending), take K; then
// the weights of the K selected keys.
void route_token(const float* logits_row, const float* bias, int E, int K, int gating,
                 int32_t* ids, float* weights, std::vector<int>& order, std::vector<float>& key) {
  for (int e = 0; e < E; ++e) key[e] = gating_key(logits_row[e], bias, e);
  std::iota(order.begin(), order.end(), 0);
  std::sort(order.begin(), order.end(), [&](int a, int b) {
    if (key[a] != key[b]) return key[a] > key[b];
    return a < b;
  });
  double z[64];
  double tot = 0.0;
  if (gating == 0) {   // softmax over the K selected keys, max subtracted
    const double kmax = key[order[0]];
    for (int j = 0; j < K; ++j) {
      z[j] = std::isfinite(kmax) ? std::exp(static_cast<double>(key[order[j]]) - kmax) : 0.0;
      tot += z[j];
    }
  } else {             // sigmoid of each selected key, renormalised
    for (int j = 0; j < K; ++j) {
      z[j] = 1.0 / (1.0 + std::exp(-static_cast<double>(key[order[j]])));
      tot += z[j];
    }
  }
  for (int j = 0; j < K; ++j) {
    ids[j] = order[j];
    weights[j] = static_cast<float>(tot > 0.0 ? z[j] / tot : 1.0 / K);
  }
}

// ------------------------------------------------------------ expert FFN

// One expert's SwiGLU FFN on m rows.  rows[i] points at row i's D bf16
// values (nullptr: a zero row).  wg, wu: [F, D] bf16; wd: [D, F] bf16.
// h: [m, F] bf16 out; out: [m, D] bf16 out (either may be nullptr).
void swiglu_expert(int64_t m, const uint16_t* const* rows, int D, int F, const uint16_t* wg,
                   const uint16_t* wu, const uint16_t* wd, uint16_t* h_out, uint16_t* out) {
  if (m == 0) return;
  std::vector<double> xv(static_cast<size_t>(m) * D);      // the rows' values
  for (int64_t i = 0; i < m; ++i)
    for (int d = 0; d < D; ++d)
      xv[i * D + d] = rows[i] ? bf16_value(rows[i][d]) : 0.0;
  std::vector<double> hv(static_cast<size_t>(m) * F);      // h as stored (bf16 values)
  // g, u and h: one output column j of every row per iteration
#pragma omp parallel for schedule(static)
  for (int j = 0; j < F; ++j) {
    std::vector<double> wgj(D), wuj(D);
    for (int d = 0; d < D; ++d) {
      wgj[d] = bf16_value(wg[static_cast<size_t>(j) * D + d]);
      wuj[d] = bf16_value(wu[static_cast<size_t>(j) * D + d]);
    }
    for (int64_t i = 0; i < m; ++i) {
      const double* xi = &xv[i * D];
      double g = 0.0, u = 0.0;
      for (int d = 0; d < D; ++d) {
        g += xi[d] * wgj[d];
        u += xi[d] * wuj[d];
      }
      g = fl32(g);
      u = fl32(u);
      const double silu = g / (1.0 + std::exp(-g));
      const uint16_t hb = store_bf16(silu * u);
      hv[i * F + j] = bf16_value(hb);
      if (h_out) h_out[i * F + j] = hb;
    }
  }
  if (!out) return;
  // out = h Wd^T: one output column c of every row per iteration
#pragma omp parallel for schedule(static)
  for (int c = 0; c < D; ++c) {
    std::vector<double> wdc(F);
    for (int j = 0; j < F; ++j) wdc[j] = bf16_value(wd[static_cast<size_t>(c) * F + j]);
    for (int64_t i = 0; i < m; ++i) {
      const double* hi = &hv[i * F];
      double o = 0.0;
      for (int j = 0; j < F; ++j) o += hi[j] * wdc[j];
      out[i * D + c] = store_bf16(o);
    }
  }
}

// ------------------------------------------------------------ FP8 weights
//
// Block-scaled FP8 expert weights ([zoe] 第四层 DeepGEMM & MegaMoE Kernel: FP8
// weights; [jsq] 5.3 技巧2: 8-bit expert weights dequantised for use).  The
// pages fix no format; the reading is the OCP microscaling layout with E4M3
// elements: 32 consecutive values along a weight row's contraction axis share
// a power-of-two scale 2^s, stored as the byte s + 127.

constexpr double kE4m3Max = 448.0;
constexpr int kScaleMin = -117;   // every dequantised value stays a normal bf16 number
constexpr int kScaleMax = 119;

// floor(log2 a) for a finite a > 0.
int floor_log2(double a) {
  int e = 0;
  std::frexp(a, &e);             // a = m 2^e, 0.5 <= m < 1
  return e - 1;
}

// A value to the nearest E4M3 code, ties to even, saturating at +-448; a
// non-finite value gives the NaN code 0x7f with the value's sign bit.
// E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is
// subnormal (M * 2^-9); S.1111.111 is NaN; the largest finite value is 448.
uint8_t e4m3_encode(double t) {
  const uint8_t sign = std::signbit(t) ? 0x80 : 0x00;
  if (!std::isfinite(t)) return sign | 0x7f;
  const double a = std::min(std::fabs(t), kE4m3Max);
  // grid step: 2^(floor(log2 a) - 3) in the normal range, 2^-9 below 2^-6
  const int step = a >= std::ldexp(1.0, -6) ? floor_log2(a) - 3 : -9;
  const double v = std::ldexp(std::nearbyint(std::ldexp(a, -step)), step);
  if (v >= std::ldexp(1.0, -6)) {
    const int e = floor_log2(v);                                   // carry may raise it
    const int man = static_cast<int>(std::ldexp(v, -e) * 8.0 - 8.0);   // exact, 0..7
    return sign | static_cast<uint8_t>(((e + 7) << 3) | man);
  }
  return sign | static_cast<uint8_t>(std::ldexp(v, 9));           // subnormal: v / 2^-9
}

double e4m3_decode(uint8_t c) {
  const int ef = (c >> 3) & 15, mf = c & 7;
  double mag;
  if (ef == 15 && mf == 7) mag = NAN;
  else if (ef == 0) mag = std::ldexp(static_cast<double>(mf), -9);
  else mag = std::ldexp(static_cast<double>(8 + mf), ef - 10);
  return (c & 0x80) ? -mag : mag;
}

}  // namespace

extern "C" {

// Quantise bf16 weights [rows, cols] (cols a multiple of 32): per block of 32
// consecutive values of a row, s = floor(log2(largest finite |w|)) - 8
// clamped to [-117, 119] (an all-zero block takes -117), so the block's
// largest value lands in E4M3's top binade [256, 512); code = E4M3(w / 2^s)
// (the division by a power of two is exact); scale byte = s + 127.
// codes [rows, cols], scales [rows, cols / 32].
void oracle_quantize_fp8(int64_t rows, int cols, const uint16_t* w, uint8_t* codes,
                         uint8_t* scales) {
  const int nb = cols / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int b = 0; b < nb; ++b) {
      const size_t o = static_cast<size_t>(r) * cols + 32 * b;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i) {
        const double v = bf16_value(w[o + i]);
        if (std::isfinite(v)) amax = std::max(amax, std::fabs(v));
      }
      int s = amax > 0.0 ? floor_log2(amax) - 8 : kScaleMin;
      s = std::min(std::max(s, kScaleMin), kScaleMax);
      for (int i = 0; i < 32; ++i) codes[o + i] = e4m3_encode(std::ldexp(bf16_value(w[o + i]), -s));
      scales[static_cast<size_t>(r) * nb + b] = static_cast<uint8_t>(s + 127);
    }
  }
}

// Dequantise: value = E4M3(code) * 2^(byte - 127), as bf16 bits (exact for the
// scale bytes the quantiser writes).  w [rows, cols] out.
void oracle_dequantize_fp8(int64_t rows, int cols, const uint8_t* codes, const uint8_t* scales,
                           uint16_t* w) {
  const int nb = cols / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int c = 0; c < cols; ++c) {
      const size_t o = static_cast<size_t>(r) * cols + c;
      const int s = static_cast<int>(scales[static_cast<size_t>(r) * nb + c / 32]) - 127;
      w[o] = bf16_bits(std::ldexp(e4m3_decode(codes[o]), s));
    }
}


int oracle_version(void) { return 1; }

// Threads the OpenMP runtime uses for the parallel loops.
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

// logits[n, e] = fl32(sum_d x[n, d] * w_router[e, d]); x [N, D] bf16 bits,
// w_router [E, D] fp32 (nn.Linear layout), logits [N, E] fp32.
void oracle_router_logits(int64_t N, int D, int E, const uint16_t* x, const float* w_router,
                          float* logits) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    std::vector<double> xn(D);
    for (int d = 0; d < D; ++d) xn[d] = bf16_value(x[n * D + d]);
    for (int e = 0; e < E; ++e) {
      const float* w = w_router + static_cast<size_t>(e) * D;
      double s = 0.0;
      for (int d = 0; d < D; ++d) s += xn[d] * static_cast<double>(w[d]);
      logits[n * E + e] = static_cast<float>(s);
    }
  }
}

// Capacity per expert, ceil(num * N * K / (den * E)) in exact integer
// arithmetic ([zoe] 范式 B with the factor num/den; [jsq] 3.2 tokens*k/E*factor).
int64_t oracle_capacity(int64_t N, int K, int E, int64_t num, int64_t den) {
  const __int128 a = static_cast<__int128>(num) * N * K;
  const __int128 b = static_cast<__int128>(den) * E;
  return static_cast<int64_t>((a + b - 1) / b);
}

// Top-K ids [N, K] and weights [N, K] from fp32 logits [N, E] and an optional
// bias [E]; gating 0 = softmax over the selected, 1 = sigmoid renormalised.
// K <= min(E, 64).
void oracle_route(int64_t N, int E, int K, int gating, const float* logits, const float* bias,
                  int32_t* ids, float* weights) {
#pragma omp parallel
  {
    std::vector<int> order(E);
    std::vector<float> key(E);
#pragma omp for schedule(static)
    for (int64_t n = 0; n < N; ++n)
      route_token(logits + n * E, bias, E, K, gating, ids + n * K, weights + n * K, order, key);
  }
}

// Counting sort of the N*K slots by expert.  cap == 0: contiguous segments,
// R = N*K rows; cap > 0: padded segments [e*cap, (e+1)*cap), R = E*cap rows.
// counts [E] (raw, before drops), offsets [E+1], row_token [R] (-1 for
// padding rows), slot_row [N*K] (-1 for dropped slots).
void oracle_permute(int64_t N, int K, int E, int64_t cap, const int32_t* ids, int32_t* counts,
                    int32_t* offsets, int32_t* row_token, int32_t* slot_row) {
  const int64_t S = N * K;
  std::vector<int64_t> cnt(E, 0);
  for (int64_t i = 0; i < S; ++i)
    if (ids[i] >= 0 && ids[i] < E) ++cnt[ids[i]];
  std::vector<int64_t> off(E + 1, 0);
  for (int e = 0; e < E; ++e) off[e + 1] = cap > 0 ? (e + 1) * cap : off[e] + cnt[e];
  const int64_t R = cap > 0 ? E * cap : S;
  for (int64_t r = 0; r < R; ++r) row_token[r] = -1;
  std::vector<int64_t> run(E, 0);
  for (int64_t i = 0; i < S; ++i) {
    const int e = ids[i];
    int64_t row = -1;
    if (e >= 0 && e < E) {
      if (cap == 0 || run[e] < cap) {
        row = off[e] + run[e];
        row_token[row] = static_cast<int32_t>(i / K);
      }
      ++run[e];
    }
    slot_row[i] = static_cast<int32_t>(row);
  }
  for (int e = 0; e < E; ++e) counts[e] = static_cast<int32_t>(cnt[e]);
  for (int e = 0; e <= E; ++e) offsets[e] = static_cast<int32_t>(off[e]);
}

// The grouped FFN over given rows.  Row i belongs to expert row_expert[i] and
// holds x[row_token[i]] (row_token < 0: a zero row).  x [N, D] bf16;
// w_gate, w_up [E, F, D] bf16; w_down [E, D, F] bf16; h [nrows, F] and
// out [nrows, D] bf16 out (h may be nullptr).  Experts are taken one at a
// time (all rows of one expert together), so the weights stream once.
void oracle_ffn_rows(int64_t nrows, const int32_t* row_expert, const int32_t* row_token,
                     const uint16_t* x, int D, int F, int E, const uint16_t* w_gate,
                     const uint16_t* w_up, const uint16_t* w_down, uint16_t* h, uint16_t* out) {
  std::vector<std::vector<int64_t>> by_e(E);
  for (int64_t i = 0; i < nrows; ++i)
    if (row_expert[i] >= 0 && row_expert[i] < E) by_e[row_expert[i]].push_back(i);
  const size_t mat = static_cast<size_t>(F) * D;
  for (int e = 0; e < E; ++e) {
    const std::vector<int64_t>& rs = by_e[e];
    const int64_t m = static_cast<int64_t>(rs.size());
    if (m == 0) continue;
    std::vector<const uint16_t*> rows(m);
    for (int64_t i = 0; i < m; ++i)
      rows[i] = row_token[rs[i]] >= 0 ? x + static_cast<size_t>(row_token[rs[i]]) * D : nullptr;
    std::vector<uint16_t> he(static_cast<size_t>(m) * F), oe(static_cast<size_t>(m) * D);
    swiglu_expert(m, rows.data(), D, F, w_gate + e * mat, w_up + e * mat, w_down + e * mat,
                  he.data(), oe.data());
    for (int64_t i = 0; i < m; ++i) {
      if (h) std::memcpy(h + rs[i] * F, &he[i * F], sizeof(uint16_t) * F);
      std::memcpy(out + rs[i] * D, &oe[i * D], sizeof(uint16_t) * D);
    }
  }
}

// Every expert's FFN over its own segment of a permuted buffer: rows
// [offsets[e], offsets[e+1]) of x_perm [R, D] belong to expert e; rows outside
// every segment are left as they are.  h [R, F] (or nullptr), out_perm [R, D].
void oracle_expert_ffn(int64_t R, int D, int F, int E, const uint16_t* x_perm,
                       const int32_t* offsets, const uint16_t* w_gate, const uint16_t* w_up,
                       const uint16_t* w_down, uint16_t* h, uint16_t* out_perm) {
  const size_t mat = static_cast<size_t>(F) * D;
  for (int e = 0; e < E; ++e) {
    const int64_t lo = offsets[e], hi = std::min<int64_t>(offsets[e + 1], R);
    if (hi <= lo) continue;   // empty expert: skipped ([jsq] 4.2, numel() > 0)
    std::vector<const uint16_t*> rows(hi - lo);
    for (int64_t r = lo; r < hi; ++r) rows[r - lo] = x_perm + r * D;
    swiglu_expert(hi - lo, rows.data(), D, F, w_gate + e * mat, w_up + e * mat, w_down + e * mat,
                  h ? h + lo * F : nullptr, out_perm + lo * D);
  }
}

// y[n] = bf16(fl32(sum over k in order, slot kept, of w[n,k] * out_perm[slot_row[n*K+k]])).
void oracle_combine(int64_t N, int K, int D, const uint16_t* out_perm, const int32_t* slot_row,
                    const float* weights, uint16_t* y) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    for (int c = 0; c < D; ++c) {
      double s = 0.0;
      for (int k = 0; k < K; ++k) {
        const int32_t r = slot_row[n * K + k];
        if (r < 0) continue;
        s += static_cast<double>(weights[n * K + k]) * bf16_value(out_perm[(int64_t)r * D + c]);
      }
      y[n * D + c] = store_bf16(s);
    }
  }
}

// The whole layer on N tokens.  logits [N, E], ids [N, K], weights [N, K],
// counts [E], offsets [E+1], row_token [R], slot_row [N*K], out_perm [R, D]
// and y [N, D] are outputs; h [R, F] is an output or nullptr.  With
// logits_given != 0 the logits are an input and the router GEMM is skipped.
// cap as in oracle_permute.  The permuted copy of x is not materialised:
// each expert reads its rows of x through row_token.
void oracle_forward(int64_t N, int D, int E, int K, int F, int gating, int64_t cap,
                    const uint16_t* x, const float* w_router, const float* bias,
                    const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                    int logits_given, float* logits, int32_t* ids, float* weights,
                    int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* slot_row,
                    uint16_t* h, uint16_t* out_perm, uint16_t* y) {
  if (!logits_given) oracle_router_logits(N, D, E, x, w_router, logits);
  oracle_route(N, E, K, gating, logits, bias, ids, weights);
  oracle_permute(N, K, E, cap, ids, counts, offsets, row_token, slot_row);
  const int64_t R = cap > 0 ? E * cap : N * K;
  std::vector<int32_t> row_expert(R, -1);
  for (int e = 0; e < E; ++e)
    for (int64_t r = offsets[e]; r < offsets[e + 1]; ++r) row_expert[r] = e;
  // padding rows (row_token -1) are zero rows of their expert's segment
  oracle_ffn_rows(R, row_expert.data(), row_token, x, D, F, E, w_gate, w_up, w_down, h, out_perm);
  oracle_combine(N, K, D, out_perm, slot_row, weights, y);
}

}  // extern "C"
