// Block-scaled FP8 expert weights: quantisation from bf16.
//
// FP8 weights in the grouped-GEMM kernel: "MoE 推理完整机制" (zoe.im), 第四层
// DeepGEMM & MegaMoE Kernel; 8-bit expert weights dequantised for use:
// "MoE工程实战" (jsqmd.com), 5.3 技巧2.  Format (OCP microscaling, FP8 E4M3
// elements): 32 consecutive values of a weight row share the scale 2^s, stored
// as the byte s + 127; s = floor(log2(largest finite |w| of the block)) - 8,
// clamped to [-117, 119] so that every dequantised value is a normal bf16
// number; each element is w / 2^s rounded to the nearest E4M3 value (ties to
// even), finite values beyond 448 saturate to 448 and non-finite values become
// NaN (0x7F | sign).
//
// Everything is exact integer work on the bf16 bit patterns.  One thread per
// 32-value block: four 16-byte loads, two 16-byte code stores, one scale byte.
// HBM-bound (2 bytes read, 1 + 1/32 written per weight).
#include "common.h"

namespace moe {
namespace {

// E4M3 code of the bf16 value with bits h, divided by 2^s (s in [-117, 119]).
__device__ __forceinline__ uint32_t e4m3_code(uint32_t h, int s) {
  const uint32_t sign = (h >> 8) & 0x80u;
  const uint32_t m = h & 0x7fffu;
  if (m >= 0x7f80u) return sign | 0x7fu;           // infinity or NaN
  const int eb = (int)(m >> 7);
  const uint32_t mb = m & 127u;
  const int et = eb - 127 - s;                    // exponent of |h| / 2^s (normal h)
  if (eb != 0 && et >= -6) {
    // normal E4M3: exponent field et + 7, top three mantissa bits, the low
    // four round the result (a carry moves into the exponent field)
    uint32_t c = ((uint32_t)(et + 7) << 3) | (mb >> 4);
    const uint32_t rem = mb & 15u;
    c += (rem > 8u || (rem == 8u && (c & 1u))) ? 1u : 0u;
    return sign | (c < 0x7eu ? c : 0x7eu);
  }
  // subnormal E4M3: |h| / 2^s in units of 2^-9 is mm * 2^-sh, sh >= 5
  const uint32_t mm = eb ? (128u | mb) : mb;
  const int sh = s + 125 - (eb ? eb : 1);
  if (sh >= 9) return sign;                         // below half a unit (mm < 256)
  uint32_t q = mm >> sh;
  const uint32_t rem = mm & ((1u << sh) - 1u), half = 1u << (sh - 1);
  q += (rem > half || (rem == half && (q & 1u))) ? 1u : 0u;
  return sign | q;
}

__global__ void __launch_bounds__(256)
quantize_fp8_kernel(const uint16_t* __restrict__ w, uint8_t* __restrict__ codes,
                    uint8_t* __restrict__ scales, int64_t nblk, int cols) {
  const int nbr = cols / 32;                      // blocks per row
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += stride) {
    const int64_t row = b / nbr;
    const int kb = (int)(b - row * nbr);
    const uint4* src = reinterpret_cast<const uint4*>(w + row * cols + (int64_t)kb * 32);
    uint32_t v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 t = src[i];
      v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
    }
    // largest finite magnitude (bit patterns of non-negative floats order
    // like their values)
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t lo = v[i] & 0x7fffu, hi = (v[i] >> 16) & 0x7fffu;
      if (lo < 0x7f80u) amax = max(amax, lo);
      if (hi < 0x7f80u) amax = max(amax, hi);
    }
    const int ea = (int)(amax >> 7);              // 0: zero or subnormal block maximum
    const int s = ea == 0 ? -117 : min(max(ea - 135, -117), 119);
    uint32_t q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t a = v[2 * i], c = v[2 * i + 1];
      q[i] = e4m3_code(a & 0xffffu, s) | (e4m3_code(a >> 16, s) << 8) |
             (e4m3_code(c & 0xffffu, s) << 16) | (e4m3_code(c >> 16, s) << 24);
    }
    uint4* dst = reinterpret_cast<uint4*>(codes + row * cols + (int64_t)kb * 32);
    dst[0] = make_uint4(q[0], q[1], q[2], q[3]);
    dst[1] = make_uint4(q[4], q[5], q[6], q[7]);
    scales[((row >> 5) * nbr + kb) * 32 + (row & 31)] = (uint8_t)(s + 127);
  }
}

}  // namespace

hipError_t launch_quantize_fp8(int64_t rows, int cols, const uint16_t* w, uint8_t* codes,
                               uint8_t* scales, hipStream_t s) {
  const int64_t nblk = rows * (cols / 32);
  const int64_t want = (nblk + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 16;
  const unsigned grid = (unsigned)(want < cap ? want : cap);
  hipLaunchKernelGGL(quantize_fp8_kernel, dim3(grid), dim3(256), 0, s, w, codes, scales, nblk,
                     cols);
  return hipGetLastError();
}

}  // namespace moe
