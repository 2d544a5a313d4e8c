// Token permutation into expert segments.
//
// "MoE 推理完整机制" (zoe.im), 第二层, 范式 A Step 1: tokens regrouped by expert
// into one contiguous buffer, expert_offsets kept as metadata for the later
// kernels; 范式 B: fixed per-expert capacity, filled in token order, overflow
// dropped.  Counts come from a histogram and offsets from an exclusive prefix
// sum, the same counting sort the A2A packer of "MoE 大规模分布式推理工程实战"
// (ybb.press) 2.2 runs over destination GPUs.
//
// Kernels (one stream, no host synchronisation):
//   0. small : for at most 1024 slots, steps 1-3 in one workgroup.
//   1. count : per-workgroup expert histogram of a chunk of slots.
//   2. scan  : per-expert exclusive prefix over workgroups, expert totals and
//              the segment offsets.
//   3. rank  : stable rank of every slot inside its expert, computed with wave
//              ballots (no atomics decide positions, so the layout is
//              deterministic); writes slot_row and row_token.
//   4. copy  : each token row is read once and written to its K rows.
//   5. pad   : (padded layout) row_token = -1 for the rows past each
//              expert's kept slots, and zero x_perm rows there when x_perm
//              is given.
#include <algorithm>

#include "common.h"

namespace moe {
namespace {

__device__ __forceinline__ bool valid_id(int id, int E) { return id >= 0 && id < E; }

__global__ void __launch_bounds__(256)
perm_count_kernel(int64_t S, int E, const int32_t* __restrict__ ids, int32_t* __restrict__ table) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kPermChunk;
  for (int i = threadIdx.x; i < kPermChunk; i += 256) {
    const int64_t s = base + i;
    if (s < S) {
      const int id = ids[s];
      if (valid_id(id, E)) atomicAdd(&hist[id], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) table[(int64_t)blockIdx.x * E + e] = hist[e];
}

// One workgroup of 1024 threads (E <= 1024).
__global__ void __launch_bounds__(1024)
perm_scan_kernel(int NB, int E, int64_t cap, int padded, int32_t* __restrict__ table,
                 int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  __shared__ int32_t sh[1024];
  const int e = threadIdx.x;
  int32_t total = 0;
  if (e < E) {
    // 16 block counts loaded together, then their exclusive prefix stored: the
    // loads of a group do not wait for one another (with one load and one
    // store per block the loads went out one round trip apart)
    constexpr int G = 16;
    for (int b0 = 0; b0 < NB; b0 += G) {
      int32_t t[G];
#pragma unroll
      for (int i = 0; i < G; ++i) t[i] = b0 + i < NB ? table[(int64_t)(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < G; ++i) {
        if (b0 + i < NB) table[(int64_t)(b0 + i) * E + e] = total;
        total += t[i];
      }
    }
    counts[e] = total;
  }
  sh[e] = (e < E) ? (padded ? (int32_t)cap : total) : 0;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = (e >= off) ? sh[e - off] : 0;
    __syncthreads();
    sh[e] += v;
    __syncthreads();
  }
  if (e < E) offsets[e + 1] = sh[e];
  if (e == 0) offsets[0] = 0;
}

// 4 waves; wave w ranks slots [base + 256w, base + 256w + 256) in 4 steps of 64.
__global__ void __launch_bounds__(256)
perm_rank_kernel(int64_t S, int E, int K, int nbits, int64_t cap, int padded,
                 const int32_t* __restrict__ ids, const int32_t* __restrict__ table,
                 const int32_t* __restrict__ offsets, int32_t* __restrict__ slot_row,
                 int32_t* __restrict__ row_token) {
  extern __shared__ int32_t run[];  // [4][E] per-wave running counts
  for (int i = threadIdx.x; i < 4 * E; i += 256) run[i] = 0;
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t base = (int64_t)blockIdx.x * kPermChunk + wave * 256;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int myid[4], local[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int64_t slot = base + s * 64 + lane;
    int id = slot < S ? ids[slot] : -1;
    const bool valid = valid_id(id, E);
    if (!valid) id = 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const int bit = (id >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & lt_mask);
    int old = 0;
    if (valid) old = run[wave * E + id];
    const int leader = __ffsll((unsigned long long)peers) - 1;
    if (valid && lane == leader) run[wave * E + id] = old + __popcll(peers);
    myid[s] = valid ? id : -1;
    local[s] = old + rank;
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int64_t slot = base + s * 64 + lane;
    if (slot >= S) continue;
    const int e = myid[s];
    int32_t row = -1;
    if (e >= 0) {
      int pre = 0;
      for (int w = 0; w < wave; ++w) pre += run[w * E + e];
      const int64_t pos = (int64_t)table[(int64_t)blockIdx.x * E + e] + pre + local[s];
      if (!padded) row = offsets[e] + (int32_t)pos;
      else if (pos < cap) row = (int32_t)(e * cap + pos);
    }
    slot_row[slot] = row;
    if (row >= 0) row_token[row] = (int32_t)(slot / K);
  }
}

// One thread per (token, 16-byte chunk), grid-stride: the chunk is read
// once and written to each kept row of the token (up to 8 slot rows are
// loaded before the stores).
__global__ void __launch_bounds__(256)
perm_copy_kernel(int64_t N, int D, int K, const uint16_t* __restrict__ x,
                 const int32_t* __restrict__ slot_row, uint16_t* __restrict__ x_perm) {
  const int cpr = D / 8;
  const int64_t items = N * cpr;
  for (int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x; item < items;
       item += (int64_t)gridDim.x * 256) {
    const int64_t n = item / cpr;
    const int c = (int)(item % cpr);
    const uint4 v = reinterpret_cast<const uint4*>(x + n * D)[c];
    for (int k0 = 0; k0 < K; k0 += 8) {
      int32_t r[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = k0 + j < K ? slot_row[n * K + k0 + j] : -1;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (r[j] >= 0) reinterpret_cast<uint4*>(x_perm + (int64_t)r[j] * D)[c] = v;
    }
  }
}

// Many tokens with wide rows: one workgroup per token (grid-stride over
// tokens), as many threads as the row has chunks rounded up to a wave (at
// most 1024).  The token's K slot rows are wave-uniform and come through
// scalar loads, so the vector-memory path carries only the row itself, and a
// token whose slots were all dropped (capacity) reads nothing.  Same bytes
// written as perm_copy_kernel.
__global__ void __launch_bounds__(1024)
perm_copy_token_kernel(int64_t N, int D, int K, const uint16_t* __restrict__ x,
                       const int32_t* __restrict__ slot_row, uint16_t* __restrict__ x_perm) {
  const int cpr = D / 8;
  for (int64_t n = blockIdx.x; n < N; n += gridDim.x) {
    int kept = 0;
    for (int k = 0; k < K; ++k) kept |= slot_row[n * K + k] >= 0;
    if (!kept) continue;   // the same for every thread of the workgroup
    for (int c = threadIdx.x; c < cpr; c += blockDim.x) {
      const uint4 v = reinterpret_cast<const uint4*>(x + n * D)[c];
      for (int k0 = 0; k0 < K; k0 += 8) {
        int32_t r[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j] = k0 + j < K ? slot_row[n * K + k0 + j] : -1;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (r[j] >= 0) reinterpret_cast<uint4*>(x_perm + (int64_t)r[j] * D)[c] = v;
      }
    }
  }
}

// Small problems (N*K <= 1024 slots): histogram, scan and stable rank in one
// workgroup of 16 waves; wave w ranks slots [64w, 64w + 64).  Same results as
// count + scan + rank.
constexpr int kSmallSlots = 1024;
__global__ void __launch_bounds__(1024)
perm_small_kernel(int64_t S, int E, int K, int nbits, int64_t cap, int padded,
                  const int32_t* __restrict__ ids, int32_t* __restrict__ counts,
                  int32_t* __restrict__ offsets, int32_t* __restrict__ slot_row,
                  int32_t* __restrict__ row_token) {
  __shared__ int32_t wcnt[16 * 1024];   // [wave][expert]: count, then exclusive prefix over waves
  __shared__ int32_t sh[1024];          // per-expert segment sizes, then inclusive prefix
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < 16 * E; i += 1024) wcnt[i] = 0;
  __syncthreads();
  const int64_t slot = tid;
  int id = slot < S ? ids[slot] : -1;
  const bool valid = valid_id(id, E);
  if (!valid) id = 0;
  uint64_t peers = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const int bit = (id >> b) & 1;
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank = __popcll(peers & lt_mask);
  if (valid && lane == __ffsll((unsigned long long)peers) - 1) wcnt[wave * E + id] = __popcll(peers);
  __syncthreads();
  if (tid < E) {
    int32_t run = 0;
    for (int w = 0; w < 16; ++w) {
      const int32_t t = wcnt[w * E + tid];
      wcnt[w * E + tid] = run;
      run += t;
    }
    counts[tid] = run;
    sh[tid] = padded ? (int32_t)cap : run;
  } else {
    sh[tid] = 0;
  }
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += v;
    __syncthreads();
  }
  if (tid < E) offsets[tid + 1] = sh[tid];
  if (tid == 0) offsets[0] = 0;
  if (slot < S) {
    int32_t row = -1;
    if (valid) {
      const int64_t pos = (int64_t)wcnt[wave * E + id] + rank;
      if (!padded) row = (id ? sh[id - 1] : 0) + (int32_t)pos;
      else if (pos < cap) row = (int32_t)(id * cap + pos);
    }
    slot_row[slot] = row;
    if (row >= 0) row_token[row] = (int32_t)(slot / K);
  }
}

// Padded layout: rows [e*cap + min(count_e, cap), (e+1)*cap) are padding:
// row_token = -1 and, when x_perm is given, a zero row.  Grid-stride over all
// E*cap rows (many workgroups, each row's test is one cached load of its
// expert's count); a workgroup writes a padding row with 16-byte stores.
__global__ void __launch_bounds__(256)
perm_pad_kernel(int64_t R, int64_t cap, int D, const int32_t* __restrict__ counts,
                int32_t* __restrict__ row_token, uint16_t* __restrict__ x_perm) {
  const int cpr = D / 8;
  const uint4 z = {0u, 0u, 0u, 0u};
  for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
    const int64_t e = r / cap;
    const int64_t kept = min<int64_t>(counts[e], cap);
    if (r - e * cap < kept) continue;             // a kept row (workgroup-uniform)
    if (threadIdx.x == 0) row_token[r] = -1;
    if (x_perm) {
      uint4* row = reinterpret_cast<uint4*>(x_perm + r * D);
      for (int c = threadIdx.x; c < cpr; c += 256) row[c] = z;
    }
  }
}

}  // namespace

size_t permute_ws_bytes(const Dims& d) {
  const int64_t nb = (d.S + kPermChunk - 1) / kPermChunk;
  return align_up((size_t)nb * d.E * sizeof(int32_t));
}

hipError_t launch_permute(const Dims& d, const uint16_t* x, const int32_t* ids, int32_t* counts,
                          int32_t* offsets, int32_t* row_token, int32_t* slot_row,
                          uint16_t* x_perm, void* ws, hipStream_t s) {
  const int nb = (int)((d.S + kPermChunk - 1) / kPermChunk);
  int32_t* table = static_cast<int32_t*>(ws);
  int nbits = 0;
  while ((1 << nbits) < d.E) ++nbits;
  if (d.S <= kSmallSlots) {
    hipLaunchKernelGGL(perm_small_kernel, dim3(1), dim3(1024), 0, s, d.S, d.E, d.K, nbits, d.cap,
                       (int)d.padded, ids, counts, offsets, slot_row, row_token);
  } else {
    hipLaunchKernelGGL(perm_count_kernel, dim3(nb), dim3(256), d.E * sizeof(int32_t), s, d.S,
                       d.E, ids, table);
    hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, s, nb, d.E, d.cap,
                       (int)d.padded, table, counts, offsets);
    hipLaunchKernelGGL(perm_rank_kernel, dim3(nb), dim3(256), 4 * d.E * sizeof(int32_t), s, d.S,
                       d.E, d.K, nbits, d.cap, (int)d.padded, ids, table, offsets, slot_row,
                       row_token);
  }
  if (d.padded) {
    // padding rows: row_token = -1 always, zero rows when x_perm is given
    const int64_t blocks = std::min<int64_t>(d.R, 8 * (int64_t)device_cu_count());
    hipLaunchKernelGGL(perm_pad_kernel, dim3((unsigned)blocks), dim3(256), 0, s, d.R, d.cap, d.D,
                       counts, row_token, x_perm);
  }
  if (!x_perm) return hipGetLastError();      // routing tables only
  if (d.N >= 1024 && d.D >= 1024) {
    const int cpr = d.D / 8;
    const int threads = std::min(1024, (cpr + 63) / 64 * 64);
    const int64_t blocks = std::min<int64_t>(d.N, 1 << 20);
    hipLaunchKernelGGL(perm_copy_token_kernel, dim3((unsigned)blocks), dim3(threads), 0, s, d.N,
                       d.D, d.K, x, slot_row, x_perm);
    return hipGetLastError();
  }
  const int64_t items = d.N * (d.D / 8);
  const int64_t blocks = std::min<int64_t>((items + 255) / 256, 1 << 20);
  hipLaunchKernelGGL(perm_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s, d.N, d.D, d.K, x,
                     slot_row, x_perm);
  return hipGetLastError();
}

}  // namespace moe
