// Routing statistics and dynamic expert bias.
//
// "MoE 大规模分布式推理工程实战" (ybb.press), 4.1 Router 辅助损失的工程化实现:
// the batch's fraction of slots per expert is folded into an exponential
// moving average, and the per-expert bias added to the router logits moves by
// (E * normalised EMA - 1) * step.  Fed by the expert_counts of moe_permute.
//
// One workgroup of 1024 threads (E <= 1024), fp32 arithmetic; the two sums
// over experts are tree reductions in a fixed order, so the result does not
// depend on scheduling.
#include "common.h"

namespace moe {
namespace {

// Sum of v over the workgroup's 1024 threads, fixed order; all threads get it.
template <typename T>
__device__ __forceinline__ T block_sum(T v, T* sh) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (t < w) sh[t] = sh[t] + sh[t + w];
    __syncthreads();
  }
  const T r = sh[0];
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(1024)
routing_stats_kernel(int E, const int32_t* __restrict__ counts, float* __restrict__ ema,
                     float* __restrict__ bias, float decay, float step) {
  __shared__ int64_t shi[1024];
  __shared__ float shf[1024];
  const int e = threadIdx.x;
  const int64_t c = e < E ? (int64_t)counts[e] : 0;
  const int64_t tot = block_sum<int64_t>(c, shi);
  if (tot == 0) return;                      // an empty batch changes nothing
  float m = 0.f;
  if (e < E) {
    const float f = (float)c / (float)tot;
    m = decay * ema[e] + (1.f - decay) * f;
  }
  const float msum = block_sum<float>(m, shf);
  if (e < E) {
    ema[e] = m;
    const float frac = m / msum;
    bias[e] = bias[e] + ((float)E * frac - 1.f) * step;
  }
}

}  // namespace

hipError_t launch_routing_stats(int E, const int32_t* counts, float* ema, float* bias, float decay,
                                float step, hipStream_t s) {
  hipLaunchKernelGGL(routing_stats_kernel, dim3(1), dim3(1024), 0, s, E, counts, ema, bias, decay,
                     step);
  return hipGetLastError();
}

}  // namespace moe
