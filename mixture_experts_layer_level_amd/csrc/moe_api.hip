// C ABI of libmoe: argument checks, workspace layout and launch sequencing.
// Every check runs on the host before the first HIP call of an entry point.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>

#include "common.h"

// Scratch of moe_forward_static, the entry point for callers that cannot
// allocate: the workspace of moe_forward for problems that need at most
// MOE_STATIC_SCRATCH_BYTES.  Each GPU the library runs on holds its own copy
// for as long as the process lives.  In host code this name is only a handle:
// its device address comes from hipGetSymbolAddress (static_scratch below).
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

namespace moe {

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

inline bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }


moe_status check_problem(const moe_problem* p, Dims* d) {
  if (!p) return MOE_ERR_INVALID_ARG;
  if (p->num_tokens < 0 || p->hidden <= 0 || p->ffn <= 0 || p->num_experts < 1 ||
      p->top_k < 1 || p->top_k > p->num_experts)
    return MOE_ERR_INVALID_ARG;
  if (p->gating != MOE_GATING_SOFTMAX_TOPK && p->gating != MOE_GATING_SIGMOID_RENORM)
    return MOE_ERR_INVALID_ARG;
  if (p->capacity_num < 0 || (p->capacity_num > 0 && p->capacity_den <= 0))
    return MOE_ERR_INVALID_ARG;
  if (p->hidden % 64 != 0 || p->ffn % 64 != 0 || p->num_experts > 1024 || p->top_k > 64)
    return MOE_ERR_UNSUPPORTED;
  d->N = p->num_tokens;
  d->D = p->hidden;
  d->F = p->ffn;
  d->E = p->num_experts;
  d->K = p->top_k;
  d->gating = p->gating;
  d->S = d->N * d->K;
  d->padded = p->capacity_num > 0;
  if (d->padded) {
    // cap = ceil(num * S / (den * E)) in exact 128-bit integer arithmetic
    const __int128 num = (__int128)p->capacity_num * d->S;
    const __int128 den = (__int128)p->capacity_den * d->E;
    const __int128 cap = (num + den - 1) / den;
    if (cap > (1ll << 31)) return MOE_ERR_UNSUPPORTED;
    d->cap = (int64_t)cap;
    d->R = d->cap * d->E;
  } else {
    d->cap = 0;
    d->R = d->S;
  }
  // row and slot indices are int32 on the device, as are element offsets
  // inside one expert's weight matrix
  if (d->S >= (1ll << 31) || d->R >= (1ll << 31) || (int64_t)d->D * d->F >= (1ll << 31))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

struct ForwardWs {
  size_t logits, ids, weights, counts, offsets, row_token, slot_row, x_perm, out_perm, perm,
      ffn, feats, roff, fused, rpart, total;
};

// One layout serves every forward entry point.  Regions whose uses never
// overlap in time share memory:
//   - the routing scratch (the split router's partial logits, the MLP
//     router's features and its GEMM's offsets) is dead once top-K has run,
//     before the permutation writes x_perm;
//   - x_perm is read only by the gate/up GEMM, which has finished before the
//     down GEMM writes out_perm over it (the fused launch, which writes
//     out_perm while it reads its rows, takes them from x, not x_perm);
//   - the permutation's scratch, the FFN's h and the fused launch's h and
//     counters belong to successive launches (the fused launch clears its
//     counters itself).
ForwardWs forward_layout(const Dims& d) {
  ForwardWs w;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes);
    return at;
  };
  w.logits = take((size_t)d.N * d.E * 4);
  w.ids = take((size_t)d.S * 4);
  w.weights = take((size_t)d.S * 4);
  w.counts = take((size_t)d.E * 4);
  w.offsets = take((size_t)(d.E + 1) * 4);
  w.row_token = take((size_t)d.R * 4);
  w.slot_row = take((size_t)d.S * 4);
  const size_t feats = align_up((size_t)d.N * (d.D / 4) * 2);   // MLP router features
  const size_t rows = std::max({(size_t)d.R * d.D * 2, router_ws_bytes(d), feats + align_up(2 * 4)});
  w.x_perm = w.out_perm = w.rpart = w.feats = take(rows);
  w.roff = w.feats + feats;
  w.perm = w.ffn = w.fused = take(std::max({permute_ws_bytes(d), ffn_ws_bytes(d),
                                            fused_ws_bytes(d)}));
  w.total = o;
  return w;
}

thread_local hipError_t t_last_hip_error = hipSuccess;

inline moe_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  t_last_hip_error = e;
  return MOE_ERR_HIP;
}

// The layer: the routing given by `route`, permute, the grouped FFN given by
// `ffn`, combine.  weights_present / weights_aligned: the caller's checks of
// its router and expert weights.  gather: `ffn` can read its rows of x
// through row_token (kGatherBf16 / kGatherFp8: with bf16 or FP8 weight
// tiles); where the tiles allow it, the permuted copy of x is then not
// written and `ffn` gets x and row_token (else x_perm and NULL).
enum GatherKind { kNoGather, kGatherBf16, kGatherFp8, kGatherFp8Packed };

template <class Route, class Ffn>
moe_status forward_impl(const moe_problem* p, const uint16_t* x, bool weights_present,
                        bool weights_aligned, uint16_t* y, float* logits, int32_t* topk_ids,
                        float* topk_weights, int32_t* expert_counts, int32_t* expert_offsets,
                        void* ws, size_t ws_bytes, void* stream, GatherKind can_gather,
                        Route route, Ffn ffn) {
  Dims d;
  moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!x || !y || !weights_present) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y) || !weights_aligned) return MOE_ERR_UNSUPPORTED;
  const ForwardWs L = forward_layout(d);
  if (d.N > 0 && (!ws || ws_bytes < L.total)) return MOE_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  (void)hipGetLastError();  // report only this call's launch errors
  char* base = static_cast<char*>(ws);
  if (!logits) logits = reinterpret_cast<float*>(base + L.logits);
  if (!topk_ids) topk_ids = reinterpret_cast<int32_t*>(base + L.ids);
  if (!topk_weights) topk_weights = reinterpret_cast<float*>(base + L.weights);
  if (!expert_counts) expert_counts = reinterpret_cast<int32_t*>(base + L.counts);
  if (!expert_offsets) expert_offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  int32_t* row_token = reinterpret_cast<int32_t*>(base + L.row_token);
  int32_t* slot_row = reinterpret_cast<int32_t*>(base + L.slot_row);
  uint16_t* x_perm = reinterpret_cast<uint16_t*>(base + L.x_perm);
  uint16_t* out_perm = reinterpret_cast<uint16_t*>(base + L.out_perm);
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = hip_status(route(d, logits, topk_ids, topk_weights, base, L, s));
  if (st != MOE_OK) return st;
  const bool gather = can_gather != kNoGather && !d.padded &&
                      (uint64_t)d.N * d.D * 2 < (1ull << 32) &&
                      gateup_gather_supported(d, can_gather >= kGatherFp8,
                                              can_gather == kGatherFp8Packed);
  st = hip_status(launch_permute(d, x, topk_ids, expert_counts, expert_offsets, row_token,
                                 slot_row, gather ? nullptr : x_perm, base + L.perm, s));
  if (st != MOE_OK) return st;
  st = hip_status(ffn(d, gather ? x : x_perm, gather ? row_token : nullptr, expert_offsets,
                      out_perm, base + L.ffn, s));
  if (st != MOE_OK) return st;
  return hip_status(launch_combine(d, out_perm, slot_row, topk_weights, y, s));
}

// The MLP router: features = bf16(GELU(x W_proj^T + b_proj)) as a one-group
// grouped GEMM, logits = features W_out^T by the router kernel, then top-K with
// b_out as the per-expert bias.
hipError_t launch_route_mlp(const Dims& d, const uint16_t* x, const uint16_t* w_proj,
                            const float* b_proj, const float* w_out, const float* b_out,
                            uint16_t* feats, int32_t* offsets2, float* logits, int32_t* ids,
                            float* weights, hipStream_t s) {
  hipError_t e = launch_dense_gelu(d.N, d.D, d.D / 4, x, w_proj, b_proj, feats, offsets2, s);
  if (e != hipSuccess) return e;
  Dims dr = d;
  dr.D = d.D / 4;
  e = launch_router_gemm(dr, feats, w_out, logits, nullptr, s);
  if (e != hipSuccess) return e;
  return launch_topk(d, logits, b_out, ids, weights, nullptr, s);
}

// Block-scaled FP8 weight stack: codes and scales present and 16-byte aligned.
inline moe_status check_fp8(const uint8_t* codes, const uint8_t* scales) {
  if (!codes || !scales) return MOE_ERR_INVALID_ARG;
  if (!aligned16(codes) || !aligned16(scales)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}
inline bool fp8_present(const uint8_t* c, const uint8_t* s) { return c && s; }
inline bool fp8_aligned(const uint8_t* c, const uint8_t* s) { return aligned16(c) && aligned16(s); }

// Device address of this device's copy of `scratch`, looked up once per
// device (with that device current) and kept.
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

moe_status static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !ptr) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol);
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return MOE_OK;
}

}  // namespace

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int v = g_cu_count[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    v = 256;
  g_cu_count[dev].store(v, std::memory_order_relaxed);
  return v;
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or alignment";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char* moe_last_hip_error(void) { return hipGetErrorString(t_last_hip_error); }

moe_status moe_permuted_rows(const moe_problem* p, int64_t* rows, int64_t* cap) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!rows) return MOE_ERR_INVALID_ARG;
  *rows = d.R;
  if (cap) *cap = d.cap;
  return MOE_OK;
}

moe_status moe_workspace_size(const moe_problem* p, size_t* bytes) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = forward_layout(d).total;
  return MOE_OK;
}

moe_status moe_route(const moe_problem* p, const uint16_t* x, const float* w_router,
                     const float* expert_bias, float* logits, int32_t* topk_ids,
                     float* topk_weights, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!logits || !topk_ids || !topk_weights || (x && !w_router)) return MOE_ERR_INVALID_ARG;
  if (x && (!aligned16(x) || !aligned16(w_router))) return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  (void)hipGetLastError();  // report only this call's launch errors
  hipStream_t s = static_cast<hipStream_t>(stream);
  // an optional workspace lets a small router run in its split form (the
  // same logits bit for bit); it is ignored when missing, small or unaligned
  const size_t need = router_ws_bytes(d);
  float* parts = (x && need > 0 && ws && aligned16(ws) && ws_bytes >= need)
                     ? static_cast<float*>(ws) : nullptr;
  if (x) {
    st = hip_status(launch_router_gemm(d, x, w_router, logits, parts, s));
    if (st != MOE_OK) return st;
  }
  return hip_status(launch_topk(d, logits, expert_bias, topk_ids, topk_weights, parts, s));
}

moe_status moe_permute(const moe_problem* p, const uint16_t* x, const int32_t* topk_ids,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* row_token,
                       int32_t* slot_row, uint16_t* x_perm, void* ws, size_t ws_bytes,
                       void* stream) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!x || !topk_ids || !expert_counts || !expert_offsets || !row_token || !slot_row)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || (x_perm && !aligned16(x_perm))) return MOE_ERR_UNSUPPORTED;
  const size_t need = permute_ws_bytes(d);
  if (d.N > 0 && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_permute(d, x, topk_ids, expert_counts, expert_offsets, row_token,
                                   slot_row, x_perm, ws, static_cast<hipStream_t>(stream)));
}

moe_status moe_grouped_ffn(const moe_problem* p, const uint16_t* x_perm,
                           const int32_t* expert_offsets, const uint16_t* w_gate,
                           const uint16_t* w_up, const uint16_t* w_down, uint16_t* out_perm,
                           uint16_t* h, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!x_perm || !expert_offsets || !w_gate || !w_up || !w_down || !out_perm)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_perm) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
      !aligned16(out_perm) || (h && !aligned16(h)))
    return MOE_ERR_UNSUPPORTED;
  const size_t need = h ? 0 : ffn_ws_bytes(d);
  if (d.N > 0 && need > 0 && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_grouped_ffn(d, x_perm, expert_offsets, w_gate, w_up, w_down, out_perm,
                                       h, ws, static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_gateup(const moe_problem* p, const uint16_t* x_perm,
                             const int32_t* expert_offsets, const uint16_t* w_gate,
                             const uint16_t* w_up, uint16_t* h, void* stream) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!x_perm || !expert_offsets || !w_gate || !w_up || !h) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_perm) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(h))
    return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_expert_gateup(d, x_perm, expert_offsets, w_gate, w_up, h,
                                         static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_gateup_gathered(const moe_problem* p, const uint16_t* x,
                                      const int32_t* row_token, const int32_t* expert_offsets,
                                      const uint16_t* w_gate, const uint16_t* w_up, uint16_t* h,
                                      void* stream) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!x || !row_token || !expert_offsets || !w_gate || !w_up || !h) return MOE_ERR_INVALID_ARG;
  if (d.padded || (uint64_t)d.N * d.D * 2 >= (1ull << 32)) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(h))
    return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  if (!gateup_gather_supported(d)) return MOE_ERR_UNSUPPORTED;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_expert_gateup_gathered(d, x, row_token, expert_offsets, w_gate, w_up,
                                                  h, static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_down(const moe_problem* p, const uint16_t* h,
                           const int32_t* expert_offsets, const uint16_t* w_down,
                           uint16_t* out_perm, void* stream) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!h || !expert_offsets || !w_down || !out_perm) return MOE_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(w_down) || !aligned16(out_perm)) return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_expert_down(d, h, expert_offsets, w_down, out_perm,
                                       static_cast<hipStream_t>(stream)));
}

moe_status moe_unpermute_combine(const moe_problem* p, const uint16_t* out_perm,
                                 const int32_t* slot_row, const float* topk_weights,
                                 uint16_t* y, void* stream) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!out_perm || !slot_row || !topk_weights || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(out_perm) || !aligned16(y)) return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_combine(d, out_perm, slot_row, topk_weights, y,
                                   static_cast<hipStream_t>(stream)));
}

moe_status moe_forward(const moe_problem* p, const uint16_t* x, const float* w_router,
                       const float* expert_bias, const uint16_t* w_gate, const uint16_t* w_up,
                       const uint16_t* w_down, uint16_t* y, float* logits, int32_t* topk_ids,
                       float* topk_weights, int32_t* expert_counts, int32_t* expert_offsets,
                       void* ws, size_t ws_bytes, void* stream) {
  const bool present = w_router && w_gate && w_up && w_down;
  const bool aligned = aligned16(w_router) && aligned16(w_gate) && aligned16(w_up) &&
                       aligned16(w_down);
  return forward_impl(p, x, present, aligned, y, logits, topk_ids, topk_weights, expert_counts,
                      expert_offsets, ws, ws_bytes, stream, kGatherBf16,
                      [&](const Dims& d, float* lg, int32_t* ids, float* w, char* base,
                          const ForwardWs& L, hipStream_t s) {
                        float* parts = router_ws_bytes(d) > 0
                                           ? reinterpret_cast<float*>(base + L.rpart)
                                           : nullptr;
                        const hipError_t e = launch_router_gemm(d, x, w_router, lg, parts, s);
                        return e != hipSuccess ? e
                                               : launch_topk(d, lg, expert_bias, ids, w, parts, s);
                      },
                      [&](const Dims& d, const uint16_t* xp, const int32_t* rt,
                          const int32_t* offs, uint16_t* op, void* fws, hipStream_t s) {
                        if (!rt)
                          return launch_grouped_ffn(d, xp, offs, w_gate, w_up, w_down, op,
                                                    nullptr, fws, s);
                        uint16_t* h = static_cast<uint16_t*>(fws);
                        const hipError_t e =
                            launch_expert_gateup_gathered(d, xp, rt, offs, w_gate, w_up, h, s);
                        return e != hipSuccess ? e
                                               : launch_expert_down(d, h, offs, w_down, op, s);
                      });
}

moe_status moe_forward_static(const moe_problem* p, const uint16_t* x, const float* w_router,
                              const float* expert_bias, const uint16_t* w_gate,
                              const uint16_t* w_up, const uint16_t* w_down, uint16_t* y,
                              float* logits, int32_t* topk_ids, float* topk_weights,
                              int32_t* expert_counts, int32_t* expert_offsets, void* stream) {
  // host-side checks first (forward_impl repeats them): problem, pointers and
  // the workspace size against the static scratch
  Dims d;
  moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!x || !y || !w_router || !w_gate || !w_up || !w_down) return MOE_ERR_INVALID_ARG;
  if (forward_layout(d).total > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  if (d.N == 0) return MOE_OK;
  void* ws = nullptr;
  if ((st = static_scratch(&ws)) != MOE_OK) return st;
  return moe_forward(p, x, w_router, expert_bias, w_gate, w_up, w_down, y, logits, topk_ids,
                     topk_weights, expert_counts, expert_offsets, ws, MOE_STATIC_SCRATCH_BYTES,
                     stream);
}

moe_status moe_routing_stats(int32_t num_experts, const int32_t* expert_counts, float* ema,
                             float* expert_bias, float decay, float step, void* stream) {
  if (num_experts < 1 || !expert_counts || !ema || !expert_bias) return MOE_ERR_INVALID_ARG;
  if (!(decay >= 0.f && decay <= 1.f) || !std::isfinite(step)) return MOE_ERR_INVALID_ARG;
  if (num_experts > 1024) return MOE_ERR_UNSUPPORTED;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_routing_stats(num_experts, expert_counts, ema, expert_bias, decay, step,
                                         static_cast<hipStream_t>(stream)));
}

moe_status moe_quantize_fp8(int64_t rows, int32_t cols, const uint16_t* w, uint8_t* codes,
                            uint8_t* scales, void* stream) {
  if (rows < 0 || cols <= 0 || !w || !codes || !scales) return MOE_ERR_INVALID_ARG;
  if (rows % 32 != 0 || cols % 32 != 0 || !aligned16(w) || !aligned16(codes))
    return MOE_ERR_UNSUPPORTED;
  if (rows > (int64_t)1 << 40 || (int64_t)cols > ((int64_t)1 << 40) / (rows > 0 ? rows : 1))
    return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(
      launch_quantize_fp8(rows, cols, w, codes, scales, static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_gateup_fp8(const moe_problem* p, const uint16_t* x_perm,
                                 const int32_t* expert_offsets, const uint8_t* w_gate_codes,
                                 const uint8_t* w_gate_scales, const uint8_t* w_up_codes,
                                 const uint8_t* w_up_scales, uint16_t* h, void* stream) {
  Dims d;
  moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!x_perm || !expert_offsets || !h) return MOE_ERR_INVALID_ARG;
  if ((st = check_fp8(w_gate_codes, w_gate_scales)) != MOE_OK) return st;
  if ((st = check_fp8(w_up_codes, w_up_scales)) != MOE_OK) return st;
  if (!aligned16(x_perm) || !aligned16(h)) return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_expert_gateup_fp8(d, x_perm, expert_offsets,
                                             Fp8Weight{w_gate_codes, w_gate_scales},
                                             Fp8Weight{w_up_codes, w_up_scales}, h,
                                             static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_gateup_fp8_gathered(const moe_problem* p, const uint16_t* x,
                                          const int32_t* row_token,
                                          const int32_t* expert_offsets,
                                          const uint8_t* w_gate_codes,
                                          const uint8_t* w_gate_scales,
                                          const uint8_t* w_up_codes, const uint8_t* w_up_scales,
                                          uint16_t* h, void* stream) {
  Dims d;
  moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!x || !row_token || !expert_offsets || !h) return MOE_ERR_INVALID_ARG;
  if ((st = check_fp8(w_gate_codes, w_gate_scales)) != MOE_OK) return st;
  if ((st = check_fp8(w_up_codes, w_up_scales)) != MOE_OK) return st;
  if (d.padded || (uint64_t)d.N * d.D * 2 >= (1ull << 32)) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(h)) return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  if (!gateup_gather_supported(d, true)) return MOE_ERR_UNSUPPORTED;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_expert_gateup_fp8_gathered(
      d, x, row_token, expert_offsets, Fp8Weight{w_gate_codes, w_gate_scales},
      Fp8Weight{w_up_codes, w_up_scales}, h, static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_down_fp8(const moe_problem* p, const uint16_t* h,
                               const int32_t* expert_offsets, const uint8_t* w_down_codes,
                               const uint8_t* w_down_scales, uint16_t* out_perm, void* stream) {
  Dims d;
  moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!h || !expert_offsets || !out_perm) return MOE_ERR_INVALID_ARG;
  if ((st = check_fp8(w_down_codes, w_down_scales)) != MOE_OK) return st;
  if (!aligned16(h) || !aligned16(out_perm)) return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_expert_down_fp8(d, h, expert_offsets,
                                           Fp8Weight{w_down_codes, w_down_scales}, out_perm,
                                           static_cast<hipStream_t>(stream)));
}

moe_status moe_grouped_ffn_fp8(const moe_problem* p, const uint16_t* x_perm,
                               const int32_t* expert_offsets, const uint8_t* w_gate_codes,
                               const uint8_t* w_gate_scales, const uint8_t* w_up_codes,
                               const uint8_t* w_up_scales, const uint8_t* w_down_codes,
                               const uint8_t* w_down_scales, uint16_t* out_perm, uint16_t* h,
                               void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!x_perm || !expert_offsets || !out_perm) return MOE_ERR_INVALID_ARG;
  if ((st = check_fp8(w_gate_codes, w_gate_scales)) != MOE_OK) return st;
  if ((st = check_fp8(w_up_codes, w_up_scales)) != MOE_OK) return st;
  if ((st = check_fp8(w_down_codes, w_down_scales)) != MOE_OK) return st;
  if (!aligned16(x_perm) || !aligned16(out_perm) || (h && !aligned16(h)))
    return MOE_ERR_UNSUPPORTED;
  const size_t need = h ? 0 : ffn_ws_bytes(d);
  if (d.N > 0 && need > 0 && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_grouped_ffn_fp8(
      d, x_perm, expert_offsets, Fp8Weight{w_gate_codes, w_gate_scales},
      Fp8Weight{w_up_codes, w_up_scales}, Fp8Weight{w_down_codes, w_down_scales}, out_perm, h, ws,
      static_cast<hipStream_t>(stream)));
}

moe_status moe_forward_fp8(const moe_problem* p, const uint16_t* x, const float* w_router,
                           const float* expert_bias, const uint8_t* w_gate_codes,
                           const uint8_t* w_gate_scales, const uint8_t* w_up_codes,
                           const uint8_t* w_up_scales, const uint8_t* w_down_codes,
                           const uint8_t* w_down_scales, uint16_t* y, float* logits,
                           int32_t* topk_ids, float* topk_weights, int32_t* expert_counts,
                           int32_t* expert_offsets, void* ws, size_t ws_bytes, void* stream) {
  const bool present = w_router && fp8_present(w_gate_codes, w_gate_scales) &&
                       fp8_present(w_up_codes, w_up_scales) &&
                       fp8_present(w_down_codes, w_down_scales);
  const bool aligned = aligned16(w_router) && fp8_aligned(w_gate_codes, w_gate_scales) &&
                       fp8_aligned(w_up_codes, w_up_scales) &&
                       fp8_aligned(w_down_codes, w_down_scales);
  const Fp8Weight wg{w_gate_codes, w_gate_scales}, wu{w_up_codes, w_up_scales},
      wd{w_down_codes, w_down_scales};
  return forward_impl(p, x, present, aligned, y, logits, topk_ids, topk_weights, expert_counts,
                      expert_offsets, ws, ws_bytes, stream, kGatherFp8,
                      [&](const Dims& d, float* lg, int32_t* ids, float* w, char* base,
                          const ForwardWs& L, hipStream_t s) {
                        float* parts = router_ws_bytes(d) > 0
                                           ? reinterpret_cast<float*>(base + L.rpart)
                                           : nullptr;
                        const hipError_t e = launch_router_gemm(d, x, w_router, lg, parts, s);
                        return e != hipSuccess ? e
                                               : launch_topk(d, lg, expert_bias, ids, w, parts, s);
                      },
                      [&](const Dims& d, const uint16_t* xp, const int32_t* rt,
                          const int32_t* offs, uint16_t* op, void* fws, hipStream_t s) {
                        if (rt) {
                          uint16_t* h = static_cast<uint16_t*>(fws);
                          const hipError_t e =
                              launch_expert_gateup_fp8_gathered(d, xp, rt, offs, wg, wu, h, s);
                          return e != hipSuccess ? e
                                                 : launch_expert_down_fp8(d, h, offs, wd, op, s);
                        }
                        return launch_grouped_ffn_fp8(d, xp, offs, wg, wu, wd, op, nullptr, fws,
                                                      s);
                      });
}

// The contraction length of an FP8 stack packed by 128-code stages must be a
// multiple of 128: D for gate/up, F for down.
inline bool fp8_pack_fits(const Dims& d, bool gateup) {
  return (gateup ? d.D : d.F) % 128 == 0;
}

moe_status moe_packed_weight_size(const moe_problem* p, int32_t kind, size_t* bytes) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!bytes || kind < MOE_PACK_GATEUP || kind > MOE_PACK_DOWN_FP8) return MOE_ERR_INVALID_ARG;
  const bool gateup = kind == MOE_PACK_GATEUP || kind == MOE_PACK_GATEUP_FP8;
  const bool fp8 = kind == MOE_PACK_GATEUP_FP8 || kind == MOE_PACK_DOWN_FP8;
  if (fp8 && !fp8_pack_fits(d, gateup)) return MOE_ERR_UNSUPPORTED;
  *bytes = packed_weight_bytes(d, gateup, fp8);
  return MOE_OK;
}

moe_status moe_pack_weights_fp8(const moe_problem* p, int32_t kind, const uint8_t* c0,
                                const uint8_t* c1, uint8_t* packed, void* stream) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  const bool gateup = kind == MOE_PACK_GATEUP_FP8;
  if ((!gateup && kind != MOE_PACK_DOWN_FP8) || !c0 || (gateup && !c1) || !packed)
    return MOE_ERR_INVALID_ARG;
  if (!fp8_pack_fits(d, gateup)) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(c0) || (gateup && !aligned16(c1)) || !aligned16(packed))
    return MOE_ERR_UNSUPPORTED;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_pack_weights(d, gateup, reinterpret_cast<const uint16_t*>(c0),
                                        reinterpret_cast<const uint16_t*>(gateup ? c1 : c0),
                                        reinterpret_cast<uint16_t*>(packed),
                                        static_cast<hipStream_t>(stream), true));
}

moe_status moe_expert_gateup_fp8_packed(const moe_problem* p, const uint16_t* x_perm,
                                        const int32_t* expert_offsets,
                                        const uint8_t* w_gateup_packed,
                                        const uint8_t* w_gate_scales, const uint8_t* w_up_scales,
                                        uint16_t* h, void* stream) {
  Dims d;
  moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!x_perm || !expert_offsets || !h) return MOE_ERR_INVALID_ARG;
  if ((st = check_fp8(w_gateup_packed, w_gate_scales)) != MOE_OK) return st;
  if ((st = check_fp8(w_gateup_packed, w_up_scales)) != MOE_OK) return st;
  if (!fp8_pack_fits(d, true) || !aligned16(x_perm) || !aligned16(h)) return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_expert_gateup_fp8(d, x_perm, expert_offsets,
                                             Fp8Weight{w_gateup_packed, w_gate_scales},
                                             Fp8Weight{nullptr, w_up_scales}, h,
                                             static_cast<hipStream_t>(stream), true));
}

moe_status moe_expert_gateup_fp8_packed_gathered(const moe_problem* p, const uint16_t* x,
                                                 const int32_t* row_token,
                                                 const int32_t* expert_offsets,
                                                 const uint8_t* w_gateup_packed,
                                                 const uint8_t* w_gate_scales,
                                                 const uint8_t* w_up_scales, uint16_t* h,
                                                 void* stream) {
  Dims d;
  moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!x || !row_token || !expert_offsets || !h) return MOE_ERR_INVALID_ARG;
  if ((st = check_fp8(w_gateup_packed, w_gate_scales)) != MOE_OK) return st;
  if ((st = check_fp8(w_gateup_packed, w_up_scales)) != MOE_OK) return st;
  if (!fp8_pack_fits(d, true)) return MOE_ERR_UNSUPPORTED;
  if (d.padded || (uint64_t)d.N * d.D * 2 >= (1ull << 32)) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(h)) return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  if (!gateup_gather_supported(d, true, true)) return MOE_ERR_UNSUPPORTED;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_expert_gateup_fp8_gathered(
      d, x, row_token, expert_offsets, Fp8Weight{w_gateup_packed, w_gate_scales},
      Fp8Weight{nullptr, w_up_scales}, h, static_cast<hipStream_t>(stream), true));
}

moe_status moe_expert_down_fp8_packed(const moe_problem* p, const uint16_t* h,
                                      const int32_t* expert_offsets,
                                      const uint8_t* w_down_packed,
                                      const uint8_t* w_down_scales, uint16_t* out_perm,
                                      void* stream) {
  Dims d;
  moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!h || !expert_offsets || !out_perm) return MOE_ERR_INVALID_ARG;
  if ((st = check_fp8(w_down_packed, w_down_scales)) != MOE_OK) return st;
  if (!fp8_pack_fits(d, false) || !aligned16(h) || !aligned16(out_perm))
    return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_expert_down_fp8(d, h, expert_offsets,
                                           Fp8Weight{w_down_packed, w_down_scales}, out_perm,
                                           static_cast<hipStream_t>(stream), true));
}

moe_status moe_forward_fp8_packed(const moe_problem* p, const uint16_t* x, const float* w_router,
                                  const float* expert_bias, const uint8_t* w_gateup_packed,
                                  const uint8_t* w_gate_scales, const uint8_t* w_up_scales,
                                  const uint8_t* w_down_packed, const uint8_t* w_down_scales,
                                  uint16_t* y, float* logits, int32_t* topk_ids,
                                  float* topk_weights, int32_t* expert_counts,
                                  int32_t* expert_offsets, void* ws, size_t ws_bytes,
                                  void* stream) {
  const bool present = w_router && fp8_present(w_gateup_packed, w_gate_scales) &&
                       fp8_present(w_gateup_packed, w_up_scales) &&
                       fp8_present(w_down_packed, w_down_scales);
  const bool aligned = aligned16(w_router) && fp8_aligned(w_gateup_packed, w_gate_scales) &&
                       fp8_aligned(w_gateup_packed, w_up_scales) &&
                       fp8_aligned(w_down_packed, w_down_scales);
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (present && x && y && (!fp8_pack_fits(d, true) || !fp8_pack_fits(d, false)))
    return MOE_ERR_UNSUPPORTED;
  const Fp8Weight wg{w_gateup_packed, w_gate_scales}, wu{nullptr, w_up_scales},
      wd{w_down_packed, w_down_scales};
  return forward_impl(p, x, present, aligned, y, logits, topk_ids, topk_weights, expert_counts,
                      expert_offsets, ws, ws_bytes, stream, kGatherFp8Packed,
                      [&](const Dims& dd, float* lg, int32_t* ids, float* w, char* base,
                          const ForwardWs& L, hipStream_t s) {
                        float* parts = router_ws_bytes(dd) > 0
                                           ? reinterpret_cast<float*>(base + L.rpart)
                                           : nullptr;
                        const hipError_t e = launch_router_gemm(dd, x, w_router, lg, parts, s);
                        return e != hipSuccess ? e
                                               : launch_topk(dd, lg, expert_bias, ids, w, parts, s);
                      },
                      [&](const Dims& dd, const uint16_t* xp, const int32_t* rt,
                          const int32_t* offs, uint16_t* op, void* fws, hipStream_t s) {
                        if (rt) {
                          uint16_t* h = static_cast<uint16_t*>(fws);
                          const hipError_t e = launch_expert_gateup_fp8_gathered(
                              dd, xp, rt, offs, wg, wu, h, s, true);
                          return e != hipSuccess
                                     ? e
                                     : launch_expert_down_fp8(dd, h, offs, wd, op, s, true);
                        }
                        return launch_grouped_ffn_fp8(dd, xp, offs, wg, wu, wd, op, nullptr, fws,
                                                      s, true);
                      });
}

moe_status moe_pack_weights(const moe_problem* p, int32_t kind, const uint16_t* w0,
                            const uint16_t* w1, uint16_t* packed, void* stream) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  const bool gateup = kind == MOE_PACK_GATEUP;
  if ((!gateup && kind != MOE_PACK_DOWN) || !w0 || (gateup && !w1) || !packed)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(w0) || (gateup && !aligned16(w1)) || !aligned16(packed))
    return MOE_ERR_UNSUPPORTED;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_pack_weights(d, gateup, w0, gateup ? w1 : w0, packed,
                                        static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_gateup_packed(const moe_problem* p, const uint16_t* x_perm,
                                    const int32_t* expert_offsets,
                                    const uint16_t* w_gateup_packed, uint16_t* h, void* stream) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!x_perm || !expert_offsets || !w_gateup_packed || !h) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_perm) || !aligned16(w_gateup_packed) || !aligned16(h))
    return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_expert_gateup(d, x_perm, expert_offsets, w_gateup_packed, nullptr, h,
                                         static_cast<hipStream_t>(stream), true));
}

moe_status moe_expert_gateup_packed_gathered(const moe_problem* p, const uint16_t* x,
                                             const int32_t* row_token,
                                             const int32_t* expert_offsets,
                                             const uint16_t* w_gateup_packed, uint16_t* h,
                                             void* stream) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!x || !row_token || !expert_offsets || !w_gateup_packed || !h) return MOE_ERR_INVALID_ARG;
  if (d.padded || (uint64_t)d.N * d.D * 2 >= (1ull << 32)) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(w_gateup_packed) || !aligned16(h)) return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  if (!gateup_gather_supported(d)) return MOE_ERR_UNSUPPORTED;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_expert_gateup_gathered(d, x, row_token, expert_offsets,
                                                  w_gateup_packed, nullptr, h,
                                                  static_cast<hipStream_t>(stream), true));
}

moe_status moe_expert_down_packed(const moe_problem* p, const uint16_t* h,
                                  const int32_t* expert_offsets, const uint16_t* w_down_packed,
                                  uint16_t* out_perm, void* stream) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!h || !expert_offsets || !w_down_packed || !out_perm) return MOE_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(w_down_packed) || !aligned16(out_perm))
    return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_expert_down(d, h, expert_offsets, w_down_packed, out_perm,
                                       static_cast<hipStream_t>(stream), true));
}

moe_status moe_forward_packed(const moe_problem* p, const uint16_t* x, const float* w_router,
                              const float* expert_bias, const uint16_t* w_gateup_packed,
                              const uint16_t* w_down_packed, uint16_t* y, float* logits,
                              int32_t* topk_ids, float* topk_weights, int32_t* expert_counts,
                              int32_t* expert_offsets, void* ws, size_t ws_bytes, void* stream) {
  const bool present = w_router && w_gateup_packed && w_down_packed;
  const bool aligned =
      aligned16(w_router) && aligned16(w_gateup_packed) && aligned16(w_down_packed);
  return forward_impl(p, x, present, aligned, y, logits, topk_ids, topk_weights, expert_counts,
                      expert_offsets, ws, ws_bytes, stream, kGatherBf16,
                      [&](const Dims& d, float* lg, int32_t* ids, float* w, char* base,
                          const ForwardWs& L, hipStream_t s) {
                        float* parts = router_ws_bytes(d) > 0
                                           ? reinterpret_cast<float*>(base + L.rpart)
                                           : nullptr;
                        const hipError_t e = launch_router_gemm(d, x, w_router, lg, parts, s);
                        return e != hipSuccess ? e
                                               : launch_topk(d, lg, expert_bias, ids, w, parts, s);
                      },
                      [&](const Dims& d, const uint16_t* xp, const int32_t* rt,
                          const int32_t* offs, uint16_t* op, void* fws, hipStream_t s) {
                        if (!rt)
                          return launch_grouped_ffn(d, xp, offs, w_gateup_packed, nullptr,
                                                    w_down_packed, op, nullptr, fws, s, true);
                        uint16_t* h = static_cast<uint16_t*>(fws);
                        const hipError_t e = launch_expert_gateup_gathered(
                            d, xp, rt, offs, w_gateup_packed, nullptr, h, s, true);
                        return e != hipSuccess
                                   ? e
                                   : launch_expert_down(d, h, offs, w_down_packed, op, s, true);
                      });
}

moe_status moe_route_mlp(const moe_problem* p, const uint16_t* x, const uint16_t* w_proj,
                         const float* b_proj, const float* w_out, const float* b_out,
                         uint16_t* features, float* logits, int32_t* topk_ids,
                         float* topk_weights, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!x || !w_proj || !b_proj || !w_out || !logits || !topk_ids || !topk_weights)
    return MOE_ERR_INVALID_ARG;
  if (d.D % 256 != 0) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(w_proj) || !aligned16(b_proj) || !aligned16(w_out) ||
      (features && !aligned16(features)))
    return MOE_ERR_UNSUPPORTED;
  const ForwardWs L = forward_layout(d);
  if (d.N > 0 && (!ws || ws_bytes < L.total)) return MOE_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  (void)hipGetLastError();  // report only this call's launch errors
  char* base = static_cast<char*>(ws);
  if (!features) features = reinterpret_cast<uint16_t*>(base + L.feats);
  return hip_status(launch_route_mlp(d, x, w_proj, b_proj, w_out, b_out, features,
                                     reinterpret_cast<int32_t*>(base + L.roff), logits, topk_ids,
                                     topk_weights, static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_up_gelu(const moe_problem* p, const uint16_t* x_perm,
                              const int32_t* expert_offsets, const uint16_t* w1, const float* b1,
                              uint16_t* h, void* stream) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!x_perm || !expert_offsets || !w1 || !b1 || !h) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_perm) || !aligned16(w1) || !aligned16(b1) || !aligned16(h))
    return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_expert_up_gelu(d, x_perm, expert_offsets, w1, b1, h,
                                          static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_up_gelu_gathered(const moe_problem* p, const uint16_t* x,
                                       const int32_t* row_token, const int32_t* expert_offsets,
                                       const uint16_t* w1, const float* b1, uint16_t* h,
                                       void* stream) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!x || !row_token || !expert_offsets || !w1 || !b1 || !h) return MOE_ERR_INVALID_ARG;
  if (d.padded || (uint64_t)d.N * d.D * 2 >= (1ull << 32)) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(w1) || !aligned16(b1) || !aligned16(h))
    return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  if (!gateup_gather_supported(d)) return MOE_ERR_UNSUPPORTED;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_expert_up_gelu_gathered(d, x, row_token, expert_offsets, w1, b1, h,
                                                   static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_down_bias(const moe_problem* p, const uint16_t* h,
                                const int32_t* expert_offsets, const uint16_t* w2,
                                const float* b2, uint16_t* out_perm, void* stream) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!h || !expert_offsets || !w2 || !b2 || !out_perm) return MOE_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(w2) || !aligned16(b2) || !aligned16(out_perm))
    return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_expert_down_bias(d, h, expert_offsets, w2, b2, out_perm,
                                            static_cast<hipStream_t>(stream)));
}

moe_status moe_grouped_ffn_gelu(const moe_problem* p, const uint16_t* x_perm,
                                const int32_t* expert_offsets, const uint16_t* w1,
                                const float* b1, const uint16_t* w2, const float* b2,
                                uint16_t* out_perm, uint16_t* h, void* ws, size_t ws_bytes,
                                void* stream) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!x_perm || !expert_offsets || !w1 || !b1 || !w2 || !b2 || !out_perm)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_perm) || !aligned16(w1) || !aligned16(b1) || !aligned16(w2) ||
      !aligned16(b2) || !aligned16(out_perm) || (h && !aligned16(h)))
    return MOE_ERR_UNSUPPORTED;
  const size_t need = h ? 0 : ffn_ws_bytes(d);
  if (d.N > 0 && need > 0 && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_grouped_ffn_gelu(d, x_perm, expert_offsets, w1, b1, w2, b2, out_perm,
                                            h, ws, static_cast<hipStream_t>(stream)));
}

moe_status moe_forward_gelu(const moe_problem* p, const uint16_t* x, const uint16_t* w_proj,
                            const float* b_proj, const float* w_out, const float* b_out,
                            const uint16_t* w1, const float* b1, const uint16_t* w2,
                            const float* b2, uint16_t* y, float* logits, int32_t* topk_ids,
                            float* topk_weights, int32_t* expert_counts,
                            int32_t* expert_offsets, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  const bool present = w_proj && b_proj && w_out && w1 && b1 && w2 && b2;
  const bool aligned = aligned16(w_proj) && aligned16(b_proj) && aligned16(w_out) &&
                       aligned16(w1) && aligned16(b1) && aligned16(w2) && aligned16(b2);
  if (present && aligned && x && y && d.D % 256 != 0) return MOE_ERR_UNSUPPORTED;
  return forward_impl(p, x, present, aligned, y, logits, topk_ids, topk_weights, expert_counts,
                      expert_offsets, ws, ws_bytes, stream, kGatherBf16,
                      [&](const Dims& dd, float* lg, int32_t* ids, float* w, char* base,
                          const ForwardWs& L, hipStream_t s) {
                        return launch_route_mlp(dd, x, w_proj, b_proj, w_out, b_out,
                                                reinterpret_cast<uint16_t*>(base + L.feats),
                                                reinterpret_cast<int32_t*>(base + L.roff), lg,
                                                ids, w, s);
                      },
                      [&](const Dims& dd, const uint16_t* xp, const int32_t* rt,
                          const int32_t* offs, uint16_t* op, void* fws, hipStream_t s) {
                        if (rt) {
                          uint16_t* h = static_cast<uint16_t*>(fws);
                          const hipError_t e =
                              launch_expert_up_gelu_gathered(dd, xp, rt, offs, w1, b1, h, s);
                          return e != hipSuccess
                                     ? e
                                     : launch_expert_down_bias(dd, h, offs, w2, b2, op, s);
                        }
                        return launch_grouped_ffn_gelu(dd, xp, offs, w1, b1, w2, b2, op, nullptr,
                                                       fws, s);
                      });
}

moe_status moe_fused_error_offset(const moe_problem* p, int32_t whole_layer, size_t* offset) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!offset) return MOE_ERR_INVALID_ARG;
  *offset = (whole_layer ? forward_layout(d).fused : 0) + fused_err_offset(d);
  return MOE_OK;
}

moe_status moe_fused_ffn(const moe_problem* p, const uint16_t* x, const int32_t* row_token,
                         const int32_t* expert_offsets, const uint16_t* w_gate,
                         const uint16_t* w_up, const uint16_t* w_down, uint16_t* out_perm,
                         void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  const moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!x || !row_token || !expert_offsets || !w_gate || !w_up || !w_down || !out_perm)
    return MOE_ERR_INVALID_ARG;
  if (d.padded || (uint64_t)d.N * d.D * 2 >= (1ull << 32)) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
      !aligned16(out_perm))
    return MOE_ERR_UNSUPPORTED;
  if (d.N > 0 && (!ws || ws_bytes < fused_ws_bytes(d))) return MOE_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  (void)hipGetLastError();  // report only this call's launch errors
  return hip_status(launch_fused_ffn(d, x, row_token, expert_offsets, w_gate, w_up, w_down,
                                     out_perm, ws, static_cast<hipStream_t>(stream)));
}

moe_status moe_forward_fused(const moe_problem* p, const uint16_t* x, const float* w_router,
                             const float* expert_bias, const uint16_t* w_gate,
                             const uint16_t* w_up, const uint16_t* w_down, uint16_t* y,
                             float* logits, int32_t* topk_ids, float* topk_weights,
                             int32_t* expert_counts, int32_t* expert_offsets, void* ws,
                             size_t ws_bytes, void* stream) {
  Dims d;
  moe_status st = check_problem(p, &d);
  if (st != MOE_OK) return st;
  if (!x || !y || !w_router || !w_gate || !w_up || !w_down) return MOE_ERR_INVALID_ARG;
  if (d.padded || (uint64_t)d.N * d.D * 2 >= (1ull << 32)) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(y) || !aligned16(w_router) || !aligned16(w_gate) ||
      !aligned16(w_up) || !aligned16(w_down))
    return MOE_ERR_UNSUPPORTED;
  const ForwardWs L = forward_layout(d);
  if (d.N > 0 && (!ws || ws_bytes < L.total)) return MOE_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return MOE_ERR_UNSUPPORTED;
  if (d.N == 0) return MOE_OK;
  (void)hipGetLastError();  // report only this call's launch errors
  char* base = static_cast<char*>(ws);
  if (!logits) logits = reinterpret_cast<float*>(base + L.logits);
  if (!topk_ids) topk_ids = reinterpret_cast<int32_t*>(base + L.ids);
  if (!topk_weights) topk_weights = reinterpret_cast<float*>(base + L.weights);
  if (!expert_counts) expert_counts = reinterpret_cast<int32_t*>(base + L.counts);
  if (!expert_offsets) expert_offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  int32_t* row_token = reinterpret_cast<int32_t*>(base + L.row_token);
  int32_t* slot_row = reinterpret_cast<int32_t*>(base + L.slot_row);
  uint16_t* out_perm = reinterpret_cast<uint16_t*>(base + L.out_perm);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* parts = router_ws_bytes(d) > 0 ? reinterpret_cast<float*>(base + L.rpart) : nullptr;
  st = hip_status(launch_router_gemm(d, x, w_router, logits, parts, s));
  if (st != MOE_OK) return st;
  st = hip_status(launch_topk(d, logits, expert_bias, topk_ids, topk_weights, parts, s));
  if (st != MOE_OK) return st;
  st = hip_status(launch_permute(d, x, topk_ids, expert_counts, expert_offsets, row_token,
                                 slot_row, nullptr, base + L.perm, s));
  if (st != MOE_OK) return st;
  st = hip_status(launch_fused_ffn(d, x, row_token, expert_offsets, w_gate, w_up, w_down,
                                   out_perm, base + L.fused, s));
  if (st != MOE_OK) return st;
  return hip_status(launch_combine(d, out_perm, slot_row, topk_weights, y, s));
}

}  // extern "C"
