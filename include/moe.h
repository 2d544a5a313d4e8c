/*
 * libmoe -- forward pass of one Mixture-of-Experts layer on one AMD Instinct
 * MI355X (gfx950) GPU, as a C ABI over hand-written HIP kernels.
 *
 * The layer (from "MoE 推理完整机制：从 Router 到 Expert Parallelism 的一切",
 * zoe.im, opening dataflow and sections 第一层 / 第二层):
 *   N x D tokens -> router logits (N x E) -> top-K experts per token and
 *   their weights -> tokens regrouped into one expert-contiguous buffer with
 *   expert_offsets -> per-expert FFN (two GEMMs) -> rows put back in token
 *   order, scaled by the router weights and summed -> N x D output.
 *
 * Conventions for every call below
 *   - Pointers are DEVICE pointers unless marked "host".  bf16 tensors are
 *     passed as raw bit patterns (uint16_t).  All tensors are dense and
 *     row-major; weights use the nn.Linear [out, in] layout.
 *   - The caller owns every buffer.  No call allocates or frees device
 *     memory; scratch comes from the caller's workspace `ws` of `ws_bytes`
 *     bytes (size from moe_workspace_size; 256-byte alignment).
 *   - Every call enqueues work on `stream` (a hipStream_t, NULL = default
 *     stream) and returns without waiting; results are ready when the
 *     stream reaches that point.  No call reads device memory on the host.
 *   - Arguments are checked on the host before any HIP call:
 *     MOE_ERR_INVALID_ARG for a null required pointer or an inconsistent
 *     problem, MOE_ERR_UNSUPPORTED for shapes or alignments the kernels do
 *     not handle, MOE_ERR_WORKSPACE for a missing or too small workspace.
 *     A failed launch returns MOE_ERR_HIP.  Nothing aborts, throws or prints.
 *   - num_tokens == 0 is valid: the call returns MOE_OK and launches nothing.
 *   - Calls are re-entrant (no mutable global state besides a per-device
 *     cache of the compute-unit count and a thread-local last HIP error);
 *     concurrent calls on different streams must use different workspaces
 *     and outputs.
 *   - Results are deterministic: routing, counts, offsets and the
 *     permutation are exact integer results; floating-point outputs do not
 *     depend on scheduling (no floating-point atomics).
 */
#ifndef LIBMOE_MOE_H_
#define LIBMOE_MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_HIP = 4
} moe_status;

/* Gating functions, zoe.im section 第一层 (Router 与 Top-K):
 *  SOFTMAX_TOPK   : top-K of the keys, then softmax over the K selected keys.
 *  SIGMOID_RENORM : top-K, weights sigmoid(key) divided by their sum over the
 *                   K selected (the "DeepSeek sigmoid + norm" variant).
 * The key of expert e is logit[e] + bias[e] (one fp32 add; bias optional), as
 * in the dynamic-bias router of "MoE 大规模分布式推理工程实战" (ybb.press)
 * section 4.1.  Selection: largest key first, equal keys by lower expert id,
 * -0.0 == +0.0, NaN keys rank below every number.  In sigmoid mode selection
 * is made on the key itself (sigmoid is increasing), so no rounding of
 * sigmoid can change the chosen set. */
typedef enum { MOE_GATING_SOFTMAX_TOPK = 0, MOE_GATING_SIGMOID_RENORM = 1 } moe_gating;

typedef struct {
  int64_t num_tokens;   /* N >= 0                                               */
  int32_t hidden;       /* D: multiple of 64, >= 64                             */
  int32_t ffn;          /* F: expert FFN width, multiple of 64, >= 64            */
  int32_t num_experts;  /* E: 1 <= E <= 1024                                     */
  int32_t top_k;        /* K: 1 <= K <= min(E, 64)                               */
  int32_t gating;       /* moe_gating                                            */
  /* Capacity factor num/den.  num == 0: contiguous layout (范式 A), no token
   * is dropped, R = N*K rows.  num > 0: capacity-padded layout (范式 B),
   * cap = ceil(num*N*K / (den*E)), expert e owns rows [e*cap, (e+1)*cap),
   * the first cap slots of each expert in slot order are kept and the rest
   * dropped, R = E*cap rows.  (zoe.im 范式 B; capacity = tokens*k/E*factor in
   * "MoE工程实战" (jsqmd.com) 3.2.) */
  int32_t capacity_num;
  int32_t capacity_den;
} moe_problem;

/* ---------------------------------------------------------------- host only */

int moe_abi_version(void);
const char* moe_status_str(moe_status s);

/* Text of the HIP error behind this thread's last MOE_ERR_HIP ("no error"
 * before any).  Thread-local; the string is static. */
const char* moe_last_hip_error(void);

/* Rows R of the permuted buffers (x_perm, out_perm, row_token): N*K in the
 * contiguous layout, E*cap in the padded one.  `rows` and `cap` are host
 * pointers; `cap` may be NULL (it receives 0 in the contiguous layout). */
moe_status moe_permuted_rows(const moe_problem* p, int64_t* rows, int64_t* cap);

/* Workspace bytes (host pointer `bytes`) that moe_forward needs for this
 * problem.  Every staged call below needs at most this much. */
moe_status moe_workspace_size(const moe_problem* p, size_t* bytes);

/* ---------------------------------------------------------------- the path */

/* Router GEMM and top-K gating (zoe.im 第一层; ybb.press 4.1).
 *   x            [N, D] bf16, or NULL: then `logits` is an INPUT and the
 *                router GEMM is skipped (selection on given fp32 logits).
 *   w_router     [E, D] fp32 (the gate Linear, no bias); ignored if x NULL.
 *   expert_bias  [E] fp32 or NULL (added to the logits before selection and
 *                used for the weights).
 *   logits       [N, E] fp32: written when x != NULL (pre-bias), read else.
 *   topk_ids     [N, K] int32, out: selected experts, largest key first.
 *   topk_weights [N, K] fp32, out: router weights, sum to 1 per row.
 * Workspace optional (ws may be NULL): given moe_workspace_size bytes,
 * 16-byte aligned, a small problem (few token x expert tiles, e.g. a decode
 * step) runs its router GEMM spread over more compute units.  The logits,
 * and so every output, are bit for bit the same with or without it. */
moe_status moe_route(const moe_problem* p, const uint16_t* x, const float* w_router,
                     const float* expert_bias, float* logits, int32_t* topk_ids,
                     float* topk_weights, void* ws, size_t ws_bytes, void* stream);

/* Permutation into expert segments (zoe.im 范式 A Step 1 / 范式 B).
 * Slot i = n*K + k.  Histogram + exclusive prefix sum give the offsets; each
 * slot takes the next row of its expert's segment in ascending slot order, so
 * a segment lists its tokens in token order.
 *   x              [N, D] bf16 input rows.
 *   topk_ids       [N, K] int32; a value outside [0, E) marks its slot as
 *                  dropped (slot_row -1, not counted).
 *   expert_counts  [E] int32 out: slots routed to each expert (before drops).
 *   expert_offsets [E+1] int32 out: segment starts; contiguous: prefix sums
 *                  of the counts, offsets[E] = N*K; padded: e*cap.
 *   row_token      [R] int32 out: token of each row, -1 for padding rows.
 *   slot_row       [N*K] int32 out: row of each slot, -1 if dropped.
 *   x_perm         [R, D] bf16 out: x_perm[r] = x[row_token[r]], padding
 *                  rows zero; or NULL: only the routing tables are written
 *                  (for moe_fused_ffn, which gathers from x itself).
 * Workspace: moe_workspace_size bytes suffice. */
moe_status moe_permute(const moe_problem* p, const uint16_t* x, const int32_t* topk_ids,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* row_token,
                       int32_t* slot_row, uint16_t* x_perm, void* ws, size_t ws_bytes,
                       void* stream);

/* Grouped SwiGLU expert FFN over the permuted rows (zoe.im 范式 A Step 2,
 * "Grouped GEMM": one launch for all experts' GEMMs of different sizes).
 * For expert e and each row r in [offsets[e], offsets[e+1]):
 *   h[r]        = bf16( silu(x_perm[r] . Wg[e]^T) * (x_perm[r] . Wu[e]^T) )
 *   out_perm[r] = bf16( h[r] . Wd[e]^T ),          silu(g) = g / (1 + e^-g)
 * with fp32 accumulation.  Rows outside every segment are not written.
 *   x_perm         [R, D] bf16;  expert_offsets [E+1] int32 (non-decreasing,
 *                  offsets[E] <= R; not checked on the device).
 *   w_gate, w_up   [E, F, D] bf16;  w_down [E, D, F] bf16.
 *   out_perm       [R, D] bf16 out.
 *   h              [R, F] bf16 out, or NULL to keep it in the workspace.
 * Workspace: needed only when h is NULL; moe_workspace_size bytes suffice. */
moe_status moe_grouped_ffn(const moe_problem* p, const uint16_t* x_perm,
                           const int32_t* expert_offsets, const uint16_t* w_gate,
                           const uint16_t* w_up, const uint16_t* w_down, uint16_t* out_perm,
                           uint16_t* h, void* ws, size_t ws_bytes, void* stream);

/* The two GEMMs of the expert FFN as separate launches (moe_grouped_ffn is
 * moe_expert_gateup followed by moe_expert_down).  Same arguments, layouts
 * and row coverage as moe_grouped_ffn; neither needs a workspace.
 *   moe_expert_gateup: h [R, F] bf16 out from x_perm, w_gate, w_up.
 *   moe_expert_down  : out_perm [R, D] bf16 out from h, w_down. */
moe_status moe_expert_gateup(const moe_problem* p, const uint16_t* x_perm,
                             const int32_t* expert_offsets, const uint16_t* w_gate,
                             const uint16_t* w_up, uint16_t* h, void* stream);
moe_status moe_expert_down(const moe_problem* p, const uint16_t* h,
                           const int32_t* expert_offsets, const uint16_t* w_down,
                           uint16_t* out_perm, void* stream);

/* moe_expert_gateup on x[row_token] without the permuted copy: each tile
 * reads its rows of x through row_token (the dispatch of zoe.im 范式 A Step 1
 * folded into the GEMM's loads, as moe_fused_ffn does).  With it,
 * moe_permute can be called with x_perm = NULL.  h is bit for bit what
 * moe_expert_gateup writes from x_perm = x[row_token].
 *   x [N, D] bf16; row_token [R] int32 and expert_offsets [E+1] int32 as
 *   written by moe_permute (values of row_token not checked on the device);
 *   w_gate, w_up [E, F, D] bf16; h [R, F] bf16 out.
 * MOE_ERR_UNSUPPORTED for a padded problem (its padding rows have no token),
 * for N * D * 2 >= 2^32 bytes of x, and where the tile shape has no gathered
 * form: R / E <= 48 rows per expert with D < 1024.  Needs no workspace. */
moe_status moe_expert_gateup_gathered(const moe_problem* p, const uint16_t* x,
                                      const int32_t* row_token, const int32_t* expert_offsets,
                                      const uint16_t* w_gate, const uint16_t* w_up, uint16_t* h,
                                      void* stream);

/* Un-permutation and weighted combine (zoe.im 范式 A Step 3):
 *   y[n] = bf16( sum_{k=0..K-1, slot_row[n*K+k] >= 0} w[n,k] * out_perm[slot_row[n*K+k]] )
 * summed in k order in fp32.  Dropped slots contribute nothing and the kept
 * weights are not renormalised.
 *   out_perm [R, D] bf16; slot_row [N*K] int32 (values < R; not checked on
 *   the device); topk_weights [N, K] fp32; y [N, D] bf16 out.
 * Needs no workspace. */
moe_status moe_unpermute_combine(const moe_problem* p, const uint16_t* out_perm,
                                 const int32_t* slot_row, const float* topk_weights,
                                 uint16_t* y, void* stream);

/* The whole layer: moe_route, moe_permute, moe_grouped_ffn and
 * moe_unpermute_combine in sequence on one stream.  Where
 * moe_expert_gateup_gathered takes the problem, the gate/up GEMM runs as it
 * (rows read from x through row_token) and no permuted copy of x is
 * written; y is the same bit for bit.
 *   x [N, D] bf16; w_router [E, D] fp32; expert_bias [E] fp32 or NULL;
 *   w_gate, w_up [E, F, D] bf16; w_down [E, D, F] bf16; y [N, D] bf16 out.
 *   logits [N, E], topk_ids [N, K], topk_weights [N, K], expert_counts [E],
 *   expert_offsets [E+1]: optional outputs (NULL = kept in the workspace).
 * Workspace: moe_workspace_size(p) bytes. */
moe_status moe_forward(const moe_problem* p, const uint16_t* x, const float* w_router,
                       const float* expert_bias, const uint16_t* w_gate, const uint16_t* w_up,
                       const uint16_t* w_down, uint16_t* y, float* logits, int32_t* topk_ids,
                       float* topk_weights, int32_t* expert_counts, int32_t* expert_offsets,
                       void* ws, size_t ws_bytes, void* stream);

/* moe_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops (a decode step), harnesses that forbid
 * hipMalloc.  It takes no workspace: the one moe_forward needs lives in a
 * static device array of MOE_STATIC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends (its address is looked up once
 * per device, on the first call there).  No call allocates or frees memory.
 *   Arguments, outputs and results as moe_forward (bit for bit the same).
 *   MOE_ERR_WORKSPACE, before any HIP call, when moe_workspace_size(p)
 *   exceeds MOE_STATIC_SCRATCH_BYTES (e.g. a decode step of the Qwen3-30B-A3B
 *   layer shape needs about 2.8 MB; prefill batches do not fit).
 *   The scratch is shared by every call on one GPU and keeps the last call's
 *   contents; nothing in it needs to start at zero.  Calls that overlap on
 *   one GPU (other streams, other threads) race on it and give undefined
 *   results: serialise them. */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)
moe_status moe_forward_static(const moe_problem* p, const uint16_t* x, const float* w_router,
                              const float* expert_bias, const uint16_t* w_gate,
                              const uint16_t* w_up, const uint16_t* w_down, uint16_t* y,
                              float* logits, int32_t* topk_ids, float* topk_weights,
                              int32_t* expert_counts, int32_t* expert_offsets, void* stream);

/* ------------------------------------------------------------ fused FFN */
/* The whole expert FFN as one persistent launch (the single-kernel MoE of
 * "MoE 推理完整机制" (zoe.im) 第四层, DeepGEMM & MegaMoE Kernel: workgroups
 * claim the gate/up tiles, then the down tiles, of every expert at run time).  Same
 * results as moe_grouped_ffn on x_perm = x[row_token] (bit for bit), but the
 * gate/up tiles gather their rows from x through row_token, so no permuted
 * copy of x exists, and down tiles of an expert's rows start as soon as that
 * row range's h is complete.  Contiguous layout only (MOE_ERR_UNSUPPORTED
 * for a padded problem) and N * D * 2 < 2^32 bytes of x.
 *   x [N, D] bf16; row_token [R] int32 and expert_offsets [E+1] int32 as
 *   written by moe_permute; weights as moe_grouped_ffn; out_perm [R, D] out.
 * Workspace: moe_workspace_size(p) bytes suffice (it holds h and the
 * launch's counters).  A wait inside the launch is bounded: if one ever ran
 * past its bound the results are wrong and the int32 error word at byte
 * offset moe_fused_error_offset(p, 0, &off) of the workspace is nonzero after
 * the call completes (zero otherwise). */
moe_status moe_fused_ffn(const moe_problem* p, const uint16_t* x, const int32_t* row_token,
                         const int32_t* expert_offsets, const uint16_t* w_gate,
                         const uint16_t* w_up, const uint16_t* w_down, uint16_t* out_perm,
                         void* ws, size_t ws_bytes, void* stream);
/* moe_forward with the fused FFN: moe_route, moe_permute (routing tables only,
 * no x_perm), moe_fused_ffn and moe_unpermute_combine.  Arguments as
 * moe_forward; contiguous layout only.  Its error word is at
 * moe_fused_error_offset(p, 1, &off). */
moe_status moe_forward_fused(const moe_problem* p, const uint16_t* x, const float* w_router,
                             const float* expert_bias, const uint16_t* w_gate,
                             const uint16_t* w_up, const uint16_t* w_down, uint16_t* y,
                             float* logits, int32_t* topk_ids, float* topk_weights,
                             int32_t* expert_counts, int32_t* expert_offsets, void* ws,
                             size_t ws_bytes, void* stream);
/* Host only: byte offset of the fused launch's error word in the workspace of
 * moe_fused_ffn (whole_layer = 0) or moe_forward_fused (whole_layer = 1). */
moe_status moe_fused_error_offset(const moe_problem* p, int32_t whole_layer, size_t* offset);

/* ------------------------------------------- GELU experts and the MLP router */
/* The second MoE layer of "MoE工程实战" (jsqmd.com): a router that first
 * compresses the hidden state with a 2-layer MLP (section 3.1 输入表征:
 * Linear(D, D/4) + GELU, then the gate Linear(D/4, E)), top-K with softmax
 * over the selected, and experts Linear(D, 4D) - GELU - Linear(4D, D)
 * (section 4.2, MoELayer).  Every Linear has its bias (nn.Linear's default);
 * GELU is the exact form v * Phi(v).  The expert width F is the problem's
 * `ffn` (4D on the page, any multiple of 64 here).  The MLP router needs
 * D % 256 == 0 (MOE_ERR_UNSUPPORTED else).  Storage and accumulation as in
 * the SwiGLU layer: bf16 activations, fp32 accumulation and biases. */

/* MLP router:
 *   features[n] = bf16( GELU(x[n] . W_proj^T + b_proj) )     [N, D/4]
 *   logits[n]   = fp32( features[n] . W_out^T )              [N, E] (no bias)
 *   top-K and weights as moe_route with b_out as the per-expert bias, i.e.
 *   on the biased gate logits logits + b_out.
 *   x [N, D] bf16; w_proj [D/4, D] bf16; b_proj [D/4] fp32; w_out [E, D/4]
 *   fp32; b_out [E] fp32 or NULL (no bias); features bf16 out or NULL (kept in
 *   the workspace); logits, topk_ids, topk_weights as in moe_route.
 * Workspace: moe_workspace_size(p) bytes. */
moe_status moe_route_mlp(const moe_problem* p, const uint16_t* x, const uint16_t* w_proj,
                         const float* b_proj, const float* w_out, const float* b_out,
                         uint16_t* features, float* logits, int32_t* topk_ids,
                         float* topk_weights, void* ws, size_t ws_bytes, void* stream);

/* GELU expert FFN over the permuted rows, for expert e and each row r of its
 * segment:
 *   h[r]        = bf16( GELU(x_perm[r] . W1[e]^T + b1[e]) )
 *   out_perm[r] = bf16( h[r] . W2[e]^T + b2[e] )
 *   w1 [E, F, D] bf16, b1 [E, F] fp32, w2 [E, D, F] bf16, b2 [E, D] fp32.
 * Padding rows of a capacity-padded buffer are zero inputs; their out_perm
 * rows hold the expert's response to a zero row (its biases), which the
 * combine never reads.  moe_grouped_ffn_gelu = moe_expert_up_gelu followed
 * by moe_expert_down_bias; arguments, coverage, workspace and errors as in
 * moe_grouped_ffn / moe_expert_gateup / moe_expert_down. */
moe_status moe_expert_up_gelu(const moe_problem* p, const uint16_t* x_perm,
                              const int32_t* expert_offsets, const uint16_t* w1, const float* b1,
                              uint16_t* h, void* stream);
/* moe_expert_up_gelu on x[row_token] without the permuted copy, as
 * moe_expert_gateup_gathered is to moe_expert_gateup (same arguments for x
 * and row_token, same refusals); h bit for bit that of moe_expert_up_gelu.
 * moe_forward_gelu uses it where the problem allows. */
moe_status moe_expert_up_gelu_gathered(const moe_problem* p, const uint16_t* x,
                                       const int32_t* row_token, const int32_t* expert_offsets,
                                       const uint16_t* w1, const float* b1, uint16_t* h,
                                       void* stream);
moe_status moe_expert_down_bias(const moe_problem* p, const uint16_t* h,
                                const int32_t* expert_offsets, const uint16_t* w2,
                                const float* b2, uint16_t* out_perm, void* stream);
moe_status moe_grouped_ffn_gelu(const moe_problem* p, const uint16_t* x_perm,
                                const int32_t* expert_offsets, const uint16_t* w1,
                                const float* b1, const uint16_t* w2, const float* b2,
                                uint16_t* out_perm, uint16_t* h, void* ws, size_t ws_bytes,
                                void* stream);

/* The whole GELU-expert layer: moe_route_mlp, moe_permute,
 * moe_grouped_ffn_gelu and moe_unpermute_combine on one stream.  Optional
 * outputs and workspace as in moe_forward (the features stay in the
 * workspace). */
moe_status moe_forward_gelu(const moe_problem* p, const uint16_t* x, const uint16_t* w_proj,
                            const float* b_proj, const float* w_out, const float* b_out,
                            const uint16_t* w1, const float* b1, const uint16_t* w2,
                            const float* b2, uint16_t* y, float* logits, int32_t* topk_ids,
                            float* topk_weights, int32_t* expert_counts,
                            int32_t* expert_offsets, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------ block-scaled FP8 weights */
/* Expert weights stored as FP8 with block scales, read by the grouped FFN and
 * dequantised inside its kernels: the FP8 weights of the grouped-GEMM kernel
 * in "MoE 推理完整机制" (zoe.im) 第四层 (DeepGEMM & MegaMoE Kernel) and the
 * 8-bit expert weights of "MoE工程实战" (jsqmd.com) 5.3 技巧2.  Format (the
 * OCP microscaling layout with E4M3 elements; the pages fix no format):
 *   - 32 consecutive values along a weight row's input dimension (the
 *     contraction dimension: D for gate/up, F for down) form a block with one
 *     scale 2^s, stored as the byte s + 127 (E8M0).
 *   - codes [rows, cols] uint8, each an E4M3 value (sign, 4 exponent bits with
 *     bias 7, 3 mantissa bits; S.1111.111 is NaN, no infinity, max 448).
 *   - scales, blocked by 32 rows: the scale of rows [32g, 32g+32) and k-block
 *     kb sits at byte ((g * (cols/32)) + kb) * 32 + (row - 32g), i.e. a
 *     [rows/32, cols/32, 32] uint8 array.
 *   - weight value = E4M3(code) * 2^(byte - 127), exactly a bf16 number for the
 *     scale bytes 10..246 that moe_quantize_fp8 writes; other bytes give
 *     unspecified values (never a fault).
 * An expert stack [E, rows, cols] is E such matrices back to back (codes
 * [E, rows, cols], scales [E, rows/32, cols/32, 32]).  The FFN runs on the
 * dequantised values: the FP8 entry points give bit-identical results to the
 * bf16 ones called with the dequantised weights. */

/* Quantise bf16 weights [rows, cols] (rows, cols multiples of 32; w and
 * codes 16-byte aligned; MOE_ERR_UNSUPPORTED else) into codes and scales as
 * above.  Per block: s = floor(log2(largest finite |w|)) - 8, clamped to
 * [-117, 119] (all-zero blocks take -117); code = w / 2^s rounded to the
 * nearest E4M3 value, ties to even, saturating at +-448; infinities and NaNs
 * give NaN codes.  Pass rows = E * per-expert rows for a whole stack.  Exact
 * integer work: the output depends only on the input bits.  Needs no
 * workspace; rows == 0 launches nothing. */
moe_status moe_quantize_fp8(int64_t rows, int32_t cols, const uint16_t* w, uint8_t* codes,
                            uint8_t* scales, void* stream);

/* moe_expert_gateup / moe_expert_down / moe_grouped_ffn / moe_forward with
 * FP8 weight stacks in place of the bf16 ones (moe_forward_fp8 gathers the
 * gate/up rows from x as moe_forward does): w_gate_*, w_up_* [E, F, D]
 * (scales [E, F/32, D/32, 32]), w_down_* [E, D, F] (scales
 * [E, D/32, F/32, 32]).  Codes and scales must be 16-byte aligned
 * (MOE_ERR_UNSUPPORTED else).  Everything else -- shapes, layouts, row
 * coverage, workspace, errors -- as in the bf16 calls. */
moe_status moe_expert_gateup_fp8(const moe_problem* p, const uint16_t* x_perm,
                                 const int32_t* expert_offsets, const uint8_t* w_gate_codes,
                                 const uint8_t* w_gate_scales, const uint8_t* w_up_codes,
                                 const uint8_t* w_up_scales, uint16_t* h, void* stream);
/* moe_expert_gateup_gathered with FP8 weight stacks: rows read from x through
 * row_token, h bit for bit that of moe_expert_gateup_fp8 on x_perm =
 * x[row_token].  Refused (MOE_ERR_UNSUPPORTED) as the bf16 call, except that
 * with R / E <= 48 the FP8 tiles also take D >= 512 in multiples of 128. */
moe_status moe_expert_gateup_fp8_gathered(const moe_problem* p, const uint16_t* x,
                                          const int32_t* row_token,
                                          const int32_t* expert_offsets,
                                          const uint8_t* w_gate_codes,
                                          const uint8_t* w_gate_scales,
                                          const uint8_t* w_up_codes, const uint8_t* w_up_scales,
                                          uint16_t* h, void* stream);
moe_status moe_expert_down_fp8(const moe_problem* p, const uint16_t* h,
                               const int32_t* expert_offsets, const uint8_t* w_down_codes,
                               const uint8_t* w_down_scales, uint16_t* out_perm, void* stream);
moe_status moe_grouped_ffn_fp8(const moe_problem* p, const uint16_t* x_perm,
                               const int32_t* expert_offsets, const uint8_t* w_gate_codes,
                               const uint8_t* w_gate_scales, const uint8_t* w_up_codes,
                               const uint8_t* w_up_scales, const uint8_t* w_down_codes,
                               const uint8_t* w_down_scales, uint16_t* out_perm, uint16_t* h,
                               void* ws, size_t ws_bytes, void* stream);
moe_status moe_forward_fp8(const moe_problem* p, const uint16_t* x, const float* w_router,
                           const float* expert_bias, const uint8_t* w_gate_codes,
                           const uint8_t* w_gate_scales, const uint8_t* w_up_codes,
                           const uint8_t* w_up_scales, const uint8_t* w_down_codes,
                           const uint8_t* w_down_scales, uint16_t* y, float* logits,
                           int32_t* topk_ids, float* topk_weights, int32_t* expert_counts,
                           int32_t* expert_offsets, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------ packed bf16 weights */
/* Expert weights in this library's packed layout: the same bf16 values as
 * the nn.Linear stacks, reordered once (at load time) so that the grouped
 * GEMMs of "MoE 推理完整机制" (zoe.im) 第二层 范式 A ("关键 kernel: Grouped
 * GEMM") stream every weight stage as one contiguous block.  The pages fix no
 * storage order; this one is the image each 256-row, 64-deep weight stage
 * has in the kernels' LDS:
 *   - a stack is cut into column panels: gate/up panels of 128 columns of h
 *     (the 128 gate rows and the matching 128 up rows, interleaved in blocks
 *     of 32: gate rows for even blocks, up rows for odd ones), down panels
 *     of 256 output columns;
 *   - each panel into 64-deep stages along the contraction dimension;
 *   - each stage is 32768 bytes: row r of the panel (0..255) at bytes
 *     [128 r, 128 r + 128), its 8 chunks of 8 values stored with chunk c at
 *     position c ^ ((r / 2) % 8);
 *   - stages in the order (expert, panel, stage).  Rows past the matrix
 *     (F % 128 != 0 for gate/up, D % 256 != 0 for down) repeat its last row.
 * The layout is an internal format: write it with moe_pack_weights only.  The
 * packed entry points give bit-identical results to the bf16 ones on the
 * weights that were packed. */
typedef enum {
  MOE_PACK_GATEUP = 0,
  MOE_PACK_DOWN = 1,
  MOE_PACK_GATEUP_FP8 = 2,  /* FP8 codes: see moe_pack_weights_fp8 */
  MOE_PACK_DOWN_FP8 = 3
} moe_pack_kind;

/* Bytes of a packed stack of `kind` for problem p (host; N is ignored):
 * E * ceil(F / 128) * (D / 64) * 32768 for MOE_PACK_GATEUP,
 * E * ceil(D / 256) * (F / 64) * 32768 for MOE_PACK_DOWN,
 * E * ceil(F / 128) * (D / 128) * 32768 for MOE_PACK_GATEUP_FP8 (D a
 * multiple of 128, MOE_ERR_UNSUPPORTED else),
 * E * ceil(D / 256) * (F / 128) * 32768 for MOE_PACK_DOWN_FP8 (F a multiple
 * of 128). */
moe_status moe_packed_weight_size(const moe_problem* p, int32_t kind, size_t* bytes);

/* Pack a stack: MOE_PACK_GATEUP reads w0 = W_gate and w1 = W_up [E, F, D]
 * bf16, MOE_PACK_DOWN reads w0 = W_down [E, D, F] (w1 unused, may be NULL).
 * packed: moe_packed_weight_size bytes, written whole.  All pointers 16-byte
 * aligned (MOE_ERR_UNSUPPORTED else).  A copy: the output depends only on
 * the input bits.  Needs no workspace; runs whatever num_tokens is. */
moe_status moe_pack_weights(const moe_problem* p, int32_t kind, const uint16_t* w0,
                            const uint16_t* w1, uint16_t* packed, void* stream);

/* moe_expert_gateup / moe_expert_gateup_gathered / moe_expert_down /
 * moe_forward with packed stacks in place of the bf16 ones: w_gateup_packed
 * from MOE_PACK_GATEUP, w_down_packed from MOE_PACK_DOWN, both 16-byte
 * aligned.  Everything else -- shapes, layouts, row coverage, workspace,
 * errors -- as in the bf16 calls, and the outputs are bit for bit theirs. */
moe_status moe_expert_gateup_packed(const moe_problem* p, const uint16_t* x_perm,
                                    const int32_t* expert_offsets,
                                    const uint16_t* w_gateup_packed, uint16_t* h, void* stream);
moe_status moe_expert_gateup_packed_gathered(const moe_problem* p, const uint16_t* x,
                                             const int32_t* row_token,
                                             const int32_t* expert_offsets,
                                             const uint16_t* w_gateup_packed, uint16_t* h,
                                             void* stream);
moe_status moe_expert_down_packed(const moe_problem* p, const uint16_t* h,
                                  const int32_t* expert_offsets, const uint16_t* w_down_packed,
                                  uint16_t* out_perm, void* stream);
moe_status moe_forward_packed(const moe_problem* p, const uint16_t* x, const float* w_router,
                              const float* expert_bias, const uint16_t* w_gateup_packed,
                              const uint16_t* w_down_packed, uint16_t* y, float* logits,
                              int32_t* topk_ids, float* topk_weights, int32_t* expert_counts,
                              int32_t* expert_offsets, void* ws, size_t ws_bytes, void* stream);

/* Packed FP8 codes.  The codes of a block-scaled FP8 stack (the format of
 * moe_quantize_fp8) in the same layout with stages 128 codes deep: a stage
 * is row r of the panel at bytes [128 r, 128 r + 128), its 16-byte chunk c
 * (codes 16c .. 16c + 15 of the stage) at position c ^ ((r / 2) % 8).  The
 * scales are not packed: the calls below take them in their own layout.
 * moe_pack_weights_fp8: MOE_PACK_GATEUP_FP8 reads c0 = the W_gate codes and
 * c1 = the W_up codes [E, F, D], MOE_PACK_DOWN_FP8 reads c0 = the W_down
 * codes [E, D, F] (c1 unused, may be NULL); packed: moe_packed_weight_size
 * bytes, written whole.  The contraction length (D, resp. F) must be a
 * multiple of 128, all pointers 16-byte aligned (MOE_ERR_UNSUPPORTED else).
 * A copy; needs no workspace; runs whatever num_tokens is. */
moe_status moe_pack_weights_fp8(const moe_problem* p, int32_t kind, const uint8_t* c0,
                                const uint8_t* c1, uint8_t* packed, void* stream);

/* moe_expert_gateup_fp8 / moe_expert_gateup_fp8_gathered / moe_expert_down_fp8
 * / moe_forward_fp8 with packed codes: w_gateup_packed from
 * MOE_PACK_GATEUP_FP8 with the gate and up scales of the stacks it was packed
 * from, w_down_packed from MOE_PACK_DOWN_FP8 with the down scales.  D (gate/up)
 * and F (down) multiples of 128 (MOE_ERR_UNSUPPORTED else); the gathered
 * gate/up then takes every D.  Everything else as in the FP8 calls, and the
 * outputs are bit for bit theirs. */
moe_status moe_expert_gateup_fp8_packed(const moe_problem* p, const uint16_t* x_perm,
                                        const int32_t* expert_offsets,
                                        const uint8_t* w_gateup_packed,
                                        const uint8_t* w_gate_scales, const uint8_t* w_up_scales,
                                        uint16_t* h, void* stream);
moe_status moe_expert_gateup_fp8_packed_gathered(const moe_problem* p, const uint16_t* x,
                                                 const int32_t* row_token,
                                                 const int32_t* expert_offsets,
                                                 const uint8_t* w_gateup_packed,
                                                 const uint8_t* w_gate_scales,
                                                 const uint8_t* w_up_scales, uint16_t* h,
                                                 void* stream);
moe_status moe_expert_down_fp8_packed(const moe_problem* p, const uint16_t* h,
                                      const int32_t* expert_offsets,
                                      const uint8_t* w_down_packed,
                                      const uint8_t* w_down_scales, uint16_t* out_perm,
                                      void* stream);
moe_status moe_forward_fp8_packed(const moe_problem* p, const uint16_t* x, const float* w_router,
                                  const float* expert_bias, const uint8_t* w_gateup_packed,
                                  const uint8_t* w_gate_scales, const uint8_t* w_up_scales,
                                  const uint8_t* w_down_packed, const uint8_t* w_down_scales,
                                  uint16_t* y, float* logits, int32_t* topk_ids,
                                  float* topk_weights, int32_t* expert_counts,
                                  int32_t* expert_offsets, void* ws, size_t ws_bytes,
                                  void* stream);

/* ------------------------------------------------------ routing statistics */

/* Router load statistics and dynamic expert bias ("MoE 大规模分布式推理工程实战"
 * (ybb.press), 4.1: the EMA of the per-expert routing fraction and the bias
 * update of its load-balancing step).  In place, on `stream`:
 *   f[e]    = expert_counts[e] / sum(expert_counts)
 *   ema[e]  = decay * ema[e] + (1 - decay) * f[e]
 *   bias[e] = bias[e] + (E * ema[e] / sum(ema) - 1) * step
 * A batch with sum(expert_counts) == 0 changes nothing.  As printed on the
 * page (step 0.1, decay 0.99) the update raises the bias of experts above the
 * uniform share; pass a negative step for the opposite direction.  The bias
 * buffer is the expert_bias that moe_route / moe_forward add to the logits.
 *   num_experts    E, 1 <= E <= 1024 (MOE_ERR_UNSUPPORTED above)
 *   expert_counts  [E] int32 (as written by moe_permute / moe_forward)
 *   ema            [E] fp32, in/out (start from 1/E)
 *   expert_bias    [E] fp32, in/out
 *   decay          in [0, 1]; step: any finite value (MOE_ERR_INVALID_ARG else)
 * fp32 arithmetic; the sums over experts use a fixed reduction order. */
moe_status moe_routing_stats(int32_t num_experts, const int32_t* expert_counts, float* ema,
                             float* expert_bias, float decay, float step, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBMOE_MOE_H_ */
