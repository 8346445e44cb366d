/*
 * moe.h - C ABI of the MI355X (gfx950) Mixture-of-Experts layer forward pass.
 *
 * One MoE layer on one GPU's share of T tokens: a top-k softmax gate, Dispatch
 * of every (token, slot) assignment into per-expert contiguous rows, the
 * routed SwiGLU experts run as a grouped GEMM, optional always-on shared
 * experts, and Combine back to token order.  The operator chain is the MoE
 * sub-block of the FarSkip-Collective review ("Core claim"; Fig. 2 caption,
 * on the MoE layer's main operators; Fig. 11 caption: Dispatch, routed
 * experts, Combine, shared expert).  Top-k routing is the gate of the
 * expert-prototyping abstract on the "Daily Papers" search page; running each
 * expert as one dense product over its grouped tokens is the "Expert-Centric
 * Scheduling" of the OmniMoE abstract on that page.  The layer's formulas are
 * not written on the pages; the readings used here are:
 *
 *   L[t,e]   = sum_i x[t,i] * w_router[e,i] + bias[e]            (fp32)
 *   ids[t,j] = expert with the (j+1)-th largest L[t,.]; equal logits go to
 *              the lower expert index
 *   w[t,j]   = exp(L[t,ids[t,j]] - L[t,ids[t,0]]) / sum_j' (same)
 *              (= softmax over all E restricted to the top k, renormalised)
 *   rows of expert e: assignments a = t*k + j with ids[t,j] == e, ascending a
 *   A        = bf16(silu(X Wg^T) * (X Wu^T)), silu(z) = z / (1 + e^-z)
 *              (fp32 workloads keep A in fp32)
 *   y        = A Wd^T                                              (fp32)
 *   shared   = sum_s  bf16(silu(x Wsg_s^T) * (x Wsu_s^T)) Wsd_s^T  (fp32)
 *   out[t]   = sum_j w[t,j] * y[row of (t,j)] + shared[t]         (fp32)
 *
 * Conventions for every entry point
 * ---------------------------------
 * Layouts: row-major, reduction dimension contiguous.
 *   x [T,d]; w_router [E,d]; bias [E] (fp32);
 *   w_gate, w_up [E,I,d]; w_down [E,d,I];
 *   wsh_gate, wsh_up [n_shared,I_shared,d]; wsh_down [n_shared,d,I_shared].
 *   dims.dtype gives the element type of x and of every weight tensor
 *   (MOE_BF16: bfloat16, MOE_F32: float32).  Everything else is int32 or fp32.
 * Ownership: the caller owns every buffer.  All pointers are device pointers,
 *   16-byte aligned, and no output may overlap another buffer.  The library
 *   allocates nothing and keeps no state; its entry points are re-entrant.
 * Asynchrony: work is enqueued on `stream` (0 = the null stream).  No entry
 *   point synchronises or copies device data to the host; MOE_OK means
 *   "enqueued".
 * Errors: arguments are validated on the host before anything is enqueued;
 *   on a validation failure nothing is enqueued and no output is touched.
 *   A failed launch returns MOE_ERR_HIP.  Limits: T >= 0 (with T == 0 only
 *   the per-expert counts and offsets are written, as zeros, by moe_dispatch
 *   and moe_layer_fwd); 1 <= k <= min(E, 16); E <= 256;
 *   d % 64 == 0; I % 64 == 0; I_shared % 64 == 0; T*k < 2^31;
 *   n_shared == 0 exactly when I_shared == 0.
 *   Expert ids outside [0,E) given to moe_dispatch are skipped (the
 *   assignment gets no row); results are then meaningless but every kernel
 *   keeps its memory accesses in bounds.
 * Determinism: no floating-point atomics; two calls on the same inputs give
 *   bit-identical outputs.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#if defined(__GNUC__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null, misaligned or overlapping pointer; bad sizes */
  MOE_ERR_UNSUPPORTED = 2, /* sizes outside the limits above */
  MOE_ERR_WORKSPACE = 3,   /* ws_bytes below moe_workspace_bytes() */
  MOE_ERR_HIP = 4,         /* a kernel launch failed */
  MOE_ERR_SCRATCH = 5      /* moe_layer_fwd_static: the sizes need more workspace
                              than MOE_STATIC_SCRATCH_BYTES */
} moe_status_t;

/* Sizes of one layer call: T tokens, hidden size d, E routed experts, top-k,
 * expert intermediate size I, n_shared shared experts of intermediate size
 * I_shared, element type of x and the weights. */
typedef struct {
  int64_t T;
  int32_t d, E, k, I, n_shared, I_shared;
  moe_dtype_t dtype;
} moe_dims_t;

/* Bytes of device workspace that moe_dispatch, moe_grouped_ffn and
 * moe_layer_fwd need for `dims` (one size serves all three).  Returns 0 for
 * invalid or unsupported dims. */
MOE_API size_t moe_workspace_bytes(const moe_dims_t* dims);

/* Static, never-NULL description of a status code. */
MOE_API const char* moe_status_str(moe_status_t status);

/* Gate: router logits, top-k ids and renormalised softmax weights.
 * Passage: top-k routing over the router's scores is the gate of the
 * expert-prototyping abstract on the "Daily Papers" search page (top-2 in the
 * ScMoE abstract there); its time is the T_gate term of the overlap window in
 * the FarSkip-Collective review (axiom ledger, Eq. 9).  Softmax, renormalising
 * over the kept k and the lower-index tie rule are readings (see the header).
 *   x [T,d], w_router [E,d] (dtype); bias [E] fp32 or NULL.
 *   logits_in [T,E] fp32 or NULL: when given, the top-k is taken on these
 *     logits and x, w_router and bias are not read (may be NULL).
 *   logits_out [T,E] fp32 or NULL: receives the logits the top-k used.
 *   topk_ids [T,k] int32, topk_w [T,k] fp32: outputs, slot 0 = largest logit.
 * bf16 logits: bf16 products accumulated in fp32 on the matrix cores.
 * fp32 logits: per (t,e), 64 partial sums (partial l takes i = l, l+64, ... in
 *   ascending i, separate multiply and add), a xor butterfly over 32,16,8,4,2,1,
 *   then + bias; all in fp32 round-to-nearest. */
MOE_API moe_status_t moe_route(const moe_dims_t* dims, const void* x, const void* w_router,
                       const float* bias, const float* logits_in, float* logits_out,
                       int32_t* topk_ids, float* topk_w, hipStream_t stream);

/* Dispatch: group the R = T*k assignments a = t*k + j by expert, stably.
 * Passage: Dispatch, the token traffic that sends each token to its experts
 * (FarSkip-Collective review, "Core claim" and Fig. 11 caption; the Luffy
 * review, "Core claim", on dispatch and combine traffic).  On one GPU's share
 * it is a stable counting sort plus a row gather; the row order inside a
 * segment (ascending a) is a reading.
 *   topk_ids [T,k] int32 in [0,E).
 *   counts [E]: assignments per expert.  offsets [E+1]: exclusive prefix sum,
 *   offsets[E] = R.  perm [R]: perm[i] = assignment at sorted row i.
 *   inv_perm [R]: inv_perm[a] = sorted row of assignment a.
 *   x_sorted [R,d] (dtype): x_sorted[i] = x[perm[i] / k].
 *   ws: workspace of ws_bytes >= moe_workspace_bytes(dims). */
MOE_API moe_status_t moe_dispatch(const moe_dims_t* dims, const void* x, const int32_t* topk_ids,
                          int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                          void* x_sorted, void* ws, size_t ws_bytes, hipStream_t stream);

/* Routed experts as a grouped GEMM, plus the shared experts.
 * Passage: the routed experts are the T_routed term of the FarSkip-Collective
 * review's overlap window (axiom ledger, Eq. 9) and the always-on shared expert
 * is the branch its Fig. 11 caption runs beside Combine; one dense product per
 * expert over its grouped tokens is the "Expert-Centric Scheduling" of the
 * OmniMoE abstract on the "Daily Papers" search page.  The SwiGLU form of the
 * expert and the bf16 rounding of A are readings.
 *   x_sorted [R,d] (dtype) and offsets [E+1] as produced by moe_dispatch.
 *   w_gate, w_up [E,I,d], w_down [E,d,I] (dtype).
 *   x [T,d] and wsh_* : shared experts; NULL when n_shared == 0.
 *   y_sorted [R,d] fp32: y_sorted[i] = expert output of sorted row i.
 *   y_shared [T,d] fp32: sum of the shared experts; NULL when n_shared == 0.
 *   On return the workspace starts with A [R,I] followed by A_shared
 *   [T, n_shared*I_shared], the SwiGLU products (bf16 for MOE_BF16, fp32 for
 *   MOE_F32), each 256-byte aligned. */
MOE_API moe_status_t moe_grouped_ffn(const moe_dims_t* dims, const void* x_sorted, const int32_t* offsets,
                             const void* w_gate, const void* w_up, const void* w_down,
                             const void* x, const void* wsh_gate, const void* wsh_up,
                             const void* wsh_down, float* y_sorted, float* y_shared,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* Combine: out[t] = sum_{j<k} topk_w[t,j] * y_sorted[inv_perm[t*k+j]] (+ y_shared[t]),
 * Passage: Combine, the return of expert outputs to token order
 * (FarSkip-Collective review, "Core claim" and Fig. 11 caption; the Luffy
 * review, "Core claim").  The fp32 slot-order sum is a reading.
 * accumulated in fp32 in ascending j, shared term last.
 *   y_sorted [R,d], inv_perm [R], topk_w [T,k], y_shared [T,d] or NULL, out [T,d]. */
MOE_API moe_status_t moe_combine(const moe_dims_t* dims, const float* y_sorted, const int32_t* inv_perm,
                         const float* topk_w, const float* y_shared, float* out,
                         hipStream_t stream);

/* The whole layer: route, dispatch, grouped FFN with shared experts, combine.
 * Passage: the MoE sub-block as the FarSkip-Collective review lays out its
 * operators ("Core claim"; Fig. 2 caption on the MoE layer's main operators;
 * Fig. 11 caption: gate, Dispatch, routed experts, shared expert, Combine).
 *   Inputs as above (wsh_* NULL when n_shared == 0); out [T,d] fp32.
 *   topk_ids_out [T,k], topk_w_out [T,k], counts_out [E], offsets_out [E+1],
 *   perm_out [R]: optional copies of the intermediate results (NULL = skip).
 *   ws: workspace of ws_bytes >= moe_workspace_bytes(dims). */
MOE_API moe_status_t moe_layer_fwd(const moe_dims_t* dims, const void* x, const void* w_router,
                           const float* bias, const void* w_gate, const void* w_up,
                           const void* w_down, const void* wsh_gate, const void* wsh_up,
                           const void* wsh_down, float* out, int32_t* topk_ids_out,
                           float* topk_w_out, int32_t* counts_out, int32_t* offsets_out,
                           int32_t* perm_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Kernel variants, for tests and measurements that compare another kernel
 * path with the default one on the same inputs (the default entry points
 * take variant 0; the choice is always the caller's, never the environment's).
 * MOE_VARIANT_GLOBAL_LOADS: the grouped GEMMs take their operands through
 *   64-bit global loads, the form the library otherwise takes only when an
 *   operand's byte offsets exceed 32 bits; same data in LDS, same MFMA order,
 *   so results are bit-identical to variant 0.
 * MOE_VARIANT_BWD_VALU (moe_layer_bwd_variant only): for fp32 layers the
 *   gradient products run on the vector ALUs in fp32 instead of the matrix
 *   cores with bf16 hi/lo operand parts; ignored for bf16 layers.
 * Any other bit: MOE_ERR_INVALID_ARG. */
#define MOE_VARIANT_GLOBAL_LOADS 1
#define MOE_VARIANT_BWD_VALU 2

/* moe_layer_fwd through the kernel variant `variant` (MOE_VARIANT_GLOBAL_LOADS
 * or 0); every other argument and the result as moe_layer_fwd. */
MOE_API moe_status_t moe_layer_fwd_variant(const moe_dims_t* dims, const void* x,
                                           const void* w_router, const float* bias,
                                           const void* w_gate, const void* w_up,
                                           const void* w_down, const void* wsh_gate,
                                           const void* wsh_up, const void* wsh_down, float* out,
                                           int32_t* topk_ids_out, float* topk_w_out,
                                           int32_t* counts_out, int32_t* offsets_out,
                                           int32_t* perm_out, void* ws, size_t ws_bytes,
                                           int variant, hipStream_t stream);

/* Bytes of the device scratch array behind moe_layer_fwd_static (one per GPU). */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/* moe_layer_fwd without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The workspace is a
 * file-scope device array of MOE_STATIC_SCRATCH_BYTES (64 MiB) in the library,
 * one per GPU, held from the first call on that GPU until the process ends;
 * the call makes no hipMalloc, hipFree or other allocating call.
 *   Sizes: moe_workspace_bytes(dims) must be at most MOE_STATIC_SCRATCH_BYTES,
 *     else MOE_ERR_SCRATCH and nothing is enqueued (e.g. 4096 tokens of d =
 *     2048, 64 experts top-6 of I = 1408 need about 320 MB: too many; the
 *     same layer fits up to about 800 tokens).
 *   Every call on one GPU shares that GPU's array and leaves its last
 *   contents there (every part is written before it is read, so no clearing is
 *   needed): calls that may overlap on one GPU (other streams, other host
 *   threads) race and must be serialised by the caller.
 * All other arguments, results, errors and the asynchrony are those of
 * moe_layer_fwd. */
MOE_API moe_status_t moe_layer_fwd_static(const moe_dims_t* dims, const void* x,
                                          const void* w_router, const float* bias,
                                          const void* w_gate, const void* w_up,
                                          const void* w_down, const void* wsh_gate,
                                          const void* wsh_up, const void* wsh_down, float* out,
                                          int32_t* topk_ids_out, float* topk_w_out,
                                          int32_t* counts_out, int32_t* offsets_out,
                                          int32_t* perm_out, hipStream_t stream);

/* moe_layer_fwd that also records HIP events on `stream` at its stage
 * boundaries, for per-stage timing.  events[0..n_events) are caller-created
 * events; event i is recorded after stage i-1 when i < n_events:
 *   0 start, 1 after route, 2 after dispatch (count, scan, rank, gather),
 *   3 after gate/up GEMM, 4 after down GEMM, 5 after combine.
 * n_events may be 0..6. */
MOE_API moe_status_t moe_layer_fwd_timed(const moe_dims_t* dims, const void* x, const void* w_router,
                                 const float* bias, const void* w_gate, const void* w_up,
                                 const void* w_down, const void* wsh_gate, const void* wsh_up,
                                 const void* wsh_down, float* out, int32_t* topk_ids_out,
                                 float* topk_w_out, int32_t* counts_out, int32_t* offsets_out,
                                 int32_t* perm_out, void* ws, size_t ws_bytes,
                                 hipEvent_t* events, int n_events, hipStream_t stream);

/* moe_layer_fwd with the shared experts on a second stream.  The shared
 * experts depend on x alone, so their two GEMMs run on `side` from the start,
 * beside the gate, the dispatch and the routed experts on `stream`; the
 * combine on `stream` waits for them.  This is the one-GPU form of running
 * the always-on shared expert concurrently with the routed path (the
 * FarSkip-Collective review: Fig. 11 caption, the shared expert beside
 * Combine; its second hardware queue in "What carries the argument").
 * Results are bit-identical to moe_layer_fwd (same kernels, same tiles).
 *   side: a stream other than `stream`, of the same device.
 *   fork, join: caller-owned events (timing may be disabled); `fork` is
 *     recorded on `stream` at entry, `join` on `side` after the shared
 *     experts.  Both are re-recorded on every call.
 * All other arguments and the workspace are those of moe_layer_fwd; the side
 * stream uses parts of the same workspace, so two calls that share a
 * workspace must not overlap.  NULL side, fork or join: MOE_ERR_INVALID_ARG.
 * Returns once both streams have their work enqueued. */
MOE_API moe_status_t moe_layer_fwd_overlap(const moe_dims_t* dims, const void* x, const void* w_router,
                                   const float* bias, const void* w_gate, const void* w_up,
                                   const void* w_down, const void* wsh_gate, const void* wsh_up,
                                   const void* wsh_down, float* out, int32_t* topk_ids_out,
                                   float* topk_w_out, int32_t* counts_out, int32_t* offsets_out,
                                   int32_t* perm_out, void* ws, size_t ws_bytes,
                                   hipStream_t stream, hipStream_t side, hipEvent_t fork,
                                   hipEvent_t join);

/* Workspace of moe_layer_fwd_condensed: moe_workspace_bytes plus the
 * condensation scratch (about 100 bytes per token).  0 for invalid dims. */
MOE_API size_t moe_condensed_workspace_bytes(const moe_dims_t* dims);

/* moe_layer_fwd with token condensation: a routed assignment whose token is
 * a near-duplicate of an earlier token routed to the same expert gets no row
 * of its own and reuses that token's expert output (the Luffy review, "Core
 * claim" and "What carries the argument": similar tokens bound for one
 * expert send one representative, whose expert output is reused).  The
 * result is an approximation of moe_layer_fwd; with cos_threshold > 1 it is
 * the same computation.
 *   Similar tokens are found in one pass (a reading; the pages' own
 *   measurement uses training history): each token gets a 16-bit key, bit b
 *   set when its projection onto hyperplane b is >= 0; tokens with equal keys
 *   form a bucket in ascending token order; token t's representative is the
 *   first of the bucket's first 32 members before t whose plain cosine with t
 *   is >= cos_threshold (computed in fp32), unless that member is itself
 *   condensed (then t stays).  Assignment (t, j) is condensed when t's
 *   representative is another token routed to the same expert.
 *   hyperplanes: [16, d], the dtype of x, device memory (the method's random
 *     draws, passed in); required.
 *   cos_threshold: the plain cosine bound (a [0,1]-normalised bound h is
 *     2h - 1); NaN: MOE_ERR_INVALID_ARG.
 *   rep_out: [T] int32 or NULL: each token's representative (itself when it
 *     is not condensed).
 *   counts_out, offsets_out, perm_out: the rows that exist, i.e. the
 *     assignments that are not condensed; perm_out is written up to
 *     offsets[E] only.  topk_ids_out, topk_w_out: as in moe_layer_fwd.
 *   ws: ws_bytes >= moe_condensed_workspace_bytes(dims).
 * All other arguments, errors and the asynchrony are those of moe_layer_fwd;
 * the shared experts run on every token, uncondensed. */
MOE_API moe_status_t moe_layer_fwd_condensed(const moe_dims_t* dims, const void* x,
                                     const void* w_router, const float* bias,
                                     const void* w_gate, const void* w_up, const void* w_down,
                                     const void* wsh_gate, const void* wsh_up,
                                     const void* wsh_down, const void* hyperplanes,
                                     float cos_threshold, float* out, int32_t* topk_ids_out,
                                     float* topk_w_out, int32_t* counts_out, int32_t* offsets_out,
                                     int32_t* perm_out, int32_t* rep_out, void* ws,
                                     size_t ws_bytes, hipStream_t stream);

/* Workspace of moe_layer_bwd: moe_workspace_bytes plus the backward scratch:
 * the sorted token rows; fp32 [T*k, I] and [T*k, d] intermediates (G, U, the
 * SwiGLU gradient and the sorted rows' input gradients; fp32 layers also A,
 * dY and the expert outputs); fp32 [T, n_shared*I_shared] intermediates of
 * the shared experts; and for bf16 layers the transposed weights, the bf16
 * hi/lo parts of the fp32 operands, the per-expert zero-padded transposed
 * operands of the weight-gradient products and split-K partial sums.  About
 * 3.6 GB for 4096 tokens, d = 2048, 64 experts top-6 of I = 1408 and two
 * shared experts.  0 for invalid dims. */
MOE_API size_t moe_backward_workspace_bytes(const moe_dims_t* dims);

/* Backward pass of moe_layer_fwd: given the upstream gradient dout = dL/dout
 * [T,d] fp32, the gradients of the layer output with respect to x, the
 * router weights and bias, and every routed and shared expert's weights.
 * The pages time training runs of MoE layers (the FarSkip-Collective review,
 * "What carries the argument"; the Luffy review, Fig. 8 caption) but do not
 * write the gradients out; they follow from the forward pass by the chain
 * rule with these readings:
 *   - the top-k choice of experts passes no gradient; the kept weights are
 *     the softmax over the kept logits, so token t's logit gradient is
 *     w_j (dw_j - sum_j' w_j' dw_j') on its kept experts, dw_j = dout[t] .
 *     (expert output of slot j);
 *   - dbias = the logit gradient summed over tokens (also when bias is NULL:
 *     the gradient at a zero bias);
 *   - the bf16 rounding of the SwiGLU product passes the gradient unchanged;
 *     dw_down uses the rounded product the forward pass multiplied.
 * The routing, the dispatch and the expert activations are recomputed from
 * the inputs (nothing is carried over from a forward call).  The products
 * run on the bf16 matrix cores with fp32 accumulation, each fp32 operand
 * taken as bf16 parts hi = bf16(v), lo = bf16(v - hi) (|v - hi - lo| <=
 * 2^-16 |v|) (moe_layer_bwd_variant with MOE_VARIANT_BWD_VALU runs them for
 * fp32 layers on the vector ALUs in fp32 instead).
 * All other arithmetic is fp32 (bf16 inputs widened), and each output element
 * is summed in a fixed order: two calls give identical bits.
 *   x, w_router, bias, w_gate, w_up, w_down, wsh_*: as in moe_layer_fwd.
 *   dout: [T,d] fp32, required.
 *   dx [T,d], dw_router [E,d], dw_gate, dw_up [E,I,d], dw_down [E,d,I]:
 *     fp32 outputs, required; dbias [E] fp32 or NULL (not computed);
 *     dwsh_gate, dwsh_up [n_shared,I_shared,d], dwsh_down
 *     [n_shared,d,I_shared]: required iff n_shared > 0.  Experts that receive
 *     no token get zero weight gradients.
 *   ws: ws_bytes >= moe_backward_workspace_bytes(dims).
 * Errors and asynchrony: as moe_layer_fwd (outputs must not overlap any
 * other buffer). */
MOE_API moe_status_t moe_layer_bwd(const moe_dims_t* dims, const void* x, const void* w_router,
                                   const float* bias, const void* w_gate, const void* w_up,
                                   const void* w_down, const void* wsh_gate, const void* wsh_up,
                                   const void* wsh_down, const float* dout, float* dx,
                                   float* dw_router, float* dbias, float* dw_gate, float* dw_up,
                                   float* dw_down, float* dwsh_gate, float* dwsh_up,
                                   float* dwsh_down, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/* moe_layer_bwd through the kernel variant `variant` (a combination of
 * MOE_VARIANT_GLOBAL_LOADS and MOE_VARIANT_BWD_VALU, or 0); every other
 * argument and the result as moe_layer_bwd. */
MOE_API moe_status_t moe_layer_bwd_variant(const moe_dims_t* dims, const void* x,
                                           const void* w_router, const float* bias,
                                           const void* w_gate, const void* w_up,
                                           const void* w_down, const void* wsh_gate,
                                           const void* wsh_up, const void* wsh_down,
                                           const float* dout, float* dx, float* dw_router,
                                           float* dbias, float* dw_gate, float* dw_up,
                                           float* dw_down, float* dwsh_gate, float* dwsh_up,
                                           float* dwsh_down, void* ws, size_t ws_bytes,
                                           int variant, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
