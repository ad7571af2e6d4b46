/*
 * moe.h — C ABI of the MI355X (gfx950) dropless MoE feed-forward layer.
 *
 * The layer, as the pages describe it in words:
 *  - a router scores each token against every expert, the top-k experts are
 *    selected and only those k run ([P2] sections 1.1 and 2.1);
 *  - the selection becomes a permutation index and the token rows are packed
 *    per expert ([P2] 2.1), written straight into each expert's input buffer
 *    ("rowwise" expert parallelism, [P1] 核心特点 二);
 *  - routing metadata stays on the GPU so the host never waits on a copy
 *    back ([P1] 二, GPU-resident routing);
 *  - the experts run as one device-scheduled grouped GEMM ([P1] 二,
 *    Grouped GEMM), dropless: no token is dropped when an expert is
 *    overloaded ([P3] "Как установить Olmo-core");
 *  - the results return along the original path and are restored to token
 *    order ([P2] 2.1); forward and backward both move every token ([P2] 1.2);
 *  - MXFP8 is supported for the expert GEMMs ([P1] 三).
 * Pages: [P1] "认识 Olmo-core 3" (meetcoding.cn/olmo-core/introduction.html);
 * [P2] the practitioner article at discosf.com/news/6174547; [P3] vibecoding.ru
 * news "Обучение MoE ускорилось: Olmo-core 3 дал прирост в 2,7 раза"; [P5] the
 * bigchange.ai article on the Olmo-core 3 MoE training stack (its overview
 * names MXFP8 for selected operations).
 *
 * Shapes: T tokens, d = d_model, E experts, k = top-k, F = d_ff, R = T*k rows.
 * Expert i/o is SwiGLU without biases:  y = (silu(x Wg) * (x Wu)) Wd.
 * Layouts (row-major): x [T,d]; W_r [d,E]; Wg, Wu [E,d,F]; Wd [E,F,d];
 * logits [T,E] fp32; topk_idx, row_of [T,k] int32; gates [T,k] fp32;
 * counts [E], offsets [E+1] int32; src_tk [R] int32; expert buffers
 * (xp, g, u, h, yp, ...) are expert-major rows [R, *] with the rows of
 * expert e at offsets[e] .. offsets[e+1]-1, in ascending token order.
 *
 * Conventions for every call:
 *  - Every pointer is a DEVICE pointer unless marked (host).  The caller owns
 *    every buffer, including the workspace registered with
 *    moe_set_workspace; the library keeps no pointer after a call returns
 *    except the registered workspace.
 *  - No call allocates device memory, copies between host and device, or
 *    synchronises: each only validates on the host and enqueues kernels on
 *    the context's stream, so the whole layer can be captured in a HIP graph.
 *    counts/offsets are never read by the host.
 *  - Errors: host-side validation returns MOE_ERR_INVALID_ARGUMENT (null or
 *    misaligned pointers, sizes out of range, two outputs of one call whose
 *    byte ranges overlap) or MOE_ERR_UNSUPPORTED, and never aborts; launch failures return MOE_ERR_HIP.  moe_last_error gives
 *    the text.  Device faults surface asynchronously, as in HIP.
 *  - Limits: 1 <= k <= min(E, 32); E <= 1024; T*k < 2^31; d % 8 == 0 and
 *    F % 8 == 0 (16-byte bf16 rows); data pointers 16-byte aligned.  The bf16
 *    grouped FFN needs d, F % 64 == 0; MXFP8 needs d, F % 128 == 0.
 *  - Preconditions: logits are finite (otherwise routing is unspecified but
 *    memory-safe).  A context is not thread-safe: one context per stream.
 *  - Gradients overwrite their outputs (no accumulation into them).
 *  - Empty batches: T = 0 (R = 0 rows) is valid for every call.  Pointers to
 *    token- or row-sized arrays may then be NULL; weights, counts, offsets
 *    and weight gradients may not.  Routing writes zero counts and offsets,
 *    and every weight gradient (router and experts) is written as zero.
 */
#ifndef MOE_H
#define MOE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_ctx moe_ctx;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_HIP = 4
} moe_status;

/* Element type of activations and weights.  MOE_F32: fp32 data and fp32
 * arithmetic.  MOE_BF16: bf16 data, fp32 accumulation, bf16 outputs.
 * MOE_MXFP8: (grouped FFN only) bf16 data in and out; every GEMM operand is
 * quantised to MXFP8 along its reduction axis (E4M3 elements, 32-element
 * blocks, e8m0 scales, see moe_mx_quantize), fp32 accumulation, bf16 outputs;
 * g and u are bf16 and SwiGLU and its backward run in fp32 on those values,
 * h, dyp, dg and du are quantised again where a GEMM consumes them.  [P1] 三 */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP8 = 2 } moe_dtype;

/* ---------------------------------------------------------------- context */

/* Create a context on `device` that enqueues on `hip_stream` (a hipStream_t,
 * NULL = the default stream).  *out (host) receives the context. */
moe_status moe_create(int device, void* hip_stream, moe_ctx** out);
moe_status moe_destroy(moe_ctx* ctx);
moe_status moe_set_stream(moe_ctx* ctx, void* hip_stream);
/* Static text of a status code. */
const char* moe_status_string(moe_status s);
/* Text of the last error on this context (owned by the context). */
const char* moe_last_error(const moe_ctx* ctx);

/* Device workspace needed by the calls that use it for a layer of this
 * shape: moe_route (per-block expert histograms), moe_permute_bwd with the
 * router term (a transposed copy of W_r), moe_router_wgrad (fp32 partials
 * per 256-row chunk), moe_route_stats and moe_expert_grad_norms (partial
 * sums).  The calls run in stream order,
 * so they share one region.  *bytes is a host output. */
moe_status moe_workspace_size(moe_ctx* ctx, int T, int d, int E, int k, moe_dtype dtype,
                              size_t* bytes);
/* Device workspace of an MXFP8 grouped FFN call (moe_grouped_ffn_fwd/bwd with
 * MOE_MXFP8: the quantised operands); *bytes is a host output.  Register
 * max(this, moe_workspace_size(...)). */
moe_status moe_mx_workspace_size(moe_ctx* ctx, int E, int R, int d, int F, size_t* bytes);
/* Device workspace of moe_grouped_ffn_bwd for this shape; *bytes (host) is 0
 * when the call needs none.  MOE_MXFP8: the quantised operands (as
 * moe_mx_workspace_size).  MOE_BF16: 256 bytes of per-XCD tile ranges for
 * the two weight gradients (planned by the down dgrad from the routed
 * counts, cost-balanced when skewed routing would overload one XCD), then
 * the split-K partials of a weight gradient whose output tiles would leave
 * block slots idle (fewer than two per compute unit, e.g. a shared expert's
 * single group of T rows): each group's rows are cut into up to 8 segments
 * whose exact fp32 partial products are summed in segment order and rounded
 * once.  MOE_F32: 0. */
moe_status moe_ffn_bwd_workspace_size(moe_ctx* ctx, int E, int R, int d, int F, moe_dtype dtype,
                                      size_t* bytes);
/* Register caller-owned device workspace (256-byte aligned). */
moe_status moe_set_workspace(moe_ctx* ctx, void* ws, size_t bytes);

/* ---------------------------------------------------------------- forward */

/* Router scores: logits[t,e] = sum_i x[t,i] * w_router[i,e], fp32
 * accumulation, fp32 output, any E up to 1024 in either dtype (bf16 with
 * E > 16, E % 8 == 0 and d % 64 == 0 runs on the matrix cores; every other
 * shape on the vector ALUs, 64 experts per pass over x).  [P2] 1.1, 2.1. */
moe_status moe_router_logits(moe_ctx* ctx, const void* x, const void* w_router, int T, int d,
                             int E, moe_dtype dtype, float* logits);

/* Routing.  For each token: the k experts with the largest logits, larger
 * logit first and the lower expert index first among equal logits
 * (+0 == -0); gates[t,j] = softmax over the k selected logits (equal to the
 * softmax over all E renormalised over the selection).  Then the expert
 * histogram counts[e], offsets = exclusive scan of counts (offsets[E] = R),
 * and the stable expert-major permutation: row_of[t,j] is the row of (t,j)
 * in the expert buffers, src_tk[row] = t*k + j its inverse.  Rows within an
 * expert are in ascending t.  Needs the registered workspace
 * (moe_workspace_size).  [P2] 2.1 (permutation index), [P1] 二
 * (GPU-resident routing metadata). */
moe_status moe_route(moe_ctx* ctx, const float* logits, int T, int E, int k, int32_t* topk_idx,
                     float* gates, int32_t* counts, int32_t* offsets, int32_t* row_of,
                     int32_t* src_tk);

/* moe_route for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, results (bit for bit) and errors, but no registered
 * workspace is used and nothing is allocated.  Its per-block expert counts
 * live in one static device array of 2^20 int32 (4 MiB), which every GPU the
 * library runs on holds until the process ends; shapes with
 * E * ceil(T / 64) > 2^20 (e.g. T > 524288 at E = 128, T > 65536 at
 * E = 1024) return MOE_ERR_UNSUPPORTED.  All calls on one GPU share that
 * array: calls in one stream are ordered, but calls that overlap in time on
 * one GPU (other streams, other threads) race.  The first call on a device
 * looks up the array's device address (hipGetSymbolAddress). */
moe_status moe_route_noalloc(moe_ctx* ctx, const float* logits, int T, int E, int k,
                             int32_t* topk_idx, float* gates, int32_t* counts, int32_t* offsets,
                             int32_t* row_of, int32_t* src_tk);

/* Rowwise permute: xp[row_of[t,j]] = x[t] for every (t,j); xp is [T*k, d].
 * [P1] 二 (rows written straight into the experts' input buffers). */
moe_status moe_permute(moe_ctx* ctx, const void* x, const int32_t* row_of, int T, int d, int k,
                       moe_dtype dtype, void* xp);

/* Grouped SwiGLU experts over the R expert-major rows, scheduled on the
 * device from `offsets` (no host sync): for the rows of expert e,
 * g = xp Wg[e], u = xp Wu[e], h = silu(g) * u, yp = h Wd[e].  g, u, h
 * ([R,F]) are saved for the backward; yp is [R,d].  An expert with no rows
 * does no work.  With w_down and yp both NULL only g, u, h are computed:
 * the recompute step of a backward that did not keep them (bit-identical to
 * the forward's).  [P1] 二 (grouped GEMM), [P3] (dropless). */
moe_status moe_grouped_ffn_fwd(moe_ctx* ctx, const void* xp, const void* w_gate,
                               const void* w_up, const void* w_down, const int32_t* offsets,
                               int E, int R, int d, int F, moe_dtype dtype, void* g, void* u,
                               void* h, void* yp);

/* Quantise-on-permute for the MXFP8 experts ([P1] 三: MXFP8, with the rows
 * written straight into the experts' buffers, [P1] 二).  Each token row of x
 * (bf16 [T,d], d % 32 == 0) is read once and quantised once along d exactly
 * as moe_mx_quantize axis 0 does, and its codes ([T*k, d] uint8), scale
 * bytes ([T*k, d/32] uint8) and, when xp is non-NULL, the bf16 row itself
 * ([T*k, d]) are written into each of its k rows row_of[t,j].  Equal to
 * moe_permute followed by moe_mx_quantize(axis 0) of xp, byte for byte. */
moe_status moe_permute_mx(moe_ctx* ctx, const void* x, const int32_t* row_of, int T, int d, int k,
                          void* xp, uint8_t* xp_codes, uint8_t* xp_scales);

/* moe_grouped_ffn_fwd with MOE_MXFP8 on rows that are already quantised
 * (moe_permute_mx): the same outputs, bit for bit, without quantising xp
 * again.  Needs the MXFP8 workspace (moe_mx_workspace_size). */
moe_status moe_grouped_ffn_fwd_mxq(moe_ctx* ctx, const uint8_t* xp_codes, const uint8_t* xp_scales,
                                   const void* w_gate, const void* w_up, const void* w_down,
                                   const int32_t* offsets, int E, int R, int d, int F, void* g,
                                   void* u, void* h, void* yp);

/* MXFP8 weight pack ([P1] 三: MXFP8; one quantisation of the expert
 * weights serves the forward and the backward of a step).  Bytes of the pack
 * for E experts of model width d and expert width F (d, F % 128 == 0);
 * *bytes is a host output. */
moe_status moe_mx_weight_pack_size(moe_ctx* ctx, int E, int d, int F, size_t* bytes);

/* Quantise w_gate, w_up ([E,d,F] bf16) and w_down ([E,F,d] bf16) into
 * `pack` (caller-owned device memory, 256-byte aligned, pack_bytes >=
 * moe_mx_weight_pack_size).  Each weight is read once and written in both
 * MX layouts the grouped FFN reads: blocks of 32 along each expert matrix's
 * rows (the forward GEMMs' K; as moe_mx_quantize axis 1 with one group per
 * expert) and along its columns (the data-gradient GEMMs' K; as axis 0).
 * The layout inside the pack is the library's own.  Quantise again after
 * every change of the weights: a pack is not tied to the weights it was
 * made from. */
moe_status moe_mx_quantize_weights(moe_ctx* ctx, const void* w_gate, const void* w_up,
                                   const void* w_down, int E, int d, int F, void* pack,
                                   size_t pack_bytes);

/* moe_grouped_ffn_fwd with MOE_MXFP8, the weights taken from a pack: the
 * same outputs bit for bit, without quantising the weights.  The rows come
 * either as bf16 xp (quantised in the call) or already quantised
 * (xp_codes, xp_scales from moe_permute_mx): give exactly one of xp and
 * xp_codes.  yp NULL: the gate/up GEMM alone (recompute of g, u, h).
 * Needs the MXFP8 workspace (moe_mx_workspace_size). */
moe_status moe_grouped_ffn_fwd_mxp(moe_ctx* ctx, const void* xp, const uint8_t* xp_codes,
                                   const uint8_t* xp_scales, const void* pack, size_t pack_bytes,
                                   const int32_t* offsets, int E, int R, int d, int F, void* g,
                                   void* u, void* h, void* yp);

/* moe_grouped_ffn_bwd with MOE_MXFP8, the weights taken from a pack: the
 * same outputs bit for bit.  Needs the MXFP8 workspace. */
moe_status moe_grouped_ffn_bwd_mxp(moe_ctx* ctx, const void* xp, const void* pack,
                                   size_t pack_bytes, const int32_t* offsets, const void* g,
                                   const void* u, const void* h, const void* dyp, int E, int R,
                                   int d, int F, void* dg, void* du, void* dxp, void* dw_gate,
                                   void* dw_up, void* dw_down);

/* moe_grouped_ffn_bwd_mxp with MXFP8 on the data-gradient GEMMs only (MXFP8
 * for selected operations, [P5] overview; [P1] 三): dh and dxp run
 * on MXFP8 operands exactly as in moe_grouped_ffn_bwd_mxp (dg, du, dxp are
 * the same bytes), while the three weight gradients run on the unquantised
 * bf16 operands (xp, dg, du, h, dyp) with fp32 sums and one bf16 rounding, as
 * MOE_BF16 computes them:
 *   dWd[e] = h_e^T dyp_e;  dWg[e] = xp_e^T dg_e;  dWu[e] = xp_e^T du_e.
 * Only the rowwise layouts of dyp, dg and du are quantised.  Arguments,
 * layouts and errors as moe_grouped_ffn_bwd_mxp; the workspace is
 * moe_mx_workspace_size's (which covers both backward forms). */
moe_status moe_grouped_ffn_bwd_mxp_bf16w(moe_ctx* ctx, const void* xp, const void* pack,
                                         size_t pack_bytes, const int32_t* offsets, const void* g,
                                         const void* u, const void* h, const void* dyp, int E,
                                         int R, int d, int F, void* dg, void* du, void* dxp,
                                         void* dw_gate, void* dw_up, void* dw_down);

/* Gate-weighted unpermute-combine: y[t] = sum_j gates[t,j] * yp[row_of[t,j]],
 * summed in slot order in fp32, rounded once.  [P2] 2.1 (return and
 * restore). */
moe_status moe_combine(moe_ctx* ctx, const void* yp, const float* gates, const int32_t* row_of,
                       int T, int d, int k, moe_dtype dtype, void* y);

/* Shared expert (an expert every token uses, besides its k routed ones;
 * [P1] 四 lists shared experts among the framework's router options): one
 * SwiGLU FFN over all T tokens, ungated, added to the routed output.  Run it
 * with moe_grouped_ffn_fwd on x itself as one group (offsets {0, T}, E = 1)
 * and add its output rows here:
 *   y[t] = sum_j gates[t,j] * yp[row_of[t,j]] + y_shared[t]
 * (slot order, then the shared row; fp32 sums, one rounding).  y_shared is
 * [T,d] in dtype. */
moe_status moe_combine_shared(moe_ctx* ctx, const void* yp, const float* gates,
                              const int32_t* row_of, const void* y_shared, int T, int d, int k,
                              moe_dtype dtype, void* y);

/* --------------------------------------------------------------- backward
 * [P2] 1.2: the backward moves every token again. */

/* dyp[row_of[t,j]] = gates[t,j] * dy[t];  dgates[t,j] = <dy[t], yp[row_of[t,j]]>
 * (fp32). */
moe_status moe_combine_bwd(moe_ctx* ctx, const void* dy, const void* yp, const float* gates,
                           const int32_t* row_of, int T, int d, int k, moe_dtype dtype,
                           void* dyp, float* dgates);

/* Logit gradient at the selected slots of the renormalised softmax gates:
 * dlogits_sel[t,j] = gates[t,j] * (dgates[t,j] - sum_i gates[t,i]*dgates[t,i]).
 * Unselected logits have gradient exactly 0 (not stored). */
moe_status moe_route_bwd(moe_ctx* ctx, const float* gates, const float* dgates, int T, int k,
                         float* dlogits_sel);

/* moe_route_bwd that also writes each value in expert-row order,
 * dl_rows[row_of[t,j]] = dlogits_sel[t,j] (dl_rows [T*k] fp32), the form the
 * folded router term of moe_grouped_ffn_bwd_router reads. */
moe_status moe_route_bwd_rows(moe_ctx* ctx, const float* gates, const float* dgates,
                              const int32_t* row_of, int T, int k, float* dlogits_sel,
                              float* dl_rows);

/* Backward of moe_grouped_ffn_fwd for upstream rows dyp [R,d]:
 *   dh = dyp Wd[e]^T;  dg = dh * u * silu'(g);  du = dh * silu(g)
 *   dxp = dg Wg[e]^T + du Wu[e]^T
 *   dWd[e] = h_e^T dyp_e;  dWg[e] = xp_e^T dg_e;  dWu[e] = xp_e^T du_e
 * dg, du ([R,F]) are outputs too.  Weight gradients of an expert with no
 * rows are exactly zero. */
moe_status moe_grouped_ffn_bwd(moe_ctx* ctx, const void* xp, const void* w_gate,
                               const void* w_up, const void* w_down, const int32_t* offsets,
                               const void* g, const void* u, const void* h, const void* dyp,
                               int E, int R, int d, int F, moe_dtype dtype, void* dg, void* du,
                               void* dxp, void* dw_gate, void* dw_up, void* dw_down);

/* moe_grouped_ffn_bwd with the router's share of the input gradient folded
 * into the gate/up dgrad (MOE_BF16 only).  Row r of expert e holds token t's
 * slot j; dl_rows[r] = dlogits_sel[t,j] (from moe_route_bwd_rows).  Its fp32
 * sum gets dl_rows[r] * w_router[:,e] before the one rounding:
 *   dxp[r] = dg Wg[e]^T + du Wu[e]^T + dlogits_sel[t,j] * W_r[:,e]
 * so moe_permute_bwd without the router term (dlogits_sel, w_router NULL)
 * then gives the whole input gradient of the layer, the router's included
 * (the router scores are x W_r, W_r [d,E] bf16).  Every other output as in
 * moe_grouped_ffn_bwd.  dl_rows [R] fp32 may be NULL only when R == 0;
 * another dtype returns MOE_ERR_INVALID_ARGUMENT. */
moe_status moe_grouped_ffn_bwd_router(moe_ctx* ctx, const void* xp, const void* w_gate,
                                      const void* w_up, const void* w_down,
                                      const int32_t* offsets, const void* g, const void* u,
                                      const void* h, const void* dyp, const float* dl_rows,
                                      const void* w_router, int E, int R, int d, int F,
                                      moe_dtype dtype, void* dg, void* du, void* dxp,
                                      void* dw_gate, void* dw_up, void* dw_down);

/* dx[t] = sum_j dxp[row_of[t,j]]  (+ sum_j dlogits_sel[t,j] * w_router[:, topk_idx[t,j]]
 * when dlogits_sel and w_router are both non-NULL), fp32 accumulation. */
moe_status moe_permute_bwd(moe_ctx* ctx, const void* dxp, const int32_t* row_of,
                           const int32_t* topk_idx, const float* dlogits_sel,
                           const void* w_router, int T, int d, int E, int k, moe_dtype dtype,
                           void* dx);

/* moe_permute_bwd plus the shared expert's input gradient dx_shared [T,d]
 * (from moe_grouped_ffn_bwd over the one all-token group with upstream rows
 * dy itself, since the shared expert is ungated):
 *   dx[t] = sum_j dxp[row_of[t,j]] + dx_shared[t] (+ the router term),
 * in that order, fp32 sums, one rounding. */
moe_status moe_permute_bwd_shared(moe_ctx* ctx, const void* dxp, const int32_t* row_of,
                                  const int32_t* topk_idx, const float* dlogits_sel,
                                  const void* w_router, const void* dx_shared, int T, int d, int E,
                                  int k, moe_dtype dtype, void* dx);

/* Router weight gradient: dw_router[i,e] = sum over the rows r of expert e
 * (ascending) of dlogits_sel[src_tk[r]] * x[src_tk[r] / k, i]; fp32
 * accumulation in a fixed order (rows summed in 256-row chunks, the chunk
 * sums added in order, so a hot expert's rows spread over the chip),
 * stored in dtype.  Needs the registered workspace (moe_workspace_size with
 * this T, d, E, k) when T > 0. */
moe_status moe_router_wgrad(moe_ctx* ctx, const void* x, const float* dlogits_sel,
                            const int32_t* src_tk, const int32_t* offsets, int T, int d, int E,
                            int k, moe_dtype dtype, void* dw_router);

/* ------------------------------------------------- routing statistics
 * [P2] 2.2: a larger expert pool amplifies load imbalance, so frameworks add
 * a load-balancing auxiliary loss; [P2] 4.2: watch the tokens each expert
 * receives (twice the mean flags imbalance); [P2] 4.3: the loss weight
 * starts small (e.g. 0.001); [P2] 5.2: log tokens per expert, mean top-1
 * probability and expert-gradient L2 norms; [P1] 四: the router supports load
 * balancing, and [P1]'s negative results warn that a balance score can
 * improve while the real load worsens, so report counts beside the loss.
 * Every result is deterministic (fixed summation orders). */

/* Per-expert statistics of one routing step and the switch-style balance
 * loss.  With p_t = softmax over all E logits of token t and top-1 expert
 * = the first selected slot (largest logit, lower index on ties):
 *   prob_mean[e]      = (1/T) sum_t p_te                      fp32 [E]
 *   top1_count[e]     = tokens whose top-1 expert is e        int32 [E]
 *   top1_prob_mean[e] = their mean top-1 probability, 0 if none  fp32 [E]
 *   aux_loss[0]       = alpha * E * sum_e (counts[e] / (T k)) * prob_mean[e]
 * (alpha exactly at uniform load and probability).  counts are moe_route's
 * [E] histogram.  Outputs are device arrays (aux_loss one float); T = 0
 * gives zeros.  Needs the registered workspace (moe_workspace_size). */
moe_status moe_route_stats(moe_ctx* ctx, const float* logits, const int32_t* counts, int T, int E,
                           int k, float alpha, float* prob_mean, int32_t* top1_count,
                           float* top1_prob_mean, float* aux_loss);

/* Gradient of dloss * aux_loss with respect to every logit (dense [T,E]
 * fp32, overwritten).  The load fractions counts[e]/(T k) are piecewise
 * constant in the logits, so only the mean probabilities carry gradient:
 *   dlogits[t,e] = dloss * p_te * (a_e - sum_i p_ti a_i),
 *   a_e = alpha * E * counts[e] / (T^2 k).
 * Every row sums to zero.  The selected-slot gradient of the gates
 * (moe_route_bwd) is separate; the two add. */
moe_status moe_aux_loss_bwd(moe_ctx* ctx, const float* logits, const int32_t* counts, int T, int E,
                            int k, float alpha, float dloss, float* dlogits);

/* The balance loss trains the router ([P1] 四: the router balances load;
 * [P2] 2.2, 4.3): its logit gradient (moe_aux_loss_bwd, dense [T,E]) flows
 * through logits = x W_r into the layer's input and router gradients.  This
 * call ADDS that share in place:
 *   dx[t,i]        += sum_e dlogits[t,e] * w_router[i,e]
 *   dw_router[i,e] += sum_t x[t,i] * dlogits[t,e]   (tokens in 512-token
 *                     chunks, the chunk sums added in chunk order)
 * fp32 sums in a fixed order, each element rounded once to dtype (MOE_F32
 * or MOE_BF16; x, dx [T,d], w_router, dw_router [d,E] in dtype).  MOE_BF16
 * with d and E multiples of 64 runs on the matrix cores with dlogits rounded
 * to bf16 as the operand; every other case uses fp32 multiply-adds.
 * Deterministic.  Call it after
 * moe_permute_bwd and moe_router_wgrad have written dx and dw_router.  Needs
 * the registered workspace (moe_workspace_size with this T, d, E) when
 * T > 0; T <= 2097120. */
moe_status moe_router_dense_bwd(moe_ctx* ctx, const void* x, const void* w_router,
                                const float* dlogits, int T, int d, int E, moe_dtype dtype,
                                void* dx, void* dw_router);

/* L2 (Frobenius) norm of each expert's weight-gradient matrix: dw is
 * [E, rows, cols] in dtype (MOE_BF16 or MOE_F32; cols % 8 == 0 for bf16,
 * % 4 for fp32), norms[e] = sqrt(sum of squares) with fp32 accumulation in
 * a fixed order.  Works for dWg, dWu ([E,d,F]) and dWd ([E,F,d]).  Needs
 * the registered workspace (moe_workspace_size with this E). */
moe_status moe_expert_grad_norms(moe_ctx* ctx, const void* dw, int E, int rows, int cols,
                                 moe_dtype dtype, float* norms);

/* ----------------------------------------------------------------- MXFP8
 * MX quantisation of a bf16 [rows, cols] matrix ([P1] 三: MXFP8).  Blocks of
 * 32 elements share the scale byte s + 127 with s = floor(log2(max |v|)) - 8
 * clamped to [-127, 127] (byte 0 for an all-zero block); each element is the
 * E4M3 value nearest to v / 2^s (ties to even, saturating at +-448, sign
 * kept, NaN -> 0x7f).
 *  axis 0: blocks along each row (cols % 32 == 0): codes [rows, cols],
 *          scales [rows, cols/32]; kpad_ld is ignored.
 *  axis 1: blocks of 32 consecutive rows of one column, restarting at every
 *          group of rows (group_offsets[groups+1] on the device; NULL means
 *          one group of all rows), the last block of a group zero-padded.
 *          Output transposed and K-contiguous: codes [cols, kpad_ld] and
 *          scales [cols, kpad_ld/32]; group g starts at K position
 *          sum_{g'<g} roundup(n_g', 128) and its positions up to
 *          roundup(n_g, 128) are written (padding as zero codes and zero
 *          scales).  kpad_ld % 128 == 0 and kpad_ld >= rows + 127*groups.
 * codes/scales are caller-owned device buffers. */
moe_status moe_mx_quantize(moe_ctx* ctx, const void* src_bf16, int rows, int cols, int axis,
                           const int32_t* group_offsets, int groups, uint8_t* codes,
                           uint8_t* scales_e8m0, int kpad_ld);

/* Both layouts of moe_mx_quantize from one read of src: codes_cols and
 * scales_cols exactly as axis 1 writes them (same group_offsets, groups,
 * kpad_ld rules), codes_rows and scales_rows exactly as axis 0 writes them
 * for the rows the groups cover (group_offsets[0] .. group_offsets[groups],
 * all rows when group_offsets is NULL).  ([P1] 三: an operand that both a
 * data-gradient GEMM and a weight-gradient GEMM read is quantised along
 * each one's K.) */
moe_status moe_mx_quantize_both(moe_ctx* ctx, const void* src_bf16, int rows, int cols,
                                const int32_t* group_offsets, int groups, uint8_t* codes_cols,
                                uint8_t* scales_cols, int kpad_ld, uint8_t* codes_rows,
                                uint8_t* scales_rows);

/* -------------------------------------------------------------- profiling
 * Per-kernel timing with HIP events recorded on the context's stream around
 * each kernel launch, for measurement runs (off by default; costs two event
 * records per launch when on).  Kernel ids: */
typedef enum {
  MOE_K_ROUTER_LOGITS = 0, /* router scores (VALU or MFMA) */
  MOE_K_TOPK,              /* softmax top-k + block histograms */
  MOE_K_SCAN,              /* per-expert block scans */
  MOE_K_RANK,              /* offsets + stable ranks -> row_of, src_tk */
  MOE_K_PERMUTE,
  MOE_K_GEMM_UP,           /* gate/up grouped GEMM + SwiGLU */
  MOE_K_GEMM_DOWN,         /* down grouped GEMM */
  MOE_K_COMBINE,
  MOE_K_COMBINE_BWD,
  MOE_K_ROUTE_BWD,
  MOE_K_GEMM_DGRAD_DOWN,   /* down dgrad + SwiGLU backward */
  MOE_K_GEMM_WGRAD_DOWN,
  MOE_K_GEMM_DGRAD_UP,
  MOE_K_GEMM_WGRAD_UP,
  MOE_K_PERMUTE_BWD,       /* incl. the W_r transpose when the router term is on */
  MOE_K_ROUTER_WGRAD,
  MOE_K_MX_QUANT,          /* MXFP8 quantisation (moe_mx_quantize and the MX FFN) */
  MOE_K_ROUTE_STATS,       /* routing statistics + balance loss */
  MOE_K_AUX_BWD,           /* balance-loss logit gradient */
  MOE_K_GRAD_NORMS,        /* per-expert weight-gradient norms */
  MOE_K_ROUTER_DENSE_BWD,  /* balance-loss gradient through the router */
  MOE_K_COUNT
} moe_kernel_id;

/* Turn event timing on (clears previous records) or off (keeps them for
 * moe_profile_query). */
moe_status moe_profile_enable(moe_ctx* ctx, int on);
/* Launch count and summed duration (ms) of one kernel id since the last
 * enable.  Waits for the recorded events (host synchronisation: measurement
 * only).  launches and total_ms are host outputs. */
moe_status moe_profile_query(moe_ctx* ctx, int kernel_id, int* launches, double* total_ms);
/* Static name of a kernel id. */
const char* moe_kernel_name(int kernel_id);

/* Measurement probe (not a step of the layer): the sustained bf16
 * matrix-core rate at the clock the chip holds under pure MFMA load, for
 * quoting the grouped GEMMs beside a measured ceiling as well as the
 * published peak.  Launches `blocks` blocks of 256 threads; every wave runs
 * `iters` rounds of four independent v_mfma_f32_32x32x16_bf16 (32768 FLOPs
 * each) on register operands whose elements are a and b rounded to bf16,
 * then writes one float per thread to the device buffer sink (blocks*256
 * floats, caller-owned): 1024*a*b*iters, exact while below 2^24.  FLOPs per
 * launch = blocks * 4 * iters * 4 * 32768.  MOE_ERR_INVALID_ARGUMENT for blocks
 * outside [1, 2^20], iters < 1 or a null sink. */
moe_status moe_mfma_peak_probe(moe_ctx* ctx, int blocks, int iters, float a, float b, float* sink);

#ifdef __cplusplus
}
#endif
#endif
