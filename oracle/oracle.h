/*
 * oracle.h — C ABI of the CPU oracle for the dropless MoE feed-forward layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library, and it never reads anything
 * the HIP library produced.
 *
 * Every array is a plain host array, row-major.  Inputs are float (bf16 and
 * fp32 values are both exact in float); floating outputs are double.  The
 * `_f64` entry points accumulate in double, the `_f32` ones in float (the
 * timed full-size CPU baseline).  Functions that take `rows`/`nrows` compute
 * only the listed rows (all rows when `rows` is NULL); the others compute
 * everything.
 *
 * Pages cited (titles as printed; sections as headed on each page):
 *  [P1] "认识 Olmo-core 3" (meetcoding.cn/olmo-core/introduction.html),
 *       核心特点 二 "三种并行 + 三个路由优化" and 三 "MXFP8".
 *  [P2] practitioner article at discosf.com/news/6174547, sections
 *       1.1 (sparse activation: a router picks the top-k experts, only those
 *       k run), 1.2 (forward and backward move every token) and
 *       2.1 (router distribution → top-k → permutation index → per-expert
 *       packets → compute → return along the original path and restore).
 *  [P3] vibecoding.ru news "Обучение MoE ускорилось: Olmo-core 3 ...",
 *       section "Как установить Olmo-core" (dropless MoE needs grouped GEMM).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* logits[t,e] = sum_i x[t,i] * wr[i,e], rounded once to float.  [P2 2.1] */
void oracle_router_logits_f64(const float* x, const float* wr, int T, int d, int E, float* logits);
void oracle_router_logits_f32(const float* x, const float* wr, int T, int d, int E, float* logits);

/* Softmax over E, top-k on the float logits (descending, lower expert index
 * first on equal logits), gates renormalised over the selected experts, the
 * expert histogram, its exclusive scan, and the stable expert-major
 * permutation (row_of[t*k+j] is the row of (t,j) in the expert buffers,
 * src_tk its inverse).  [P2 1.1, 2.1], [P1 二] */
void oracle_route_f64(const float* logits, int T, int E, int k, int32_t* topk_idx, double* gates,
                      int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* src_tk);
void oracle_route_f32(const float* logits, int T, int E, int k, int32_t* topk_idx, double* gates,
                      int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* src_tk);

/* Per-row SwiGLU expert: row r of xp (d wide) belongs to expert e with
 * offsets[e] <= r < offsets[e+1].  g = xp_r*Wg_e, u = xp_r*Wu_e,
 * h = silu(g)*u, yp_r = h*Wd_e.  Wg,Wu are [E,d,F], Wd is [E,F,d].
 * g,u,h are [R,F] and yp is [R,d]; any of g,u,h may be NULL. */
void oracle_expert_fwd_f64(const float* xp, const int32_t* offsets, int E, int R, int d, int F,
                           const float* wg, const float* wu, const float* wd,
                           const int32_t* rows, int nrows,
                           double* g, double* u, double* h, double* yp);
void oracle_expert_fwd_f32(const float* xp, const int32_t* offsets, int E, int R, int d, int F,
                           const float* wg, const float* wu, const float* wd,
                           const int32_t* rows, int nrows,
                           double* g, double* u, double* h, double* yp);

/* Backward of the per-row expert for upstream rows dyp [R,d]: recomputes
 * g,u,h from xp, then dh = dyp_r*Wd_e^T, dg = dh*u*silu'(g), du = dh*silu(g),
 * dxp_r = dg*Wg_e^T + du*Wu_e^T.  dg,du are [R,F], dxp is [R,d]; any may be
 * NULL.  Rows as in oracle_expert_fwd. */
void oracle_expert_dgrad_f64(const float* xp, const float* dyp, const int32_t* offsets, int E, int R,
                             int d, int F, const float* wg, const float* wu, const float* wd,
                             const int32_t* rows, int nrows, double* dg, double* du, double* dxp);
void oracle_expert_dgrad_f32(const float* xp, const float* dyp, const int32_t* offsets, int E, int R,
                             int d, int F, const float* wg, const float* wu, const float* wd,
                             const int32_t* rows, int nrows, double* dg, double* du, double* dxp);

/* Expert weight gradients, each the sum over that expert's rows in row
 * order: dWg_e = xp_e^T dg_e, dWu_e = xp_e^T du_e, dWd_e = h_e^T dyp_e,
 * exactly zero for an expert with no rows.  Outputs [E,d,F],[E,d,F],[E,F,d]. */
void oracle_expert_wgrad_f64(const float* xp, const float* dyp, const int32_t* offsets, int E, int R,
                             int d, int F, const float* wg, const float* wu, const float* wd,
                             double* dwg, double* dwu, double* dwd);
void oracle_expert_wgrad_f32(const float* xp, const float* dyp, const int32_t* offsets, int E, int R,
                             int d, int F, const float* wg, const float* wu, const float* wd,
                             double* dwg, double* dwu, double* dwd);

/* Selected elements of the weight gradients: which = 0 (dWg), 1 (dWu) or
 * 2 (dWd); elem[n] = (e, a, b) indexes dW[e][a][b].  Each element is its own
 * sum over the expert's rows, from the definition above. */
void oracle_expert_wgrad_elems_f64(const float* xp, const float* dyp, const int32_t* offsets, int E,
                                   int R, int d, int F, const float* wg, const float* wu,
                                   const float* wd, int which, const int32_t* elem, int nelem,
                                   double* out);

/* Whole layer, token by token (no expert buffers are built): for every
 * (t,j) with e = topk[t,j] the expert runs on x_t; y_t = sum_j gates[t,j]*Y_tj
 * in slot order.  Ytj [T,k,d] may be NULL.  [P2 2.1] */
void oracle_layer_fwd_f64(const float* x, const int32_t* topk, const double* gates, int T, int d,
                          int E, int k, int F, const float* wg, const float* wu, const float* wd,
                          double* y, double* ytj);
void oracle_layer_fwd_f32(const float* x, const int32_t* topk, const double* gates, int T, int d,
                          int E, int k, int F, const float* wg, const float* wu, const float* wd,
                          double* y, double* ytj);

/* Whole-layer backward for upstream dy [T,d] (renormalised top-k gates,
 * router wr [d,E]): dgates, dlogits at the selected slots, dx (through the
 * experts and through the router), dWg, dWu, dWd and dWr.  [P2 1.2] */
void oracle_layer_bwd_f64(const float* x, const float* wr, const int32_t* topk, const double* gates,
                          const float* dy, int T, int d, int E, int k, int F, const float* wg,
                          const float* wu, const float* wd, double* dgates, double* dlogits_sel,
                          double* dx, double* dwg, double* dwu, double* dwd, double* dwr);

/* ---- MXFP8 (E4M3 elements, 32-element blocks, e8m0 scales) [P1 三] ---- */

/* E4M3 ("FN": bias 7, no infinities, 0x7f/0xff are NaN, max 448) code of
 * v, round to nearest even, saturating to +-448; NaN -> 0x7f. */
uint8_t oracle_e4m3_encode(float v);
/* Exact value of an E4M3 code (NaN codes return NaN). */
float oracle_e4m3_decode(uint8_t c);
/* e8m0 scale code of a block with the given largest magnitude:
 * 0 when amax == 0, else floor(log2 amax) - 8 + 127, clamped to [0, 254]. */
uint8_t oracle_mx_scale_code(float amax);
/* Quantise a [rows, cols] float matrix in 32-element blocks.
 * axis 0: blocks run along each row (cols % 32 == 0); codes [rows,cols],
 *         scales [rows, cols/32].
 * axis 1: blocks run down each column inside each group of rows
 *         (group g = rows offsets[g]..offsets[g+1]; offsets NULL = one group),
 *         the last block of a group zero-padded; codes are [rows, cols] in
 *         place, scales [sum_g ceil(n_g/32), cols] (group-major blocks). */
void oracle_mx_quantize(const float* src, int rows, int cols, int axis, const int32_t* offsets,
                        int groups, uint8_t* codes, uint8_t* scales);

#ifdef __cplusplus
}
#endif
#endif
