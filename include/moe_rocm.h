/*
 * moe_rocm.h -- C ABI of one GPU's routed mixture-of-experts expert layer on
 * MI355X (gfx950).
 *
 * The layer (KOSMOS: Self-scheduling Persistent Kernels for Communication-
 * Compute Overlap, section 3.3.1 "Forward Pass", section 3.3.2 "Backward
 * Pass"; OLMo-core MoE, Appendix A: Kernel Interfaces and Profiling Reference,
 * A.1-A.5):
 *
 *   router logits -> softmax + top-K -> route map (dst_rows[N,K], route id
 *   t*K+k, -1 = invalid) -> dispatch of token rows into expert-contiguous rows
 *   -> grouped GEMM gate/up with SwiGLU -> grouped GEMM down -> combine
 *   (probability-weighted fold [N,K,D] -> [N,D]); plus the adjoint backward and
 *   an MXFP8 variant (E4M3 data, one E8M0 scale per 32 elements).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership: the caller allocates every buffer (device memory unless stated)
 *   and the workspace; the library allocates nothing and keeps no state.
 * Execution: every call only enqueues kernels on `stream` (a hipStream_t;
 *   NULL = the default stream) and returns; nothing synchronises the host and
 *   no device value is copied to the host.  Results are bitwise identical run
 *   to run.
 * Layout: row-major everywhere.  bf16 tensors are 16-bit patterns.  Expert
 *   weights are stored output-major, [E][n_out][k_in] (the contraction
 *   dimension contiguous): W_gate and W_up [E][H][D], W_down [E][D][H].
 *   MXFP8 data are OCP E4M3FN bytes; scales are E8M0 bytes (value 2^(s-127)),
 *   one per 32 consecutive elements along the contraction dimension, stored
 *   row-major [rows][cols/32] (OLMo-core Appendix A, A.4).
 * Pointers: every tensor pointer must be 16-byte aligned (MOE_ERR_ALIGN).
 * Errors: functions return a status code below; on any non-zero status
 *   nothing has been enqueued, except MOE_ERR_HIP, which reports a failed
 *   launch (see moe_last_hip_error).  Device-side bad values never trap.
 */
#ifndef MOE_ROCM_H
#define MOE_ROCM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define MOE_OK 0
#define MOE_ERR_NULL (-1)        /* a required pointer is NULL                    */
#define MOE_ERR_SHAPE (-2)       /* N<0, K<1, K>E, E + n_shared > 1024, D or H not a
                                    multiple of 8 (32 for MXFP8), align not 1/32,
                                    N*K >= 2^31                                     */
#define MOE_ERR_DTYPE (-3)       /* unknown dtype or epilogue                      */
#define MOE_ERR_WORKSPACE (-4)   /* workspace smaller than moe_workspace_size      */
#define MOE_ERR_ALIGN (-5)       /* a pointer is not 16-byte aligned               */
#define MOE_ERR_UNSUPPORTED (-6) /* valid request this build does not implement    */
#define MOE_ERR_HIP (-7)         /* a kernel launch failed                         */

/* ---- device status word ---------------------------------------------------
 * moe_layer_fwd writes these bits into the optional device int32
 * moe_layer_saved.status (0 = nothing to report).  They describe device-side
 * events that no host check can see; the call itself has returned MOE_OK. */
#define MOE_STATUS_WAIT_EXPIRED 1   /* MOE_SCHED_READY / MOE_SCHED_SINGLE: a bounded
                                       readiness or barrier wait gave up; the items
                                       (or, at a barrier, the rest of the launch) that
                                       waited were skipped, so the outputs are
                                       incomplete                                    */
#define MOE_STATUS_NO_FINITE_LOGIT 2 /* a token had fewer than K non-NaN logits; each
                                       slot left without one has topk_idx = -1,
                                       probability 0 and no row (an invalid route)   */

/* ---- enums ------------------------------------------------------------- */
#define MOE_BF16 0
#define MOE_MXFP8 1

#define MOE_EPI_NONE 0        /* store the product as bf16                       */
#define MOE_EPI_SWIGLU 1      /* forward, two weights: G, U and H = silu(G)*U      */
#define MOE_EPI_SWIGLU_BWD 2  /* backward dgrad of the down GEMM: dG, dU from dH   */

/* workspace query operations */
#define MOE_OP_ROUTE 1
#define MOE_OP_GEMM 2
#define MOE_OP_LAYER_FWD 3
#define MOE_OP_LAYER_BWD 4
#define MOE_OP_ROUTER 5
#define MOE_OP_LAYER_BWD_MXFP8 6
#define MOE_OP_LAYER_BWD_MXFP8_NATIVE 7   /* MXFP8 backward with mx_wgrad = 1 */

/* ---- shapes -------------------------------------------------------------
 * N tokens, D model width, E experts, K routes per token, H expert (SwiGLU)
 * width; align = 1 (bf16) or 32 (MXFP8: each expert's rows padded to a
 * multiple of 32, KOSMOS section 3.3.1 step 3); renorm = 1 divides the K
 * selected probabilities by their sum. */
typedef struct moe_dims {
  int64_t N, D, E, K, H;
  int32_t align;
  int32_t renorm;
  /* Group-limited top-K (KOSMOS section 3.3.1 step 1), on when n_group > 1:
   * the E experts form n_group contiguous groups (E % n_group == 0,
   * n_group <= 64); a group scores the sum of its two largest routing
   * probabilities; the topk_group best groups (ties to the lower group) are
   * kept and top-K runs over their experts (1 <= topk_group <= n_group,
   * topk_group * E / n_group >= K).  0 or 1: plain top-K. */
  int32_t n_group;
  int32_t topk_group;
  /* Shared expert (KOSMOS Appendix A, Table A.1: in the same launch as the
   * routed experts), 0 or 1.  In the layer calls the expert weights then hold
   * E + 1 experts, the shared one last; it sees every token with weight 1.
   * moe_route appends counts[E] = N and offsets[E+1] (its segment, N rows
   * rounded up to align, after the routed ones; so counts/offsets hold E + 1 /
   * E + 2 entries), and rows_cap grows by N + align - 1.  moe_dispatch,
   * moe_combine and moe_combine_bwd reject it (MOE_ERR_UNSUPPORTED), as do
   * the MOE_SCHED_READY and MOE_SCHED_SINGLE layers. */
  int32_t n_shared;
  int32_t reserved;     /* 0 */
} moe_dims;

/* Rows of every expert-contiguous buffer: N*K + E*(align-1), plus
 * N + align - 1 with a shared expert.  No routing can need more, so these
 * buffers never overflow. */
int64_t moe_rows_cap(const moe_dims* d);

/* Bytes of workspace an operation needs (0 if none).  For MOE_OP_GEMM only
 * d->E and moe_rows_cap(d) matter. */
size_t moe_workspace_size(int op, const moe_dims* d);

const char* moe_status_string(int status);
/* hipError_t of the last failed launch in this process (0 if none). */
int moe_last_hip_error(void);

/* ---- router ------------------------------------------------------------
 * logits[t,e] = sum_d x[t,d] * w_r[e,d] (fp32 accumulate) + bias[e].
 * (KOSMOS section 3.3.1 step 1: router logits X W_r^T in FP32 tiles.)
 * x bf16 [N][D]; w_r bf16 [E][D]; bias fp32 [E] or NULL; logits fp32 [N][E].
 * ws: moe_workspace_size(MOE_OP_ROUTER) bytes (may be 0; ws may then be NULL):
 * the contraction is split into fixed ranges whose fp32 partial products are
 * added there in a fixed order. */
int moe_router_logits(const void* x, const void* w_r, const float* bias, const moe_dims* d,
                      float* logits, void* ws, size_t ws_bytes, void* stream);

/* ---- route -------------------------------------------------------------
 * Softmax and top-K of each token, then the route map (KOSMOS section 3.3.1
 * steps 1-2 "Route" and "Plan": score, top-k, dispatch weights, stable
 * counting sort into per-expert lists; OLMo-core Appendix A, A.2-A.3: route
 * tensors dst_rows[N,K], route id token_row*top_k + k, negative = invalid).
 *   topk_idx  int32 [N][K]  experts by descending logit, ties to the lower index
 *   topk_prob fp32  [N][K]  softmax probability (renormalised if d->renorm)
 *   counts    int32 [E]     valid routes per expert
 *   offsets   int32 [E+1]   first row of each expert's segment (segments are
 *                           counts rounded up to d->align; offsets[E] = total)
 *   dst_rows  int32 [N][K]  row of each route, -1 if invalid
 *   row_route int32 [rows_cap] route id held by each row, -1 for padding/unused
 * drop: u8 [N][K] or NULL; a non-zero entry marks that route invalid (it keeps
 * its topk_idx/topk_prob but gets no row).  ws: moe_workspace_size(MOE_OP_ROUTE).
 * NaN logits never win a slot; a slot left with no candidate (fewer than K
 * non-NaN logits) gets topk_idx -1, probability 0 and no row. */
int moe_route(const float* logits, const uint8_t* drop, const moe_dims* d, int32_t* topk_idx,
              float* topk_prob, int32_t* counts, int32_t* offsets, int32_t* dst_rows,
              int32_t* row_route, void* ws, size_t ws_bytes, void* stream);

/* ---- dispatch ----------------------------------------------------------
 * Row permute into expert-contiguous rows (OLMo-core Appendix A, A.2-A.3:
 * rowwise dispatch PUT per route; KOSMOS section 3.3.1 step 3):
 *   out_dtype MOE_BF16:  xd[dst_rows[t,k]] = x[t]            (weight == NULL)
 *                        xd[dst_rows[t,k]] = bf16(w[t,k]*x[t]) (fp32 product)
 *   out_dtype MOE_MXFP8: each token row quantized once along D, its bytes and
 *                        scales written to all its rows (weight must be NULL).
 * Padding rows inside a segment (align > 1) are written as zeros (q = 0,
 * s = 0); counts/offsets are needed only then.  Rows at or beyond offsets[E]
 * are left untouched.  x bf16 [N][D]; xd bf16 [rows_cap][D] or u8
 * [rows_cap][D]; xd_scales u8 [rows_cap][D/32] (MXFP8 only). */
int moe_dispatch(const void* x, const int32_t* dst_rows, const float* weight,
                 const int32_t* counts, const int32_t* offsets, const moe_dims* d, int out_dtype,
                 void* xd, uint8_t* xd_scales, void* stream);

/* ---- combine -----------------------------------------------------------
 * Fold of each token's K rows (KOSMOS section 3.3.1 step 5; OLMo-core
 * Appendix A, A.2 rowwise_combine_get):
 *   out[t] = bf16( sum_{k ascending, dst_rows[t,k] >= 0} w[t,k] * y[dst_rows[t,k]] )
 * with an fp32 accumulator (fmaf, fixed k order); weight NULL means 1 (the
 * dispatch backward).  y bf16 [rows_cap][D]; out bf16 [N][D]. */
int moe_combine(const void* y, const int32_t* dst_rows, const float* weight, const moe_dims* d,
                void* out, void* stream);

/* ---- combine backward --------------------------------------------------
 * Adjoint of the weighted combine plus the route-weight gradient (KOSMOS
 * section 3.3.2: router-weighted dY dispatch, dw_j = <dY, Y_j>; OLMo-core
 * Appendix A, A.1: combine backward is a weighted dispatch):
 *   dyd[dst_rows[t,k]] = bf16(w[t,k] * dout[t])          (fp32 product)
 *   dprob[t,k] = sum_d dout[t,d] * y[dst_rows[t,k],d]    (fp32; 0 if invalid)
 * dprob may be NULL. */
int moe_combine_bwd(const void* dout, const int32_t* dst_rows, const float* weight, const void* y,
                    const moe_dims* d, void* dyd, float* dprob, void* stream);

/* ---- MXFP8 quantization --------------------------------------------------
 * Row-wise blocks of 32 along cols (KOSMOS section 2.2; OLMo-core Appendix A,
 * A.4-A.5): s = clamp(floor(log2 amax) - 8, -127, 127) + 127 (0 if amax = 0),
 * q = E4M3FN(v * 2^-(s-127)) rounded to nearest even, saturated to +-448.
 * src bf16 [rows][cols]; q u8 [rows][cols]; scales u8 [rows][cols/32]. */
int moe_quantize_mxfp8(const void* src, int64_t rows, int64_t cols, uint8_t* q, uint8_t* scales,
                       void* stream);

/* Column-wise blocks with transpose, the same element and scale rules: the
 * copy of a matrix for the product that contracts over its other dimension,
 * quantized from the bf16 source (KOSMOS section 2.2: both orientations come
 * from the high-precision tensor; OLMo-core Appendix A, A.13: the right-hand
 * operand prequantized for dgrad).
 *   src bf16 [batch][rows][cols]  ->  q[b][c][col0 + r]  (row stride ld),
 *   each block = 32 consecutive r of one column c;
 *   scales[b][c][(col0 + r) / 32]  (row stride ld / 32).
 * Only columns col0 .. col0 + rows - 1 of each q row are written, so two calls
 * with col0 = 0 and col0 = rows fill [A^T | B^T].  rows % 32, cols % 8,
 * ld % 32 and col0 % 32 must be 0 and col0 + rows <= ld (else MOE_ERR_SHAPE);
 * src and q 16-byte aligned (else MOE_ERR_ALIGN). */
int moe_quantize_mxfp8_cols(const void* src, int64_t batch, int64_t rows, int64_t cols, int64_t ld,
                            int64_t col0, uint8_t* q, uint8_t* scales, void* stream);

/* ---- SwiGLU ------------------------------------------------------------
 * h = bf16(silu(g) * u) from bf16 g, u [rows][n] (KOSMOS section 3.3.1 step 3
 * epilogue).  out_dtype MOE_MXFP8 also quantizes h row-wise into h_q/h_scales
 * (h may then be NULL). */
int moe_swiglu(const void* g, const void* u, int64_t rows, int64_t n, int out_dtype, void* h,
               uint8_t* h_q, uint8_t* h_scales, void* stream);

/* ---- grouped GEMM, forward ----------------------------------------------
 * For each expert e, rows i in [offsets[e], offsets[e+1]):
 *   c0[i][n] = sum_k a[i][k] * b0[e][n][k]          (fp32 accumulate, bf16 out)
 * MOE_EPI_SWIGLU (two weights): c0 = G (with b0), c1 = U (with b1) and
 *   act = bf16(silu(G)*U); act_q/act_scales (optional) receive act quantized
 *   to MXFP8 along n.
 * dtype MOE_MXFP8: a, b0, b1 are E4M3 bytes with E8M0 scales along k and the
 *   product is eq. 87 of OLMo-core Appendix A, A.5 (block-scaled MMA).
 * Rows at or beyond offsets[E] are not touched.  (OLMo-core Appendix A,
 * A.13 grouped_mm with caller-provided outputs; KOSMOS section 3.3.1 steps
 * 3-4.)  ws: moe_workspace_size(MOE_OP_GEMM). */
typedef struct moe_gemm_fwd_args {
  int32_t dtype;
  int32_t epilogue;
  int64_t E, rows_cap, k_dim, n_dim;
  const int32_t* offsets;   /* [E+1] device */
  const void* a;            /* [rows_cap][k_dim] */
  const uint8_t* a_scales;  /* MXFP8: [rows_cap][k_dim/32] */
  const void* b0;           /* [E][n_dim][k_dim] */
  const uint8_t* b0_scales; /* MXFP8: [E][n_dim][k_dim/32] */
  const void* b1;           /* SWIGLU: second weight, like b0 */
  const uint8_t* b1_scales;
  void* c0;                 /* bf16 [rows_cap][n_dim] */
  void* c1;                 /* SWIGLU: bf16 [rows_cap][n_dim] */
  void* act;                /* SWIGLU: bf16 [rows_cap][n_dim]; may be NULL for MXFP8
                               when act_q is given (H then only stored quantized) */
  uint8_t* act_q;           /* optional: u8 [rows_cap][n_dim] */
  uint8_t* act_scales;      /* optional: u8 [rows_cap][n_dim/32] */
} moe_gemm_fwd_args;
int moe_grouped_gemm_fwd(const moe_gemm_fwd_args* g, void* ws, size_t ws_bytes, void* stream);

/* ---- grouped GEMM, backward ---------------------------------------------
 * Gradients of the forward product c[i][n] = sum_k a[i][k] b[e][n][k]
 * (KOSMOS section 3.3.2: dgrad2 with the SwiGLU backward in its epilogue,
 * wgrad2, dgrad1, wgrad1; OLMo-core Appendix A, A.1 adjoint sequence):
 *   dgrad (da != NULL or dg != NULL):
 *     da[i][k] = sum_n dc0[i][n] b0[e][n][k] (+ sum_n dc1[i][n] b1[e][n][k]
 *                when dc1 != NULL; one fp32 sum)            bf16 [rows_cap][k_dim]
 *     MOE_EPI_SWIGLU_BWD: the sum is dH and, with the saved bf16 g, u
 *     [rows_cap][k_dim], s = sigmoid(g):  dg = bf16(dH*u*s*(1 + g*(1-s))),
 *     du = bf16(dH*g*s) are written instead of da.
 *   wgrad (db0 != NULL):
 *     db0[e][n][k] = sum_{i in e, ascending} dc0[i][n] a[i][k]   bf16 [E][n_dim][k_dim]
 *     db1 likewise with dc1 (when db1 != NULL).  Experts with no rows get 0.
 * Only dtype MOE_BF16. */
typedef struct moe_gemm_bwd_args {
  int32_t dtype;
  int32_t epilogue;
  int64_t E, rows_cap, k_dim, n_dim;
  const int32_t* offsets;   /* [E+1] device */
  const void* a;            /* forward input [rows_cap][k_dim] (wgrad) */
  const void* b0;           /* forward weight [E][n_dim][k_dim] (dgrad) */
  const void* b1;
  const void* dc0;          /* upstream gradient [rows_cap][n_dim] */
  const void* dc1;
  void* da;                 /* [rows_cap][k_dim] */
  const void* g;            /* SWIGLU_BWD: saved pre-activations [rows_cap][k_dim] */
  const void* u;
  void* dg;
  void* du;
  void* db0;                /* [E][n_dim][k_dim] */
  void* db1;
} moe_gemm_bwd_args;
int moe_grouped_gemm_bwd(const moe_gemm_bwd_args* g, void* ws, size_t ws_bytes, void* stream);

/* ---- whole layer ----------------------------------------------------------
 * Forward: router logits -> route -> dispatch -> GEMM1 (gate/up, SwiGLU) ->
 * GEMM2 (down) -> weighted combine, writing every tensor the backward needs
 * into `saved` (OLMo-core Appendix A, A.1 fused routed-expert node and A.14
 * saved tensors; KOSMOS section 3.3.1 steps 1-5).  For MXFP8 the dispatch
 * quantizes (xd_q/xd_s), GEMM1 is block-scaled, H is quantized (h_q/h_s), and
 * GEMM2 is block-scaled; the combine is bf16.  The MXFP8 forward stores H
 * only quantized: saved->h is ignored there and may be NULL.
 * Backward: combine-bwd and dprob -> down dgrad with the SwiGLU
 * backward -> down wgrad -> gate/up dgrad (one sum) -> gate/up wgrad ->
 * dispatch-bwd (KOSMOS section 3.3.2).  The intermediates dY_d, dG, dU, dX_d
 * live in the workspace (moe_workspace_size(MOE_OP_LAYER_BWD)).
 * MXFP8 backward (workspace MOE_OP_LAYER_BWD_MXFP8): dY_d is quantized
 * row-wise along D from its bf16 values; the down dgrad is block-scaled with
 * wdt_q, its epilogue stores dG, dU (bf16) and [dG | dU] quantized along 2H;
 * the gate/up dgrad is one block-scaled product with wgut_q over 2H; the
 * weight gradients are bf16 products of the bf16 dY_d, dG, dU with the
 * saved activations dequantized from xd_q and h_q (OLMo-core Appendix A,
 * A.13: dgrad on the scaled grouped GEMM, wgrad in bf16 on dequantized
 * operands).  It reads the saved xd_q/xd_s, g, u, h_q/h_s, y and no bf16
 * expert weights; it needs D % 128 == 0 and H % 64 == 0 (else MOE_ERR_SHAPE).
 * With saved->h_q NULL (SwiGLU-recompute mode, OLMo-core Appendix A, A.14:
 * H is rebuilt in the backward instead of being saved) the down weight
 * gradient takes H = bf16(silu(G) U) recomputed from the saved bf16 G and U
 * instead of the dequantized h_q; h_s is then ignored.
 * An empty batch (N = 0) is accepted under every schedule: the forward writes
 * counts and offsets (all 0), row_route (every row -1) and an aux loss of 0;
 * the backward writes every weight gradient as 0 (and db_r when given).
 * Buffers that then hold no element (of N tokens, or of rows_cap rows) may be
 * NULL. */
#define MOE_SCHED_STAGED 0  /* dispatch, GEMM1, GEMM2: one persistent launch each  */
#define MOE_SCHED_READY 1   /* dispatch, GEMM1 and GEMM2 in one persistent
                               launch: GEMM1 tiles (in the staged launch's queue
                               order) gated on the dispatch, GEMM2 tiles gated on
                               their GEMM1 row blocks, so GEMM2 starts while
                               GEMM1's last tiles run.  bf16: align 1,
                               D % 64 == 0 and H % 64 == 0.  MXFP8 (the dispatch
                               quantizes and zeroes the padding rows, GEMM1
                               stores H quantized): D % 128 == 0,
                               H % 128 == 0.  MOE_ERR_UNSUPPORTED for a shared
                               expert or shapes off these rules                 */
/* MOE_SCHED_SINGLE (KOSMOS section 3.3, Figure 6: one launch from route to
 * fold): the whole bf16 layer forward in one persistent launch, after a
 * one-workgroup reset of its barrier words.  Its workgroups (one per CU) run
 * the router tiles, then the logits, softmax and top-K per chunk of tokens,
 * the histogram scan and plans (one workgroup), the scatter, each step ended
 * by a grid barrier, then the MOE_SCHED_READY queue (dispatch, GEMM1 after
 * it, GEMM2 gated on GEMM1 row blocks) followed by the fold, which
 * waits until every workgroup has stored its GEMM2 tiles.  Every output is
 * bitwise the staged forward's.  bf16 only, under the bf16 rules of
 * MOE_SCHED_READY and also the tiled router (D % 64 == 0, 16 <= E <= 512),
 * K <= 32, no grouped top-K and no aux loss; else MOE_ERR_UNSUPPORTED.  Workspace MOE_OP_LAYER_FWD.
 * moe_layer_bwd with MOE_SCHED_SINGLE (KOSMOS section 3.3.2) runs the whole
 * bf16 backward in one persistent launch (after the same kind of reset):
 * the combine backward and the GEMM plans; the down dgrad (SwiGLU backward)
 * and wgrad queues and the router backward blocks; the gate/up dgrad, the
 * gate and up wgrads and the router's dX_r and dW_r; then the router's
 * reductions and the fold, phases separated by grid barriers.  Every
 * gradient is bitwise the staged backward's.  It needs the saved H (no
 * recompute), routed experts only, E <= 512 and the persistent GEMMs' shape
 * rules (with the router backward, E % 64 == 0: dX_r contracts over E in
 * whole steps); else MOE_ERR_UNSUPPORTED.  An expired barrier wait is or-ed into
 * saved->status (MOE_STATUS_WAIT_EXPIRED).  MOE_SCHED_READY backward calls
 * run staged. */
#define MOE_SCHED_SINGLE 2

typedef struct moe_layer_args {
  moe_dims dims;
  int32_t dtype;
  int32_t sched;        /* MOE_SCHED_STAGED, _READY (forward) or _SINGLE        */
  const void* x;        /* bf16 [N][D] */
  const void* w_r;      /* bf16 [E][D] */
  const float* bias;    /* fp32 [E] or NULL */
  const uint8_t* drop;  /* u8 [N][K] or NULL */
  const void* w_gate;   /* bf16 [E][H][D] */
  const void* w_up;     /* bf16 [E][H][D] */
  const void* w_down;   /* bf16 [E][D][H] */
  const uint8_t* wg_q;  /* MXFP8 pre-quantized weights and scales */
  const uint8_t* wg_s;
  const uint8_t* wu_q;
  const uint8_t* wu_s;
  const uint8_t* wd_q;
  const uint8_t* wd_s;
  /* Aux loss (KOSMOS section 3.3.1 step 1: the routing step's aux-loss
   * inputs, reduced once): aux = aux_alpha * E * sum_e f_e P_e with f_e the
   * share of valid routes to e and P_e the mean routing probability of e.
   * Computed into saved->aux when aux_alpha != 0 and saved->aux != NULL. */
  float aux_alpha;
  /* MXFP8 backward: the weight copies of the data gradients, quantized from
   * the bf16 weights along their other dimension (moe_quantize_mxfp8_cols):
   * wdt_q [E][H][D] = W_down^T along D, scales [E][H][D/32];
   * wgut_q [E][D][2H] = [W_gate^T | W_up^T] along H, scales [E][D][2H/32]. */
  const uint8_t* wdt_q;
  const uint8_t* wdt_s;
  const uint8_t* wgut_q;
  const uint8_t* wgut_s;
  /* Testing the status word only; 0 in normal use.  A positive value makes a
   * MOE_SCHED_READY or MOE_SCHED_SINGLE forward withhold its readiness flags
   * (and barrier arrivals) and give up every bounded wait after this many
   * polls, so that each wait expires, the waiting items are skipped, every
   * kernel exits normally and MOE_STATUS_WAIT_EXPIRED is reported.  Ignored
   * by the staged schedule. */
  int32_t ready_test_polls;
  /* MXFP8 backward only: 0 = weight gradients as bf16 products on the
   * dequantized activations (OLMo-core Appendix A, A.13); 1 = native
   * block-scaled weight gradients (A.15) on column-wise MXFP8 copies of dY_d,
   * H, dG, dU and X_d, each quantized from its bf16 values (KOSMOS section
   * 3.3.1 step 3, section 3.3.2 step 1): dY_d as it lands, H recomputed from
   * the saved G and U, X_d gathered from the token rows x through row_route.
   * Workspace MOE_OP_LAYER_BWD_MXFP8_NATIVE; needs saved->row_route. */
  int32_t mx_wgrad;
} moe_layer_args;

typedef struct moe_layer_saved {
  float* logits;        /* [N][E] */
  int32_t* topk_idx;    /* [N][K] */
  float* topk_prob;     /* [N][K] */
  int32_t* counts;      /* [E] */
  int32_t* offsets;     /* [E+1] */
  int32_t* dst_rows;    /* [N][K] */
  int32_t* row_route;   /* [rows_cap] */
  void* xd;             /* bf16 [rows_cap][D] (bf16 path) */
  uint8_t* xd_q;        /* MXFP8 [rows_cap][D] */
  uint8_t* xd_s;        /* MXFP8 [rows_cap][D/32] */
  void* g;              /* bf16 [rows_cap][H] */
  void* u;              /* bf16 [rows_cap][H] */
  void* h;              /* bf16 [rows_cap][H]; may be NULL for moe_layer_bwd, which then
                           recomputes H = silu(G) U from g and u (KOSMOS's SwiGLU-recompute
                           mode), bitwise equal to the forward's H */
  uint8_t* h_q;         /* MXFP8 [rows_cap][H]; may be NULL for moe_layer_bwd (recompute) */
  uint8_t* h_s;         /* MXFP8 [rows_cap][H/32] */
  void* y;              /* bf16 [rows_cap][D] */
  float* aux;           /* fp32 [1], optional: the aux loss */
  int32_t* status;      /* int32 [1], optional: the device status word (MOE_STATUS_*
                           bits), written by every moe_layer_fwd that gets it */
} moe_layer_saved;

/* Bytes of one buffer that holds every tensor moe_layer_fwd saves for this
 * shape and dtype (OLMo-core Appendix A, A.14: the saved set of the routed
 * expert node), each at a 256-byte offset: logits, topk_idx, topk_prob,
 * counts, offsets, dst_rows, row_route, then xd (bf16) or xd_q, xd_s (MXFP8),
 * g, u, h (bf16) or h_q, h_s (MXFP8; no bf16 H), y, aux and status.
 * 0 if the dims are invalid. */
size_t moe_saved_size(const moe_dims* d, int dtype);
/* Points every field of *out into base (moe_saved_size bytes, 256-byte
 * aligned, caller-owned) in the order above; fields the dtype does not use
 * are set to NULL.  Returns a status code. */
int moe_saved_carve(const moe_dims* d, int dtype, void* base, size_t bytes, moe_layer_saved* out);

int moe_layer_fwd(const moe_layer_args* a, moe_layer_saved* saved, void* out, void* ws,
                  size_t ws_bytes, void* stream);

/* Allocation-free forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): moe_layer_fwd with its workspace in the library's own static
 * device scratch of MOE_NOALLOC_SCRATCH_BYTES (64 MiB), one copy per GPU,
 * held until the process ends.  The caller still passes every
 * input, output and saved tensor.  No call allocates: not this function, not
 * the kernels, not a library routine.  A shape whose
 * moe_workspace_size(MOE_OP_LAYER_FWD) exceeds the scratch returns
 * MOE_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU shares
 * that GPU's scratch, which keeps the last call's contents (each call rebuilds
 * what it reads); calls that overlap on one GPU, on different streams or from
 * different threads, race and must be serialized by the caller. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_layer_fwd_noalloc(const moe_layer_args* a, moe_layer_saved* saved, void* out, void* stream);

typedef struct moe_layer_grads {
  void* dx;        /* bf16 [N][D] */
  float* dprob;    /* fp32 [N][K] */
  void* dw_gate;   /* bf16 [E][H][D] */
  void* dw_up;     /* bf16 [E][H][D] */
  void* dw_down;   /* bf16 [E][D][H] */
  /* Router backward (KOSMOS section 3.3.2 step 2: the router's dX_r and dW_r),
   * run when dw_r is not NULL: dlogits through the (optionally renormalised)
   * softmax weights, dw_r = dlogits^T x, db_r = column sums of dlogits, and
   * dx then also holds dlogits W_r.  Needs saved logits and topk_idx, a->x and
   * a->w_r, and E a multiple of 8 (else MOE_ERR_SHAPE).  db_r and dlogits
   * may be NULL. */
  void* dw_r;      /* bf16 [E][D] */
  float* db_r;     /* fp32 [E] */
  float* dlogits;  /* fp32 [N][E] */
  /* Upstream gradient of the aux loss (a host value; 0 = none).  With
   * a->aux_alpha != 0 the router backward adds d_aux times the aux loss's
   * logit gradient, the counts held fixed. */
  float d_aux;
} moe_layer_grads;

int moe_layer_bwd(const moe_layer_args* a, const moe_layer_saved* saved, const void* dout,
                  moe_layer_grads* grads, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_ROCM_H */
