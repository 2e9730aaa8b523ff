// Host-side launchers of the HIP kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// forward grouped GEMM request (bf16 or MXFP8)
struct GemmFwd {
  int64_t E, rows_cap, k_dim, n_dim;
  const int32_t* offsets;
  const void* a;
  const uint8_t* a_scales;
  const void* b0;
  const uint8_t* b0_scales;
  const void* b1;
  const uint8_t* b1_scales;
  void* c0;
  void* c1;
  void* act;
  uint8_t* act_q;
  uint8_t* act_scales;
  bool swiglu;
  // MXFP8 data gradient of the down projection (single B): the epilogue takes
  // acc = dH, applies the SwiGLU backward with the saved g/u [rows][n_dim],
  // stores dG in c0 and dU in c1 (bf16) and [dG | dU] quantized row-wise in
  // act_q [rows][2 n_dim] / act_scales [rows][2 n_dim / 32]
  bool dswiglu = false;
  const void* g = nullptr;
  const void* u = nullptr;
};

// backward grouped GEMM request (bf16)
struct GemmBwd {
  int64_t E, rows_cap, k_dim, n_dim;
  const int32_t* offsets;
  const void* a;
  const void* b0;
  const void* b1;
  const void* dc0;
  const void* dc1;
  void* da;
  const void* g;
  const void* u;
  void* dg;
  void* du;
  bool swiglu_bwd;
};

// router.hip
size_t router_workspace_bytes(int64_t N, int64_t D, int64_t E);
hipError_t launch_router_logits(const void* x, const void* w_r, const float* bias, int64_t N,
                                int64_t D, int64_t E, float* logits, void* ws, hipStream_t s);
// router backward: dlogits (fp32 and bf16) from the route-weight gradient,
// per-64-token column partials of dlogits, and the token-split offsets
// (S + 1 entries) plus the whole-range offsets {0, N} for the router's GEMMs
int router_wgrad_splits(int64_t N, int64_t D, int64_t E);
hipError_t launch_router_bwd(const float* logits, const int32_t* topk_idx, const float* dprob, int64_t N,
                             int64_t E, int64_t K, int renorm, float* dl, uint16_t* dlb, float* colpart,
                             int32_t* offs, int S, int32_t* offs1, hipStream_t s,
                             const int32_t* aux_counts = nullptr, float aux_c = 0.0f);
// dw_r = bf16(sum over S fp32 partials [S][E*D], in order) when part != NULL;
// db_r = sum over the ceil(N/64) column partials, in a fixed order, when db_r != NULL
hipError_t launch_router_bwd_reduce(const float* part, int S, int64_t ED, uint16_t* dw_r, const float* colpart,
                                    int64_t P, int64_t E, float* db_r, hipStream_t s);

// route.hip
size_t route_workspace_bytes(int64_t N, int64_t E, int64_t K);
hipError_t launch_route(const float* logits, const uint8_t* drop, int64_t N, int64_t E, int64_t K,
                        int renorm, int align, int64_t rows_cap, int32_t* topk_idx, float* topk_prob,
                        int32_t* counts, int32_t* offsets, int32_t* dst_rows, int32_t* row_route,
                        void* ws, hipStream_t s,
                        int n_group = 0, int topk_group = 0, bool aux_inputs = false, int n_shared = 0,
                        int32_t* status = nullptr);
// the device status word (moe_layer_saved.status) set to 0 on the stream
hipError_t launch_status_clear(int32_t* status, hipStream_t s);
// aux loss of the routed layer from the route step's probability sums (left
// in the route workspace by launch_route with aux_inputs) and the counts
hipError_t launch_aux_loss(void* route_ws, int64_t N, int64_t E, int64_t K, const int32_t* counts, float alpha,
                           float* aux, hipStream_t s);

// permute.hip
hipError_t launch_dispatch_bf16(const void* x, const int32_t* dst_rows, const float* weight,
                                int64_t N, int64_t D, int64_t K, void* xd, hipStream_t s,
                         const int32_t* shared_row0 = nullptr);
// pad_counts/pad_offsets (optional): also zero the padding rows of pad_E
// experts, in trailing workgroups of the same launch
hipError_t launch_dispatch_mxfp8(const void* x, const int32_t* dst_rows, int64_t N, int64_t D,
                                 int64_t K, uint8_t* q, uint8_t* sc, hipStream_t s,
                                 const int32_t* shared_row0 = nullptr, const int32_t* pad_counts = nullptr,
                                 const int32_t* pad_offsets = nullptr, int64_t pad_E = 0);
// zero `bytes` bytes at p (16-byte aligned), with a kernel (no memset node
// in a captured graph)
hipError_t launch_zero_bytes(void* p, int64_t bytes, hipStream_t s);

// zero the padding rows of every expert segment in a (row_bytes, a multiple
// of 16), b and c (optional)
hipError_t launch_zero_padding(const int32_t* counts, const int32_t* offsets, int64_t E,
                               int64_t row_bytes, void* a, int64_t row_bytes2, void* b,
                               hipStream_t s, int64_t row_bytes3 = 0, void* c = nullptr);
// addend (bf16 [N][D], optional) is added to each token's fp32 sum before rounding
hipError_t launch_combine(const void* y, const int32_t* dst_rows, const float* weight, int64_t N,
                          int64_t D, int64_t K, void* out, hipStream_t s, const void* addend = nullptr,
                          const int32_t* shared_row0 = nullptr);
// q/sc (optional): dY_d also quantized row-wise to MXFP8 as it is written
// (needs combine_bwd_quant_ok)
hipError_t launch_combine_bwd(const void* dout, const int32_t* dst_rows, const float* weight,
                              const void* y, int64_t N, int64_t D, int64_t K, void* dyd,
                              float* dprob, hipStream_t s,
                         const int32_t* shared_row0 = nullptr, uint8_t* q = nullptr, uint8_t* sc = nullptr);
bool combine_bwd_quant_ok(int64_t D, const void* q, const void* sc);
hipError_t launch_quantize_rows(const void* src, int64_t rows, int64_t cols, uint8_t* q,
                                uint8_t* sc, hipStream_t s, const int32_t* rows_end = nullptr);
// src bf16 [batch][rows][cols] -> q[b][c][col0 + r] (row stride ld), quantized
// along r; scales [b][c][(col0 + r) / 32] (row stride ld / 32)
hipError_t launch_quantize_cols(const void* src, int64_t batch, int64_t rows, int64_t cols, int64_t ld,
                                int64_t col0, uint8_t* q, uint8_t* sc, hipStream_t s);
// column-wise copies for the native MXFP8 wgrad, one contiguous block per
// expert: toff[e] = exclusive scan of the segments rounded up to 128 rows
// (Ex + 1 entries); the copy of src bf16 [rows][cols] (or of the token rows x
// [N][cols] gathered through row_route / K and the shared segment at
// *shared0 when row_route is given) holds expert e as q[C * toff[e] +
// c * len128 + i] (E4M3, blocks of 32 rows i), scales at the byte offset / 32;
// max_cols bounds toff[Ex] (the grid's extent)
hipError_t launch_seg128_scan(const int32_t* offsets, int64_t Ex, int32_t* toff, hipStream_t s);
hipError_t launch_quantize_cols_seg(const void* src, int64_t cols, const int32_t* offsets, int64_t Ex,
                                    const int32_t* toff, int64_t max_cols, const int32_t* row_route, int64_t K,
                                    const int32_t* shared0, int64_t N, uint8_t* q, uint8_t* sc, hipStream_t s);
// bf16 [rows][cols] from E4M3 + E8M0 row-wise blocks; rows >= *rows_end skipped
hipError_t launch_dequant_rows(const uint8_t* q, const uint8_t* sc, int64_t rows, int64_t cols,
                               const int32_t* rows_end, void* out, hipStream_t s);
hipError_t launch_swiglu(const void* g, const void* u, int64_t rows, int64_t n, void* h,
                         uint8_t* hq, uint8_t* hs, hipStream_t s);

// gemm_bf16.hip
int64_t mtile_table_ints(int64_t rows_cap, int64_t E, int BM);
hipError_t launch_build_mtiles(const int32_t* offsets, int64_t E, int BM, int32_t* table, hipStream_t s);
hipError_t launch_gemm_fwd_bf16(const GemmFwd& f, int32_t* table, hipStream_t s);
hipError_t launch_gemm_dgrad_bf16(const GemmBwd& b, int32_t* table, hipStream_t s);
hipError_t launch_gemm_wgrad_bf16(const GemmBwd& b, const void* dc, void* db, hipStream_t s);

// fused bf16 expert forward: dispatch -> GEMM1 (SwiGLU) -> GEMM2 in one
// persistent launch (gemm_fwd.hip)
struct ExpertsFwd {
  int64_t E, K, D, H, rows_cap;
  int64_t N_tokens;                  // tokens (the single-launch layer)
  const int32_t* offsets;
  const int32_t* row_route;
  const int32_t* dst_rows;
  const void* x;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  void* xd;
  void* g;
  void* u;
  void* h;
  void* y;
  int32_t* status;   // optional device status word: MOE_STATUS_WAIT_EXPIRED is or-ed in
  int test_polls;    // > 0: withhold readiness, bound every wait to this many polls
  // MXFP8 (the readiness-gated launch): xd, w_* hold E4M3 codes, these their
  // E8M0 scales; h_q / h_s the quantized H (h is not written); counts for the
  // padding rows of the 32-row groups
  bool mx = false;
  const uint8_t* xd_s = nullptr;
  const uint8_t* wg_s = nullptr;
  const uint8_t* wu_s = nullptr;
  const uint8_t* wd_s = nullptr;
  uint8_t* h_q = nullptr;
  uint8_t* h_s = nullptr;
  const int32_t* counts = nullptr;
};

// gemm_fwd.hip: persistent forward grouped GEMM, bf16 or MXFP8 (shape and
// alignment rule in gemm_fwd_fast_ok), and the fused bf16 expert forward
// (k_dim % 64 == 0, n_dim % 16 == 0 for both of its GEMMs)
size_t experts_fused_ws_ints(int64_t rows_cap, int64_t E);
hipError_t launch_experts_fwd_fused(const ExpertsFwd& x, int32_t* ws, hipStream_t s);

// single-launch layer forward (gemm_fwd.hip): router, route, dispatch, GEMM1,
// GEMM2 and the fold in one persistent launch (after a one-workgroup reset
// of its barrier words); bf16 routed experts, the fused queue's shape rules,
// plus layer_fwd_single_ok.  ws: the GEMM table workspace; route_ws and
// router_ws: the route and router workspaces of the staged launches.
struct LayerFwdSingle {
  ExpertsFwd x;                      // x.x: the token rows; offsets / row_route: the route outputs
  const void* x_tokens;              // [N][D] (the same as x.x)
  const void* w_r;                   // [E][D]
  const float* bias;                 // [E] or null
  float* logits;                     // [N][E]
  const uint8_t* drop;               // [N][K] or null
  int renorm;
  int32_t* topk_idx;
  float* topk_prob;
  int32_t* counts;
  int32_t* dst_rows;
  void* out;                         // [N][D]
};
bool layer_fwd_single_ok(int64_t D, int64_t E, int64_t K);
hipError_t launch_layer_fwd_single(const LayerFwdSingle& a, int32_t* ws, void* route_ws, void* router_ws,
                                   hipStream_t s);
size_t gemm_fwd_plan_ints(int64_t E);
// The persistent GEMMs' workspace starts with the per-XCD queue heads, each
// on its own 128-byte line (claims on one head serialize at the memory side;
// heads that shared a line serialized every claim on the chip).
constexpr int64_t kGemmHeadInts = 256;
bool gemm_fwd_fast_ok(int64_t k_dim, int64_t n_dim);
bool gemm_fwd_fast_ok(const GemmFwd& f, bool mx);
hipError_t launch_gemm_fwd_fast(const GemmFwd& f, bool mx, int32_t* ws, hipStream_t s);

// gemm_bwd.hip: persistent backward GEMMs (shape and alignment rules in the
// *_fast_ok predicates; ws is the GEMM table workspace)
bool gemm_dgrad_fast_ok(const GemmBwd& b);
hipError_t launch_gemm_dgrad_fast(const GemmBwd& b, int32_t* ws, hipStream_t s);
bool gemm_wgrad_fast_ok(const GemmBwd& b, const void* dc, const void* db);
hipError_t launch_gemm_wgrad_fast(const GemmBwd& b, const void* dc, void* db, int32_t* ws, hipStream_t s,
                                  bool f32 = false);
// native MXFP8 wgrad: db[e][m][n] = sum over expert e's rows r of aT[m][r] bT[n][r]
// with the per-expert column-wise copies of launch_quantize_cols_seg (aT of
// width M, bT of width N, both laid out by toff); bf16 db [E][M][N]
bool gemm_wgrad_mx_ok(int64_t M, int64_t N, int64_t max_len);
hipError_t launch_gemm_wgrad_mx(const int32_t* offsets, const int32_t* toff, int64_t E, int64_t M, int64_t N,
                                const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs, void* db,
                                int32_t* ws, hipStream_t s);

// single-launch layer backward (gemm_bwd.hip): the combine backward, the
// expert dgrads and wgrads, the router backward and the fold in one
// persistent launch (after a one-workgroup reset of its barrier words); bf16,
// routed experts, the fast paths' shape rules, E <= 512.  ws: the plans and
// barriers block of layer_bwd_single_ints ints.
struct LayerBwdSingle {
  const void* dout;                  // [N][D]
  const int32_t* dst_rows;           // [N][K]
  const float* topk_prob;            // [N][K]
  const void* y;                     // saved Y
  int64_t N, D, K, E;
  void* dyd;                         // dY_d scratch
  float* dprob;                      // [N][K]
  GemmBwd down;                      // down dgrad (SwiGLU backward) and, with dc = dyd, its wgrad
  GemmBwd gu;                        // gate/up dgrad (dc0 = dG, dc1 = dU) and their wgrads
  void* dw_down;
  void* dw_gate;
  void* dw_up;
  int router;                        // router backward on
  const float* logits;
  const int32_t* topk_idx;
  int renorm;
  float* dl;
  uint16_t* dlb;
  float* colpart;
  int32_t* offs;
  int S;
  int32_t* offs1;
  const int32_t* aux_counts;
  float aux_c;
  GemmBwd rt;                        // dX_r = dL W_r (one expert of N rows; dc0 = dL bf16)
  GemmBwd rs;                        // dW_r over the S token splits (dc0 = dL bf16)
  bool split;                        // dW_r through fp32 partials (part) reduced in order
  float* part;
  void* dw_r;
  float* db_r;
  const void* dxd;                   // dX_d
  void* dx;                          // [N][D]
  const void* dxr;                   // dX_r or null
  int32_t* status;                   // optional status word (expired barrier waits)
  int test_polls;
};
size_t layer_bwd_single_ints(int64_t E, int S);
bool layer_bwd_single_ok(const LayerBwdSingle& a);
hipError_t launch_layer_bwd_single(const LayerBwdSingle& a, int32_t* ws, hipStream_t s);

// gemm_mxfp8.hip
hipError_t launch_gemm_fwd_mxfp8(const GemmFwd& f, int32_t* table, hipStream_t s);

}  // namespace moe
