// C ABI of the MoE expert layer: argument checks, workspace carving and the
// order of kernel launches.  Every call only enqueues work on the caller's
// stream; nothing here synchronises or copies device data to the host.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "../../include/moe_rocm.h"
#include "launch.h"

namespace {

std::atomic<int> g_last_hip_error{0};

constexpr int64_t kMaxE = 1024;
constexpr int64_t kMaxK = 32;

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error.store((int)e);
  return MOE_ERR_HIP;
}

// routed rows, each expert's alignment padding, and the shared expert's segment
int64_t rows_cap_of(const moe_dims& d) {
  return d.N * d.K + d.E * (int64_t)(d.align - 1) + (int64_t)d.n_shared * (d.N + d.align - 1);
}
// experts of the grouped GEMMs: the routed ones and the shared one
int64_t experts_of(const moe_dims& d) { return d.E + d.n_shared; }

// shape rules shared by every entry point
int check_dims(const moe_dims* d, bool need_h, bool mxfp8) {
  if (!d) return MOE_ERR_NULL;
  if (d->N < 0 || d->E < 1 || d->E > kMaxE || d->K < 1 || d->K > d->E || d->K > kMaxK)
    return MOE_ERR_SHAPE;
  if (d->D <= 0 || d->D % 8) return MOE_ERR_SHAPE;
  if (need_h && (d->H <= 0 || d->H % 8)) return MOE_ERR_SHAPE;
  if (d->align != 1 && d->align != 32) return MOE_ERR_SHAPE;
  if (mxfp8 && (d->D % 32 || (need_h && d->H % 32) || d->align != 32)) return MOE_ERR_SHAPE;
  if (d->N * d->K >= (int64_t(1) << 31) || rows_cap_of(*d) >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
  if (d->n_group < 0 || d->n_shared < 0 || d->n_shared > 1) return MOE_ERR_SHAPE;
  if (experts_of(*d) > kMaxE) return MOE_ERR_SHAPE;   // the planners give one thread per expert
  if (d->n_group > 1 && (d->n_group > 64 || d->E % d->n_group || d->topk_group < 1 ||
                         d->topk_group > d->n_group || d->topk_group * (d->E / d->n_group) < d->K))
    return MOE_ERR_SHAPE;
  return MOE_OK;
}

#define REQUIRE(p)                          \
  do {                                      \
    if (!(p)) return MOE_ERR_NULL;          \
    if (!aligned16(p)) return MOE_ERR_ALIGN; \
  } while (0)
#define OPTIONAL(p)                                \
  do {                                             \
    if ((p) && !aligned16(p)) return MOE_ERR_ALIGN; \
  } while (0)
// a buffer whose size is zero when `empty` holds may be NULL then
#define REQUIRE_UNLESS(empty, p) \
  do {                           \
    if (empty) OPTIONAL(p);      \
    else REQUIRE(p);             \
  } while (0)

size_t table_bytes(int64_t rows_cap, int64_t E) {
  const size_t a = (size_t)moe::mtile_table_ints(rows_cap, E, 64) * 4;
  const size_t b = (moe::kGemmHeadInts + moe::gemm_fwd_plan_ints(E)) * 4;
  const size_t c = moe::experts_fused_ws_ints(rows_cap, E) * 4;
  size_t m = a > b ? a : b;
  m = m > c ? m : c;
  return round_up(m, 256);
}

// forward GEMM: the persistent kernel where its shape and alignment rule
// holds, else the m-tile kernels
hipError_t gemm_fwd_bf16(const moe::GemmFwd& f, int32_t* ws, hipStream_t s) {
  if (moe::gemm_fwd_fast_ok(f, false)) return moe::launch_gemm_fwd_fast(f, false, ws, s);
  return moe::launch_gemm_fwd_bf16(f, ws, s);
}

// backward GEMMs: the persistent kernels where their rules hold
hipError_t gemm_dgrad(const moe::GemmBwd& b, int32_t* ws, hipStream_t s) {
  if (moe::gemm_dgrad_fast_ok(b)) return moe::launch_gemm_dgrad_fast(b, ws, s);
  return moe::launch_gemm_dgrad_bf16(b, ws, s);
}

hipError_t gemm_wgrad(const moe::GemmBwd& b, const void* dc, void* db, int32_t* ws, hipStream_t s) {
  if (moe::gemm_wgrad_fast_ok(b, dc, db)) return moe::launch_gemm_wgrad_fast(b, dc, db, ws, s);
  return moe::launch_gemm_wgrad_bf16(b, dc, db, s);
}

hipError_t gemm_fwd_mxfp8(const moe::GemmFwd& f, int32_t* ws, hipStream_t s) {
  if (moe::gemm_fwd_fast_ok(f, true)) return moe::launch_gemm_fwd_fast(f, true, ws, s);
  return moe::launch_gemm_fwd_mxfp8(f, ws, s);
}

size_t route_bytes(const moe_dims& d) { return round_up(moe::route_workspace_bytes(d.N, d.E, d.K), 256); }

size_t router_bytes(const moe_dims& d) { return round_up(moe::router_workspace_bytes(d.N, d.D, d.E), 256); }

// router backward scratch: dlogits fp32 and bf16, dX_r, split offsets, wgrad
// partials and column partials
struct RouterBwdLayout {
  size_t dl, dlb, dxr, offs, part, colpart, total;
  int S;
};

RouterBwdLayout router_bwd_layout(const moe_dims& d) {
  RouterBwdLayout l{};
  const size_t N = (size_t)d.N, E = (size_t)d.E, D = (size_t)d.D;
  l.S = moe::router_wgrad_splits(d.N, d.D, d.E);
  size_t o = 0;
  l.dl = o;
  o += round_up(N * E * 4, 256);
  l.dlb = o;
  o += round_up(N * E * 2, 256);
  l.dxr = o;
  o += round_up(N * D * 2, 256);
  l.offs = o;
  o += 256;
  l.part = o;
  o += round_up((size_t)l.S * E * D * 4, 256);
  l.colpart = o;
  o += round_up(((N + 63) / 64) * E * 4, 256);
  l.total = o;
  return l;
}

// layer backward scratch (after the GEMM table): dY_d, dX_d, dG, dU and H
// (recomputed, or dequantized from h_q), then for MXFP8 dY_d quantized,
// [dG | dU] quantized and X_d dequantized, then the router backward's scratch
struct BwdLayout {
  size_t dyd, dxd, dg, du, h, dyq, dys, guq, gus, xdeq, router, single, total;
  // native MXFP8 wgrad: per-expert block offsets and the column-wise copies
  // (width x ldt codes, width x ldt / 32 scales)
  size_t toff, dyt_q, dyt_s, xt_q, xt_s, ht_q, ht_s, dgt_q, dgt_s, dut_q, dut_s;
  int64_t ldt;
};

// columns of the column-wise copies: each expert's rows rounded up to whole
// 128-column contraction steps, so at most rows_cap + 96 per expert
int64_t cols_ld(const moe_dims& d) { return (rows_cap_of(d) + 96 * experts_of(d) + 127) / 128 * 128; }

BwdLayout bwd_layout(const moe_dims& d, bool mx, bool mxw = false) {
  BwdLayout l{};
  const size_t rc = (size_t)rows_cap_of(d), D = (size_t)d.D, H = (size_t)d.H;
  size_t o = 0;
  auto take = [&o](size_t& at, size_t bytes) {
    at = o;
    o += round_up(bytes, 256);
  };
  take(l.dyd, rc * D * 2);
  take(l.dxd, rc * D * 2);
  take(l.dg, rc * H * 2);
  take(l.du, rc * H * 2);
  take(l.h, rc * H * 2);
  if (mx) {
    take(l.dyq, rc * D);
    take(l.dys, rc * D / 32);
    take(l.guq, rc * 2 * H);
    take(l.gus, rc * 2 * H / 32);
    take(l.xdeq, rc * D * 2);
  }
  if (mx && mxw) {
    const size_t ldt = (size_t)cols_ld(d);
    l.ldt = (int64_t)ldt;
    take(l.toff, ((size_t)experts_of(d) + 1) * 4);
    take(l.dyt_q, D * ldt);
    take(l.dyt_s, D * ldt / 32);
    take(l.xt_q, D * ldt);
    take(l.xt_s, D * ldt / 32);
    take(l.ht_q, H * ldt);
    take(l.ht_s, H * ldt / 32);
    take(l.dgt_q, H * ldt);
    take(l.dgt_s, H * ldt / 32);
    take(l.dut_q, H * ldt);
    take(l.dut_s, H * ldt / 32);
  }
  take(l.router, router_bwd_layout(d).total);
  // the single-launch backward's queue plans and barrier words
  take(l.single, moe::layer_bwd_single_ints(experts_of(d), router_bwd_layout(d).S) * 4);
  l.total = o;
  return l;
}

size_t bwd_scratch_bytes(const moe_dims& d, bool mx, bool mxw = false) { return bwd_layout(d, mx, mxw).total; }

// The saved set carved from one buffer, every tensor at a 256-byte offset;
// at[i] = SIZE_MAX marks a field the dtype does not use.
struct SavedLayout {
  size_t at[18];
  size_t total;
};

SavedLayout saved_layout(const moe_dims& d, bool mx) {
  SavedLayout l{};
  const size_t N = (size_t)d.N, D = (size_t)d.D, E = (size_t)d.E, K = (size_t)d.K, H = (size_t)d.H;
  const size_t Ex = (size_t)experts_of(d), rc = (size_t)rows_cap_of(d);
  const size_t none = SIZE_MAX;
  // logits, topk_idx, topk_prob, counts, offsets, dst_rows, row_route, xd, xd_q,
  // xd_s, g, u, h, h_q, h_s, y, aux, status (the field order of moe_layer_saved)
  const size_t bytes[18] = {N * E * 4, N * K * 4, N * K * 4, Ex * 4, (Ex + 1) * 4, N * K * 4, rc * 4,
                            mx ? none : rc * D * 2, mx ? rc * D : none, mx ? rc * D / 32 : none,
                            rc * H * 2, rc * H * 2, mx ? none : rc * H * 2, mx ? rc * H : none,
                            mx ? rc * H / 32 : none, rc * D * 2, 4, 4};
  size_t o = 0;
  for (int i = 0; i < 18; ++i) {
    if (bytes[i] == none) {
      l.at[i] = none;
      continue;
    }
    l.at[i] = o;
    o += round_up(bytes[i] > 0 ? bytes[i] : 1, 256);
  }
  l.total = o;
  return l;
}

// Scratch of the allocation-free forward: a file-scope device array, one copy
// per GPU, alive until the process ends.  Host code never uses its name as an
// address (that is a host-side stand-in): each device's address comes from
// hipGetSymbolAddress, taken once with that device current.
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the current device's scratch address, or NULL with *err set
void* scratch_ptr(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int64_t moe_rows_cap(const moe_dims* d) { return d ? rows_cap_of(*d) : -1; }

size_t moe_workspace_size(int op, const moe_dims* d) {
  if (!d) return 0;
  const int64_t rc = rows_cap_of(*d);
  switch (op) {
    case MOE_OP_ROUTE: return route_bytes(*d);
    case MOE_OP_GEMM: return table_bytes(rc, experts_of(*d));
    case MOE_OP_ROUTER: return router_bytes(*d);
    case MOE_OP_LAYER_FWD: return route_bytes(*d) + table_bytes(rc, experts_of(*d)) + router_bytes(*d);
    case MOE_OP_LAYER_BWD: return table_bytes(rc, experts_of(*d)) + bwd_scratch_bytes(*d, false);
    case MOE_OP_LAYER_BWD_MXFP8: return table_bytes(rc, experts_of(*d)) + bwd_scratch_bytes(*d, true);
    case MOE_OP_LAYER_BWD_MXFP8_NATIVE: return table_bytes(rc, experts_of(*d)) + bwd_scratch_bytes(*d, true, true);
    default: return 0;
  }
}

size_t moe_saved_size(const moe_dims* d, int dtype) {
  if (dtype != MOE_BF16 && dtype != MOE_MXFP8) return 0;
  if (check_dims(d, true, dtype == MOE_MXFP8)) return 0;
  return saved_layout(*d, dtype == MOE_MXFP8).total;
}

int moe_saved_carve(const moe_dims* d, int dtype, void* base, size_t bytes, moe_layer_saved* out) {
  if (dtype != MOE_BF16 && dtype != MOE_MXFP8) return MOE_ERR_DTYPE;
  const bool mx = dtype == MOE_MXFP8;
  int st = check_dims(d, true, mx);
  if (st) return st;
  if (!out) return MOE_ERR_NULL;
  REQUIRE(base);
  if ((uintptr_t)base & 255u) return MOE_ERR_ALIGN;
  const SavedLayout l = saved_layout(*d, mx);
  if (bytes < l.total) return MOE_ERR_WORKSPACE;
  void* p[18];
  for (int i = 0; i < 18; ++i) p[i] = l.at[i] == SIZE_MAX ? nullptr : (char*)base + l.at[i];
  out->logits = (float*)p[0];
  out->topk_idx = (int32_t*)p[1];
  out->topk_prob = (float*)p[2];
  out->counts = (int32_t*)p[3];
  out->offsets = (int32_t*)p[4];
  out->dst_rows = (int32_t*)p[5];
  out->row_route = (int32_t*)p[6];
  out->xd = p[7];
  out->xd_q = (uint8_t*)p[8];
  out->xd_s = (uint8_t*)p[9];
  out->g = p[10];
  out->u = p[11];
  out->h = p[12];
  out->h_q = (uint8_t*)p[13];
  out->h_s = (uint8_t*)p[14];
  out->y = p[15];
  out->aux = (float*)p[16];
  out->status = (int32_t*)p[17];
  return MOE_OK;
}

const char* moe_status_string(int s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null argument";
    case MOE_ERR_SHAPE: return "bad shape";
    case MOE_ERR_DTYPE: return "bad dtype or epilogue";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_ALIGN: return "pointer not 16-byte aligned";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int moe_last_hip_error(void) { return g_last_hip_error.load(); }

int moe_router_logits(const void* x, const void* w_r, const float* bias, const moe_dims* d,
                      float* logits, void* ws, size_t ws_bytes, void* stream) {
  int st = check_dims(d, false, false);
  if (st) return st;
  REQUIRE_UNLESS(d->N == 0, x);
  REQUIRE(w_r);
  REQUIRE_UNLESS(d->N == 0, logits);
  OPTIONAL(bias);
  const size_t need = router_bytes(*d);
  REQUIRE_UNLESS(need == 0, ws);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_router_logits(x, w_r, bias, d->N, d->D, d->E, logits, ws, (hipStream_t)stream));
}

int moe_route(const float* logits, const uint8_t* drop, const moe_dims* d, int32_t* topk_idx,
              float* topk_prob, int32_t* counts, int32_t* offsets, int32_t* dst_rows,
              int32_t* row_route, void* ws, size_t ws_bytes, void* stream) {
  int st = check_dims(d, false, false);
  if (st) return st;
  const bool no_tok = d->N == 0;
  REQUIRE_UNLESS(no_tok, logits);
  REQUIRE_UNLESS(no_tok, topk_idx);
  REQUIRE_UNLESS(no_tok, topk_prob);
  REQUIRE(counts);
  REQUIRE(offsets);
  REQUIRE_UNLESS(no_tok, dst_rows);
  REQUIRE_UNLESS(rows_cap_of(*d) == 0, row_route);
  REQUIRE(ws);
  OPTIONAL(drop);
  if (ws_bytes < route_bytes(*d)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_route(logits, drop, d->N, d->E, d->K, d->renorm, d->align,
                                      rows_cap_of(*d), topk_idx, topk_prob, counts, offsets,
                                      dst_rows, row_route, ws, (hipStream_t)stream, d->n_group,
                                      d->topk_group, false, d->n_shared));
}

int moe_dispatch(const void* x, const int32_t* dst_rows, const float* weight, const int32_t* counts,
                 const int32_t* offsets, const moe_dims* d, int out_dtype, void* xd,
                 uint8_t* xd_scales, void* stream) {
  if (out_dtype != MOE_BF16 && out_dtype != MOE_MXFP8) return MOE_ERR_DTYPE;
  const bool mx = out_dtype == MOE_MXFP8;
  int st = check_dims(d, false, mx);
  if (!st && d->n_shared) return MOE_ERR_UNSUPPORTED;   // the shared expert is a layer-level option
  if (st) return st;
  REQUIRE_UNLESS(d->N == 0, x);
  REQUIRE_UNLESS(d->N == 0, dst_rows);
  REQUIRE_UNLESS(rows_cap_of(*d) == 0, xd);
  OPTIONAL(weight);
  if (mx) {
    REQUIRE_UNLESS(rows_cap_of(*d) == 0, xd_scales);
    if (weight) return MOE_ERR_UNSUPPORTED;
  }
  if (d->align > 1) {
    REQUIRE(counts);
    REQUIRE(offsets);
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (mx)   // the padding rows are zeroed in the same launch
    e = moe::launch_dispatch_mxfp8(x, dst_rows, d->N, d->D, d->K, (uint8_t*)xd, xd_scales, s, nullptr,
                                   d->align > 1 ? counts : nullptr, offsets, d->E);
  else
    e = moe::launch_dispatch_bf16(x, dst_rows, weight, d->N, d->D, d->K, xd, s);
  if (e == hipSuccess && d->align > 1 && !mx)
    e = moe::launch_zero_padding(counts, offsets, d->E, d->D * 2, xd, 0, nullptr, s);
  return hip_status(e);
}

int moe_combine(const void* y, const int32_t* dst_rows, const float* weight, const moe_dims* d,
                void* out, void* stream) {
  int st = check_dims(d, false, false);
  if (!st && d->n_shared) return MOE_ERR_UNSUPPORTED;   // the shared expert is a layer-level option
  if (st) return st;
  REQUIRE_UNLESS(d->N == 0, y);
  REQUIRE_UNLESS(d->N == 0, dst_rows);
  REQUIRE_UNLESS(d->N == 0, out);
  OPTIONAL(weight);
  return hip_status(moe::launch_combine(y, dst_rows, weight, d->N, d->D, d->K, out, (hipStream_t)stream));
}

int moe_combine_bwd(const void* dout, const int32_t* dst_rows, const float* weight, const void* y,
                    const moe_dims* d, void* dyd, float* dprob, void* stream) {
  int st = check_dims(d, false, false);
  if (!st && d->n_shared) return MOE_ERR_UNSUPPORTED;   // the shared expert is a layer-level option
  if (st) return st;
  const bool no_tok = d->N == 0;
  REQUIRE_UNLESS(no_tok, dout);
  REQUIRE_UNLESS(no_tok, dst_rows);
  REQUIRE_UNLESS(no_tok, weight);
  REQUIRE_UNLESS(no_tok, dyd);
  OPTIONAL(dprob);
  if (dprob) REQUIRE_UNLESS(no_tok, y);
  return hip_status(moe::launch_combine_bwd(dout, dst_rows, weight, y, d->N, d->D, d->K, dyd, dprob,
                                            (hipStream_t)stream));
}

int moe_quantize_mxfp8(const void* src, int64_t rows, int64_t cols, uint8_t* q, uint8_t* scales,
                       void* stream) {
  if (rows < 0 || cols <= 0 || cols % 32 || rows * cols >= (int64_t(1) << 40)) return MOE_ERR_SHAPE;
  REQUIRE(src);
  REQUIRE(q);
  REQUIRE(scales);
  return hip_status(moe::launch_quantize_rows(src, rows, cols, q, scales, (hipStream_t)stream));
}

int moe_quantize_mxfp8_cols(const void* src, int64_t batch, int64_t rows, int64_t cols, int64_t ld,
                            int64_t col0, uint8_t* q, uint8_t* scales, void* stream) {
  if (batch < 0 || rows < 0 || cols < 0 || rows % 32 || cols % 8 || ld <= 0 || ld % 32 || col0 < 0 ||
      col0 % 32 || col0 + rows > ld || batch > 65535 || (rows + 127) / 128 > 65535 ||
      batch * cols * ld >= (int64_t(1) << 40))
    return MOE_ERR_SHAPE;
  REQUIRE(src);
  REQUIRE(q);
  REQUIRE(scales);
  return hip_status(moe::launch_quantize_cols(src, batch, rows, cols, ld, col0, q, scales, (hipStream_t)stream));
}

int moe_swiglu(const void* g, const void* u, int64_t rows, int64_t n, int out_dtype, void* h,
               uint8_t* h_q, uint8_t* h_scales, void* stream) {
  if (out_dtype != MOE_BF16 && out_dtype != MOE_MXFP8) return MOE_ERR_DTYPE;
  if (rows < 0 || n <= 0 || n % 8) return MOE_ERR_SHAPE;
  REQUIRE(g);
  REQUIRE(u);
  if (out_dtype == MOE_MXFP8) {
    if (n % 32) return MOE_ERR_SHAPE;
    REQUIRE(h_q);
    REQUIRE(h_scales);
    OPTIONAL(h);
  } else {
    REQUIRE(h);
    h_q = nullptr;
    h_scales = nullptr;
  }
  return hip_status(moe::launch_swiglu(g, u, rows, n, h, h_q, h_scales, (hipStream_t)stream));
}

int moe_grouped_gemm_fwd(const moe_gemm_fwd_args* g, void* ws, size_t ws_bytes, void* stream) {
  if (!g) return MOE_ERR_NULL;
  if (g->dtype != MOE_BF16 && g->dtype != MOE_MXFP8) return MOE_ERR_DTYPE;
  if (g->epilogue != MOE_EPI_NONE && g->epilogue != MOE_EPI_SWIGLU) return MOE_ERR_DTYPE;
  const bool mx = g->dtype == MOE_MXFP8;
  const bool sw = g->epilogue == MOE_EPI_SWIGLU;
  const int64_t mult = mx ? 32 : 8;
  if (g->E < 1 || g->E > kMaxE || g->rows_cap < 0 || g->rows_cap >= (int64_t(1) << 31) ||
      g->k_dim <= 0 || g->n_dim <= 0 || g->k_dim % mult || g->n_dim % 8)
    return MOE_ERR_SHAPE;
  REQUIRE(g->offsets);
  REQUIRE(g->a);
  REQUIRE(g->b0);
  REQUIRE(g->c0);
  REQUIRE(ws);
  if (mx) {
    REQUIRE(g->a_scales);
    REQUIRE(g->b0_scales);
  }
  if (sw) {
    REQUIRE(g->b1);
    REQUIRE(g->c1);
    if (mx && g->act_q) OPTIONAL(g->act);   // H may be kept quantized only
    else REQUIRE(g->act);
    if (mx) REQUIRE(g->b1_scales);
  }
  OPTIONAL(g->act_q);
  OPTIONAL(g->act_scales);
  if ((g->act_q != nullptr) != (g->act_scales != nullptr)) return MOE_ERR_NULL;
  if (g->act_q && (!sw || g->n_dim % 32)) return MOE_ERR_SHAPE;
  if (ws_bytes < table_bytes(g->rows_cap, g->E)) return MOE_ERR_WORKSPACE;
  moe::GemmFwd f{g->E, g->rows_cap, g->k_dim, g->n_dim, g->offsets, g->a, g->a_scales, g->b0,
                 g->b0_scales, g->b1, g->b1_scales, g->c0, g->c1, g->act, g->act_q,
                 g->act_scales, sw};
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = mx ? gemm_fwd_mxfp8(f, (int32_t*)ws, s)
                    : gemm_fwd_bf16(f, (int32_t*)ws, s);
  if (e == hipSuccess && !mx && g->act_q)
    e = moe::launch_quantize_rows(g->act, g->rows_cap, g->n_dim, g->act_q, g->act_scales, s);
  return hip_status(e);
}

int moe_grouped_gemm_bwd(const moe_gemm_bwd_args* g, void* ws, size_t ws_bytes, void* stream) {
  if (!g) return MOE_ERR_NULL;
  if (g->dtype != MOE_BF16) return g->dtype == MOE_MXFP8 ? MOE_ERR_UNSUPPORTED : MOE_ERR_DTYPE;
  if (g->epilogue != MOE_EPI_NONE && g->epilogue != MOE_EPI_SWIGLU_BWD) return MOE_ERR_DTYPE;
  const bool swb = g->epilogue == MOE_EPI_SWIGLU_BWD;
  if (g->E < 1 || g->E > kMaxE || g->rows_cap < 0 || g->rows_cap >= (int64_t(1) << 31) ||
      g->k_dim <= 0 || g->n_dim <= 0 || g->k_dim % 8 || g->n_dim % 8)
    return MOE_ERR_SHAPE;
  REQUIRE(g->offsets);
  REQUIRE(g->dc0);
  REQUIRE(ws);
  OPTIONAL(g->dc1);
  const bool want_dgrad = swb ? (g->dg != nullptr) : (g->da != nullptr);
  const bool want_wgrad = g->db0 != nullptr || g->db1 != nullptr;
  if (!want_dgrad && !want_wgrad) return MOE_ERR_NULL;
  if (want_dgrad) {
    REQUIRE(g->b0);
    if (g->dc1) REQUIRE(g->b1);
    if (swb) {
      if (g->dc1) return MOE_ERR_UNSUPPORTED;
      REQUIRE(g->g);
      REQUIRE(g->u);
      REQUIRE(g->dg);
      REQUIRE(g->du);
    } else {
      REQUIRE(g->da);
    }
  }
  if (want_wgrad) {
    REQUIRE(g->a);
    OPTIONAL(g->db0);
    OPTIONAL(g->db1);
    if (g->db1) REQUIRE(g->dc1);
  }
  if (ws_bytes < table_bytes(g->rows_cap, g->E)) return MOE_ERR_WORKSPACE;
  moe::GemmBwd b{g->E, g->rows_cap, g->k_dim, g->n_dim, g->offsets, g->a, g->b0, g->b1,
                 g->dc0, g->dc1, g->da, g->g, g->u, g->dg, g->du, swb};
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (want_dgrad) e = gemm_dgrad(b, (int32_t*)ws, s);
  if (e == hipSuccess && g->db0) e = gemm_wgrad(b, g->dc0, g->db0, (int32_t*)ws, s);
  if (e == hipSuccess && g->db1) e = gemm_wgrad(b, g->dc1, g->db1, (int32_t*)ws, s);
  return hip_status(e);
}

int moe_layer_fwd(const moe_layer_args* a, moe_layer_saved* sv, void* out, void* ws,
                  size_t ws_bytes, void* stream) {
  if (!a || !sv) return MOE_ERR_NULL;
  if (a->dtype != MOE_BF16 && a->dtype != MOE_MXFP8) return MOE_ERR_DTYPE;
  if (a->sched != MOE_SCHED_STAGED && a->sched != MOE_SCHED_READY && a->sched != MOE_SCHED_SINGLE)
    return MOE_ERR_DTYPE;
  const bool mx = a->dtype == MOE_MXFP8;
  const moe_dims& d = a->dims;
  int st = check_dims(&d, true, mx);
  if (st) return st;
  const bool ready = a->sched == MOE_SCHED_READY;
  const bool single = a->sched == MOE_SCHED_SINGLE;
  // the readiness-ordered launches run the persistent GEMM engine on routed
  // experts only: bf16 unpadded, or MXFP8 (READY only) with both GEMMs'
  // reduction dimensions whole 128-value steps
  if ((ready || single) && d.n_shared) return MOE_ERR_UNSUPPORTED;
  if (single && mx) return MOE_ERR_UNSUPPORTED;
  if ((ready || single) && !mx &&
      (d.align != 1 || !moe::gemm_fwd_fast_ok(d.D, d.H) || !moe::gemm_fwd_fast_ok(d.H, d.D)))
    return MOE_ERR_UNSUPPORTED;
  if (ready && mx && (d.D % 128 || d.H % 128 || d.D * d.H >= (int64_t(1) << 31)))
    return MOE_ERR_UNSUPPORTED;
  // the single launch also runs the tiled router and the plain top-K
  if (single && (!moe::layer_fwd_single_ok(d.D, d.E, d.K) || d.n_group > 1 ||
                 (sv->aux != nullptr && a->aux_alpha != 0.0f)))
    return MOE_ERR_UNSUPPORTED;
  if (a->ready_test_polls < 0) return MOE_ERR_SHAPE;
  // buffers of N tokens, or of rows_cap rows, may be NULL when that is 0
  const bool no_tok = d.N == 0, no_rows = rows_cap_of(d) == 0;
  REQUIRE_UNLESS(no_tok, a->x);
  REQUIRE(a->w_r);
  OPTIONAL(a->bias);
  OPTIONAL(a->drop);
  REQUIRE_UNLESS(no_tok, out);
  REQUIRE(ws);
  REQUIRE_UNLESS(no_tok, sv->logits);
  REQUIRE_UNLESS(no_tok, sv->topk_idx);
  REQUIRE_UNLESS(no_tok, sv->topk_prob);
  REQUIRE(sv->counts);
  REQUIRE(sv->offsets);
  REQUIRE_UNLESS(no_tok, sv->dst_rows);
  REQUIRE_UNLESS(no_rows, sv->row_route);
  REQUIRE_UNLESS(no_rows, sv->g);
  REQUIRE_UNLESS(no_rows, sv->u);
  REQUIRE_UNLESS(no_rows, sv->y);
  OPTIONAL(sv->status);
  if (mx) {
    OPTIONAL(sv->h);   // not written: the MXFP8 path keeps H quantized only
    REQUIRE(a->wg_q);
    REQUIRE(a->wg_s);
    REQUIRE(a->wu_q);
    REQUIRE(a->wu_s);
    REQUIRE(a->wd_q);
    REQUIRE(a->wd_s);
    REQUIRE_UNLESS(no_rows, sv->xd_q);
    REQUIRE_UNLESS(no_rows, sv->xd_s);
    REQUIRE_UNLESS(no_rows, sv->h_q);
    REQUIRE_UNLESS(no_rows, sv->h_s);
  } else {
    REQUIRE(a->w_gate);
    REQUIRE(a->w_up);
    REQUIRE(a->w_down);
    REQUIRE_UNLESS(no_rows, sv->xd);
    REQUIRE_UNLESS(no_rows, sv->h);
  }
  OPTIONAL(sv->aux);
  const bool aux = sv->aux != nullptr && a->aux_alpha != 0.0f;
  const int64_t rc = rows_cap_of(d);
  const int64_t Ex = experts_of(d);
  const int32_t* shared_row0 = d.n_shared ? sv->offsets + d.E : nullptr;   // the shared expert's segment
  const size_t rb = route_bytes(d), tb = table_bytes(rc, Ex);
  if (ws_bytes < rb + tb + router_bytes(d)) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  void* ws_route = ws;
  int32_t* table = (int32_t*)((char*)ws + rb);
  void* ws_router = (char*)ws + rb + tb;

  if (no_tok) {
    // no tokens, under every schedule: the route step alone (counts and
    // offsets 0, every row of row_route -1, no expert row to compute) and an
    // aux loss of 0
    hipError_t e = sv->status ? moe::launch_status_clear(sv->status, s) : hipSuccess;
    if (e == hipSuccess)
      e = moe::launch_route(nullptr, nullptr, 0, d.E, d.K, d.renorm, d.align, rc, nullptr, nullptr, sv->counts,
                            sv->offsets, nullptr, sv->row_route, ws_route, s, d.n_group, d.topk_group, false,
                            d.n_shared, sv->status);
    if (e == hipSuccess && aux) e = moe::launch_zero_bytes(sv->aux, 4, s);
    return hip_status(e);
  }
  if (single) {
    // router, route, dispatch, GEMM1, GEMM2 and the fold in one persistent launch
    moe::LayerFwdSingle one{};
    one.x = moe::ExpertsFwd{d.E,     d.K,      d.D,      d.H,    rc,     d.N,     sv->offsets,
                            sv->row_route, sv->dst_rows, a->x, a->w_gate, a->w_up, a->w_down, sv->xd,
                            sv->g,   sv->u,    sv->h,    sv->y,  sv->status, a->ready_test_polls};
    one.x_tokens = a->x;
    one.w_r = a->w_r;
    one.bias = a->bias;
    one.logits = sv->logits;
    one.drop = a->drop;
    one.renorm = d.renorm;
    one.topk_idx = sv->topk_idx;
    one.topk_prob = sv->topk_prob;
    one.counts = sv->counts;
    one.dst_rows = sv->dst_rows;
    one.out = out;
    return hip_status(moe::launch_layer_fwd_single(one, table, ws_route, ws_router, s));
  }
  hipError_t e = sv->status ? moe::launch_status_clear(sv->status, s) : hipSuccess;
  if (e == hipSuccess)
    e = moe::launch_router_logits(a->x, a->w_r, a->bias, d.N, d.D, d.E, sv->logits, ws_router, s);
  if (e == hipSuccess)
    e = moe::launch_route(sv->logits, a->drop, d.N, d.E, d.K, d.renorm, d.align, rc, sv->topk_idx,
                          sv->topk_prob, sv->counts, sv->offsets, sv->dst_rows, sv->row_route,
                          ws_route, s, d.n_group, d.topk_group, aux, d.n_shared, sv->status);
  if (e == hipSuccess && aux) e = moe::launch_aux_loss(ws_route, d.N, d.E, d.K, sv->counts, a->aux_alpha, sv->aux, s);
  if (mx && ready) {
    // quantize-on-dispatch, GEMM1 (H stored quantized) and GEMM2 in one
    // persistent launch scheduled by readiness
    moe::ExpertsFwd xf{d.E,     d.K,        d.D,      d.H,      rc,    d.N,   sv->offsets, sv->row_route,
                       sv->dst_rows, a->x, a->wg_q, a->wu_q, a->wd_q, sv->xd_q, sv->g, sv->u,
                       nullptr, sv->y,      sv->status, a->ready_test_polls};
    xf.mx = true;
    xf.xd_s = sv->xd_s;
    xf.wg_s = a->wg_s;
    xf.wu_s = a->wu_s;
    xf.wd_s = a->wd_s;
    xf.h_q = sv->h_q;
    xf.h_s = sv->h_s;
    xf.counts = sv->counts;
    if (e == hipSuccess) e = moe::launch_experts_fwd_fused(xf, table, s);
  } else if (mx) {
    // quantize-on-dispatch; the same launch zeroes the padding rows
    if (e == hipSuccess)
      e = moe::launch_dispatch_mxfp8(a->x, sv->dst_rows, d.N, d.D, d.K, sv->xd_q, sv->xd_s, s, shared_row0,
                                     sv->counts, sv->offsets, Ex);
    moe::GemmFwd g1{Ex, rc, d.D, d.H, sv->offsets, sv->xd_q, sv->xd_s, a->wg_q, a->wg_s, a->wu_q,
                    a->wu_s, sv->g, sv->u, nullptr, sv->h_q, sv->h_s, true};
    if (e == hipSuccess) e = gemm_fwd_mxfp8(g1, table, s);
    moe::GemmFwd g2{Ex, rc, d.H, d.D, sv->offsets, sv->h_q, sv->h_s, a->wd_q, a->wd_s, nullptr,
                    nullptr, sv->y, nullptr, nullptr, nullptr, nullptr, false};
    if (e == hipSuccess) e = gemm_fwd_mxfp8(g2, table, s);
  } else if (ready) {
    // dispatch, GEMM1 and GEMM2 in one persistent launch scheduled by readiness
    moe::ExpertsFwd xf{d.E,     d.K,        d.D,   d.H,   rc,    d.N,   sv->offsets, sv->row_route,
                       sv->dst_rows, a->x, a->w_gate, a->w_up, a->w_down, sv->xd, sv->g, sv->u,
                       sv->h,   sv->y,      sv->status, a->ready_test_polls};
    if (e == hipSuccess) e = moe::launch_experts_fwd_fused(xf, table, s);
  } else {
    if (e == hipSuccess)
      e = moe::launch_dispatch_bf16(a->x, sv->dst_rows, nullptr, d.N, d.D, d.K, sv->xd, s, shared_row0);
    if (e == hipSuccess && d.align > 1)
      e = moe::launch_zero_padding(sv->counts, sv->offsets, Ex, d.D * 2, sv->xd, 0, nullptr, s);
    moe::GemmFwd g1{Ex, rc, d.D, d.H, sv->offsets, sv->xd, nullptr, a->w_gate, nullptr, a->w_up,
                    nullptr, sv->g, sv->u, sv->h, nullptr, nullptr, true};
    if (e == hipSuccess) e = gemm_fwd_bf16(g1, table, s);
    moe::GemmFwd g2{Ex, rc, d.H, d.D, sv->offsets, sv->h, nullptr, a->w_down, nullptr, nullptr,
                    nullptr, sv->y, nullptr, nullptr, nullptr, nullptr, false};
    if (e == hipSuccess) e = gemm_fwd_bf16(g2, table, s);
  }
  if (e == hipSuccess)
    e = moe::launch_combine(sv->y, sv->dst_rows, sv->topk_prob, d.N, d.D, d.K, out, s, nullptr, shared_row0);
  return hip_status(e);
}

int moe_layer_fwd_noalloc(const moe_layer_args* a, moe_layer_saved* sv, void* out, void* stream) {
  if (!a || !sv) return MOE_ERR_NULL;
  const bool mx = a->dtype == MOE_MXFP8;
  int st = check_dims(&a->dims, true, mx);
  if (st) return st;
  // the workspace moe_layer_fwd would take must fit the static scratch
  const moe_dims& d = a->dims;
  if (route_bytes(d) + table_bytes(rows_cap_of(d), experts_of(d)) + router_bytes(d) > kScratchBytes)
    return MOE_ERR_WORKSPACE;
  hipError_t err = hipSuccess;
  void* ws = scratch_ptr(&err);
  if (!ws) return hip_status(err);
  // every part of the workspace is written by the kernels that read it (plans,
  // queue heads and route histograms are built in the same call), so stale
  // contents from an earlier call do not matter
  return moe_layer_fwd(a, sv, out, ws, kScratchBytes, stream);
}

int moe_layer_bwd(const moe_layer_args* a, const moe_layer_saved* sv, const void* dout,
                  moe_layer_grads* gr, void* ws, size_t ws_bytes, void* stream) {
  if (!a || !sv || !gr) return MOE_ERR_NULL;
  if (a->dtype != MOE_BF16 && a->dtype != MOE_MXFP8) return MOE_ERR_DTYPE;
  const bool mx = a->dtype == MOE_MXFP8;
  const moe_dims& d = a->dims;
  int st = check_dims(&d, true, mx);
  if (st) return st;
  if (a->mx_wgrad != 0 && (a->mx_wgrad != 1 || !mx)) return MOE_ERR_DTYPE;
  const bool mxw = mx && a->mx_wgrad == 1;
  if (a->sched != MOE_SCHED_STAGED && a->sched != MOE_SCHED_READY && a->sched != MOE_SCHED_SINGLE)
    return MOE_ERR_DTYPE;
  // MOE_SCHED_SINGLE: the bf16 routed-expert backward from the saved H, in one launch
  const bool single = a->sched == MOE_SCHED_SINGLE;
  if (single && (mx || d.n_shared || d.align != 1 || (!sv->h && rows_cap_of(d) > 0) || d.E > 512))
    return MOE_ERR_UNSUPPORTED;
  if (single && a->ready_test_polls < 0) return MOE_ERR_SHAPE;
  // MXFP8: the block-scaled dgrads run on the persistent engine, whole
  // 128-element contraction steps over D and over 2H; the router's GEMMs read
  // dlogits rows in 16-byte chunks
  if (mx && (d.D % 128 || d.H % 64)) return MOE_ERR_SHAPE;
  if (gr->dw_r && d.E % 8) return MOE_ERR_SHAPE;
  if (d.N == 0) {
    // no tokens, under every schedule: every weight gradient is 0 (dx,
    // dprob and dlogits hold no element)
    REQUIRE(gr->dw_gate);
    REQUIRE(gr->dw_up);
    REQUIRE(gr->dw_down);
    OPTIONAL(gr->dw_r);
    OPTIONAL(gr->db_r);
    hipStream_t s = (hipStream_t)stream;
    const int64_t Ex = experts_of(d), whd = Ex * d.H * d.D * 2;
    hipError_t e = moe::launch_zero_bytes(gr->dw_gate, whd, s);
    if (e == hipSuccess) e = moe::launch_zero_bytes(gr->dw_up, whd, s);
    if (e == hipSuccess) e = moe::launch_zero_bytes(gr->dw_down, whd, s);
    if (e == hipSuccess && gr->dw_r) e = moe::launch_zero_bytes(gr->dw_r, d.E * d.D * 2, s);
    if (e == hipSuccess && gr->dw_r && gr->db_r) e = moe::launch_zero_bytes(gr->db_r, d.E * 4, s);
    return hip_status(e);
  }
  if (mx) {
    if (mxw) {
      REQUIRE(sv->row_route);
      REQUIRE(a->x);
      const int64_t max_len = (rows_cap_of(d) + 127) / 128 * 128;   // one expert holding every row
      if (!moe::gemm_wgrad_mx_ok(d.D, d.H, max_len) || !moe::gemm_wgrad_mx_ok(d.H, d.D, max_len))
        return MOE_ERR_SHAPE;
    }
    REQUIRE(a->wdt_q);
    REQUIRE(a->wdt_s);
    REQUIRE(a->wgut_q);
    REQUIRE(a->wgut_s);
    REQUIRE(sv->xd_q);
    REQUIRE(sv->xd_s);
    OPTIONAL(sv->h_q);   // NULL: H recomputed from G and U for the down weight gradient
    if (sv->h_q) REQUIRE(sv->h_s);
  } else {
    REQUIRE(a->w_gate);
    REQUIRE(a->w_up);
    REQUIRE(a->w_down);
    REQUIRE(sv->xd);
    OPTIONAL(sv->h);   // NULL: recomputed from G and U
  }
  REQUIRE(dout);
  REQUIRE(ws);
  REQUIRE(sv->topk_prob);
  REQUIRE(sv->counts);
  REQUIRE(sv->offsets);
  REQUIRE(sv->dst_rows);
  REQUIRE(sv->g);
  REQUIRE(sv->u);
  REQUIRE(sv->y);
  REQUIRE(gr->dx);
  REQUIRE(gr->dprob);
  REQUIRE(gr->dw_gate);
  REQUIRE(gr->dw_up);
  REQUIRE(gr->dw_down);
  if (gr->dw_r) {
    REQUIRE(gr->dw_r);
    REQUIRE(sv->logits);
    REQUIRE(sv->topk_idx);
    REQUIRE(a->x);
    REQUIRE(a->w_r);
    OPTIONAL(gr->db_r);
    OPTIONAL(gr->dlogits);
  }
  const int64_t rc = rows_cap_of(d);
  const int64_t Ex = experts_of(d);
  const int32_t* shared_row0 = d.n_shared ? sv->offsets + d.E : nullptr;   // the shared expert's segment
  const size_t tb = table_bytes(rc, Ex);
  if (ws_bytes < tb + bwd_scratch_bytes(d, mx, mxw)) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  int32_t* table = (int32_t*)ws;
  char* p0 = (char*)ws + tb;
  const BwdLayout bl = bwd_layout(d, mx, mxw);
  void* dyd = p0 + bl.dyd;
  void* dxd = p0 + bl.dxd;
  void* dg = p0 + bl.dg;
  void* du = p0 + bl.du;
  const int32_t* rows_end = sv->offsets + Ex;   // rows past the last segment are never read

  hipError_t e = hipSuccess;
  if (mx) {
    uint8_t* dyq = (uint8_t*)(p0 + bl.dyq);
    uint8_t* dys = (uint8_t*)(p0 + bl.dys);
    uint8_t* guq = (uint8_t*)(p0 + bl.guq);
    uint8_t* gus = (uint8_t*)(p0 + bl.gus);
    void* hdq = p0 + bl.h;
    void* xdq = p0 + bl.xdeq;
    // down dgrad, block-scaled: dH = dY_d . (W_down^T)^T over D, the SwiGLU
    // backward and the quantization of [dG | dU] in its epilogue
    moe::GemmFwd dn{Ex, rc, d.D, d.H, sv->offsets, dyq, dys, a->wdt_q, a->wdt_s, nullptr,
                    nullptr, dg, du, nullptr, guq, gus, false};
    dn.dswiglu = true;
    dn.g = sv->g;
    dn.u = sv->u;
    // gate/up dgrad, block-scaled: dX_d = [dG | dU] . [W_gate^T | W_up^T]^T over 2H
    moe::GemmFwd gu{Ex, rc, 2 * d.H, d.D, sv->offsets, guq, gus, a->wgut_q, a->wgut_s, nullptr,
                    nullptr, dxd, nullptr, nullptr, nullptr, nullptr, false};
    if (!moe::gemm_fwd_fast_ok(dn, true) || !moe::gemm_fwd_fast_ok(gu, true)) return MOE_ERR_SHAPE;
    // dY arrives in bf16 and is quantized where it lands (KOSMOS section 3.3.2
    // step 1): in the combine backward itself when D % 128 == 0, else by a
    // pass over dY_d
    const bool fuse_q = moe::combine_bwd_quant_ok(d.D, dyq, dys);
    e = moe::launch_combine_bwd(dout, sv->dst_rows, sv->topk_prob, sv->y, d.N, d.D, d.K, dyd, gr->dprob, s,
                                shared_row0, fuse_q ? dyq : nullptr, fuse_q ? dys : nullptr);
    if (e == hipSuccess)
      e = fuse_q ? moe::launch_zero_padding(sv->counts, sv->offsets, Ex, d.D * 2, dyd, d.D, dyq, s, d.D / 32, dys)
                 : moe::launch_zero_padding(sv->counts, sv->offsets, Ex, d.D * 2, dyd, 0, nullptr, s);
    if (e == hipSuccess && !fuse_q) e = moe::launch_quantize_rows(dyd, rc, d.D, dyq, dys, s, rows_end);
    if (e == hipSuccess) e = moe::launch_gemm_fwd_fast(dn, true, table, s);
    if (e == hipSuccess) e = moe::launch_gemm_fwd_fast(gu, true, table, s);
    if (mxw) {
      // native block-scaled weight gradients on column-wise copies, each
      // quantized from its bf16 values: dY_d as it landed, H rebuilt from the
      // saved G and U, dG and dU from the down dgrad, X_d gathered from x
      const int64_t ld = bl.ldt;
      auto cp = [&](size_t o) { return (uint8_t*)(p0 + o); };
      int32_t* toff = (int32_t*)(p0 + bl.toff);
      if (e == hipSuccess) e = moe::launch_seg128_scan(sv->offsets, Ex, toff, s);
      if (e == hipSuccess) e = moe::launch_swiglu(sv->g, sv->u, rc, d.H, hdq, nullptr, nullptr, s);
      if (e == hipSuccess)
        e = moe::launch_quantize_cols_seg(dyd, d.D, sv->offsets, Ex, toff, ld, nullptr, 0, nullptr, 0, cp(bl.dyt_q),
                                          cp(bl.dyt_s), s);
      if (e == hipSuccess)
        e = moe::launch_quantize_cols_seg(hdq, d.H, sv->offsets, Ex, toff, ld, nullptr, 0, nullptr, 0, cp(bl.ht_q),
                                          cp(bl.ht_s), s);
      if (e == hipSuccess)
        e = moe::launch_quantize_cols_seg(dg, d.H, sv->offsets, Ex, toff, ld, nullptr, 0, nullptr, 0, cp(bl.dgt_q),
                                          cp(bl.dgt_s), s);
      if (e == hipSuccess)
        e = moe::launch_quantize_cols_seg(du, d.H, sv->offsets, Ex, toff, ld, nullptr, 0, nullptr, 0, cp(bl.dut_q),
                                          cp(bl.dut_s), s);
      if (e == hipSuccess)
        e = moe::launch_quantize_cols_seg(a->x, d.D, sv->offsets, Ex, toff, ld, sv->row_route, d.K, shared_row0, d.N,
                                          cp(bl.xt_q), cp(bl.xt_s), s);
      // dW_down[e] [D][H] = dY_e^T H_e; dW_gate / dW_up [H][D] = dG_e^T X_e, dU_e^T X_e
      if (e == hipSuccess)
        e = moe::launch_gemm_wgrad_mx(sv->offsets, toff, Ex, d.D, d.H, cp(bl.dyt_q), cp(bl.dyt_s), cp(bl.ht_q),
                                      cp(bl.ht_s), gr->dw_down, table, s);
      if (e == hipSuccess)
        e = moe::launch_gemm_wgrad_mx(sv->offsets, toff, Ex, d.H, d.D, cp(bl.dgt_q), cp(bl.dgt_s), cp(bl.xt_q),
                                      cp(bl.xt_s), gr->dw_gate, table, s);
      if (e == hipSuccess)
        e = moe::launch_gemm_wgrad_mx(sv->offsets, toff, Ex, d.H, d.D, cp(bl.dut_q), cp(bl.dut_s), cp(bl.xt_q),
                                      cp(bl.xt_s), gr->dw_up, table, s);
    } else {
      // weight gradients: bf16 products on the dequantized activations; in the
      // SwiGLU-recompute mode (no saved h_q) on H = silu(G) U rebuilt in bf16
      if (e == hipSuccess) {
        if (sv->h_q) e = moe::launch_dequant_rows(sv->h_q, sv->h_s, rc, d.H, rows_end, hdq, s);
        else e = moe::launch_swiglu(sv->g, sv->u, rc, d.H, hdq, nullptr, nullptr, s);
      }
      if (e == hipSuccess) e = moe::launch_dequant_rows(sv->xd_q, sv->xd_s, rc, d.D, rows_end, xdq, s);
      moe::GemmBwd wd{Ex, rc, d.H, d.D, sv->offsets, hdq, nullptr, nullptr, dyd, nullptr, nullptr,
                      nullptr, nullptr, nullptr, nullptr, false};
      if (e == hipSuccess) e = gemm_wgrad(wd, dyd, gr->dw_down, table, s);
      moe::GemmBwd wgu{Ex, rc, d.D, d.H, sv->offsets, xdq, nullptr, nullptr, dg, du, nullptr,
                       nullptr, nullptr, nullptr, nullptr, false};
      if (e == hipSuccess) e = gemm_wgrad(wgu, dg, gr->dw_gate, table, s);
      if (e == hipSuccess) e = gemm_wgrad(wgu, du, gr->dw_up, table, s);
    }
  } else if (single) {
    // the whole backward in one persistent launch (the router's too when asked)
    moe::LayerBwdSingle one{};
    one.dout = dout;
    one.dst_rows = sv->dst_rows;
    one.topk_prob = sv->topk_prob;
    one.y = sv->y;
    one.N = d.N;
    one.D = d.D;
    one.K = d.K;
    one.E = d.E;
    one.dyd = dyd;
    one.dprob = gr->dprob;
    one.down = moe::GemmBwd{Ex, rc, d.H, d.D, sv->offsets, sv->h, a->w_down, nullptr, dyd, nullptr, nullptr,
                            sv->g, sv->u, dg, du, true};
    one.gu = moe::GemmBwd{Ex, rc, d.D, d.H, sv->offsets, sv->xd, a->w_gate, a->w_up, dg, du, dxd,
                          nullptr, nullptr, nullptr, nullptr, false};
    one.dw_down = gr->dw_down;
    one.dw_gate = gr->dw_gate;
    one.dw_up = gr->dw_up;
    one.router = gr->dw_r != nullptr;
    if (one.router) {
      char* p = p0 + bl.router;
      const RouterBwdLayout l = router_bwd_layout(d);
      const bool aux = a->aux_alpha != 0.0f && gr->d_aux != 0.0f;
      one.logits = sv->logits;
      one.topk_idx = sv->topk_idx;
      one.renorm = d.renorm;
      one.dl = gr->dlogits ? gr->dlogits : (float*)(p + l.dl);
      one.dlb = (uint16_t*)(p + l.dlb);
      one.colpart = (float*)(p + l.colpart);
      one.offs = (int32_t*)(p + l.offs);
      one.offs1 = one.offs + 48;
      one.S = l.S;
      one.aux_counts = aux ? sv->counts : nullptr;
      one.aux_c = aux ? gr->d_aux * a->aux_alpha * (float)d.E / ((float)d.N * (float)d.N * (float)d.K) : 0.0f;
      one.rt = moe::GemmBwd{1, d.N, d.D, d.E, one.offs1, a->x, a->w_r, nullptr, one.dlb, nullptr, p + l.dxr,
                            nullptr, nullptr, nullptr, nullptr, false};
      one.rs = moe::GemmBwd{l.S, d.N, d.D, d.E, one.offs, a->x, a->w_r, nullptr, one.dlb, nullptr, nullptr,
                            nullptr, nullptr, nullptr, nullptr, false};
      one.part = (float*)(p + l.part);
      one.split = moe::gemm_wgrad_fast_ok(one.rs, one.dlb, one.part);
      one.dw_r = gr->dw_r;
      one.db_r = gr->db_r;
      one.dxr = p + l.dxr;
    }
    one.dxd = dxd;
    one.dx = gr->dx;
    one.status = sv->status;
    one.test_polls = a->ready_test_polls;
    if (!moe::layer_bwd_single_ok(one)) return MOE_ERR_UNSUPPORTED;
    return hip_status(moe::launch_layer_bwd_single(one, (int32_t*)(p0 + bl.single), s));
  } else {
    // SwiGLU-recompute mode: H = silu(G) U from the saved bf16 G and U, the
    // same arithmetic as GEMM1's epilogue, so it equals the forward's H bit for bit
    const void* h = sv->h ? sv->h : (const void*)(p0 + bl.h);
    e = moe::launch_combine_bwd(dout, sv->dst_rows, sv->topk_prob, sv->y, d.N, d.D, d.K, dyd, gr->dprob, s,
                                shared_row0);
    if (e == hipSuccess && !sv->h) e = moe::launch_swiglu(sv->g, sv->u, rc, d.H, (void*)h, nullptr, nullptr, s);
    if (e == hipSuccess && d.align > 1)
      e = moe::launch_zero_padding(sv->counts, sv->offsets, Ex, d.D * 2, dyd, 0, nullptr, s);
    // down: forward y = h . w_down^T  (k_dim = H, n_dim = D)
    moe::GemmBwd down{Ex, rc, d.H, d.D, sv->offsets, h, a->w_down, nullptr, dyd, nullptr, nullptr,
                      sv->g, sv->u, dg, du, true};
    if (e == hipSuccess) e = gemm_dgrad(down, table, s);
    if (e == hipSuccess) e = gemm_wgrad(down, dyd, gr->dw_down, table, s);
    // gate/up: forward g = xd . w_gate^T, u = xd . w_up^T  (k_dim = D, n_dim = H)
    moe::GemmBwd gu{Ex, rc, d.D, d.H, sv->offsets, sv->xd, a->w_gate, a->w_up, dg, du, dxd,
                    nullptr, nullptr, nullptr, nullptr, false};
    if (e == hipSuccess) e = gemm_dgrad(gu, table, s);
    if (e == hipSuccess) e = gemm_wgrad(gu, dg, gr->dw_gate, table, s);
    if (e == hipSuccess) e = gemm_wgrad(gu, du, gr->dw_up, table, s);
  }
  const void* dxr = nullptr;
  if (e == hipSuccess && gr->dw_r) {
    // router backward, after the expert backward so the fold below adds dX_r
    char* p = p0 + bl.router;
    const RouterBwdLayout l = router_bwd_layout(d);
    float* dl = gr->dlogits ? gr->dlogits : (float*)(p + l.dl);
    uint16_t* dlb = (uint16_t*)(p + l.dlb);
    int32_t* offs = (int32_t*)(p + l.offs);
    int32_t* offs1 = offs + 48;   // the block is 64 ints; the S + 1 <= 33 split offsets come first
    float* part = (float*)(p + l.part);
    float* colpart = (float*)(p + l.colpart);
    dxr = p + l.dxr;
    // the aux loss's gradient: d_aux alpha E / N * p (f - sum_j p_j f_j), f = counts / (N K)
    const bool aux = a->aux_alpha != 0.0f && gr->d_aux != 0.0f;
    const float aux_c = aux ? gr->d_aux * a->aux_alpha * (float)d.E / ((float)d.N * (float)d.N * (float)d.K) : 0.0f;
    e = moe::launch_router_bwd(sv->logits, sv->topk_idx, gr->dprob, d.N, d.E, d.K, d.renorm, dl, dlb, colpart,
                               offs, l.S, offs1, s, aux ? sv->counts : nullptr, aux_c);
    // forward L = x . w_r^T: k_dim = D, n_dim = E, one expert over all N rows
    moe::GemmBwd rt{1, d.N, d.D, d.E, offs1, a->x, a->w_r, nullptr, dlb, nullptr, (void*)dxr,
                    nullptr, nullptr, nullptr, nullptr, false};
    if (e == hipSuccess) e = gemm_dgrad(rt, table, s);
    // dW_r: the token range cut into S pseudo-experts, fp32 partials summed in order
    moe::GemmBwd rs{l.S, d.N, d.D, d.E, offs, a->x, a->w_r, nullptr, dlb, nullptr, nullptr,
                    nullptr, nullptr, nullptr, nullptr, false};
    const bool split = moe::gemm_wgrad_fast_ok(rs, dlb, part);
    if (e == hipSuccess) {
      if (split) e = moe::launch_gemm_wgrad_fast(rs, dlb, part, table, s, true);
      else e = gemm_wgrad(rt, dlb, gr->dw_r, table, s);
    }
    if (e == hipSuccess)
      e = moe::launch_router_bwd_reduce(split ? part : nullptr, l.S, d.E * d.D, (uint16_t*)gr->dw_r, colpart,
                                        (d.N + 63) / 64, d.E, gr->db_r, s);
  }
  if (e == hipSuccess)
    e = moe::launch_combine(dxd, sv->dst_rows, nullptr, d.N, d.D, d.K, gr->dx, s, dxr, shared_row0);
  return hip_status(e);
}

}  // extern "C"
