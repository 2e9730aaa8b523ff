// Persistent, self-scheduling grouped GEMM of the expert forward on bf16 MFMA
// (gfx950 v_mfma_f32_16x16x32_bf16, fp32 accumulation).
//
//   GEMM1 (DUAL): per expert e and row block, G = X_d W_gate[e]^T and
//     U = X_d W_up[e]^T share the A tile; the epilogue stores G, U (the
//     pre-activations kept for the backward) and H = bf16(silu(G) * U)
//     (KOSMOS section 3.3.1 step 3, GEMM1 with SwiGLU fused in its epilogue).
//   GEMM2 (single): Y_d = H W_down[e]^T (KOSMOS section 3.3.1 step 4).
//
// Scheduling (KOSMOS section 3.1: persistent workgroups claiming tiles from a
// device queue).  The grid is the number of workgroups that can be resident at
// once; every workgroup claims items from one atomic head counter until the
// queue is empty.  An item is (expert, n-tile, row block); inside an expert the
// row blocks of one n-tile are consecutive, so the weight tile they share is
// fetched once and served from cache to the others.  Experts with many rows
// use 256-row tiles, the others 128-row tiles (KOSMOS section 3.4 uses 256x256
// tiles; small expert batches would waste most of such a tile).  A
// one-workgroup planner builds the expert order and the item prefix sums on
// the device from the expert offsets (no host round trip), interleaving the
// two tile classes in proportion to their work so that weight-streaming tiles
// of small experts run beside the MFMA-bound tiles of large ones, and resets
// the queue head.  Which workgroup computes an item never changes its result.
//
// The MFMA main loop (direct-to-LDS operand ring) is the shared tile engine;
// eight waves per workgroup (two per SIMD).
#include "common.h"
#include "launch.h"
#include "mfma_tile.h"

namespace moe {

namespace {

constexpr int kBigRows = 256;    // experts with at least this many rows use 256-row tiles

struct FwdParams {
  const int32_t* offsets;   // [E+1]
  const int32_t* plan;      // planner output (layout below)
  int32_t* head;            // queue head counter
  int E, N, K;              // N output columns per weight, K contraction
  int n_tiles;              // ceil(N / NCOL)
  const uint16_t* a;        // [rows][K]
  const uint16_t* b0;       // [E][N][K]
  const uint16_t* b1;       // DUAL: [E][N][K]
  uint16_t* c0;             // [rows][N]  (G or Y)
  uint16_t* c1;             // DUAL: U
  uint16_t* c2;             // DUAL: H
};

// plan layout (int32): [0] total items, [1] number of listed experts L,
// [2 .. 2+L) expert ids in processing order, [2+E .. 2+E+L] item prefix sums
// (entry L = total).

// A claimed queue item, decoded: rows [m_start, min(m_start + BM, m1)) of
// expert e, output columns [n0, n0 + NCOL), tile class by the expert's rows.
struct Item {
  int e, m_start, m1, n0;
  bool big, valid;
};

// The two tile classes; both have BN = 256 (DUAL: 128 gate + 128 up columns).
template <bool DUAL>
using BigTile = tile::TileCfg<256, 256, 2, 4, 2, DUAL>;     // 2 x 64 KB ring
template <bool DUAL>
using SmallTile = tile::TileCfg<128, 256, 3, 2, 4, DUAL>;   // 3 x 48 KB ring
constexpr int kLdsBytes = 3 * (128 + 256) * tile::kRB;     // the larger ring
static_assert(kLdsBytes >= 2 * (256 + 256) * tile::kRB, "ring size");

__device__ __host__ __forceinline__ bool is_big(int rows) { return rows >= kBigRows; }

// Claim the next item from the queue and decode it (every thread gets the
// same result; li is the workgroup's position in the expert list, which only
// moves forward because each workgroup's claims increase).
template <bool DUAL>
__device__ __forceinline__ Item claim(const FwdParams& p, int* s_item, int& li) {
  if (threadIdx.x == 0) *s_item = atomicAdd(p.head, 1);
  __syncthreads();
  const int item = *s_item;
  Item it{};
  const int total = p.plan[0];
  if (item >= total) return it;
  const int L = p.plan[1];
  const int32_t* order = p.plan + 2;
  const int32_t* pref = p.plan + 2 + p.E;
  while (li + 1 < L && pref[li + 1] <= item) ++li;
  it.e = order[li];
  const int m0 = p.offsets[it.e];
  it.m1 = p.offsets[it.e + 1];
  it.big = is_big(it.m1 - m0);
  const int bm = it.big ? BigTile<DUAL>::BM : SmallTile<DUAL>::BM;
  const int nmb = (it.m1 - m0 + bm - 1) / bm;
  const int w = item - pref[li];
  const int n_t = w / nmb, mb = w - n_t * nmb;
  it.m_start = m0 + mb * bm;
  it.n0 = n_t * BigTile<DUAL>::NCOL;
  it.valid = true;
  return it;
}

// This lane's DMA source pointers for an item (rows past the expert's segment
// or columns past N load a clamped valid row and are never stored).
template <class C>
__device__ __forceinline__ void sources(const FwdParams& p, const Item& it, const uint16_t** a_src,
                                        const uint16_t** b_src) {
  using namespace tile;
  const int wave = threadIdx.x >> 6;
  const int64_t K = p.K;
  const int d_chunk = dma_chunk();
#pragma unroll
  for (int q = 0; q < C::A_INS; ++q) {
    const int row = min(it.m_start + dma_row(wave, C::A_INS, q), it.m1 - 1);
    a_src[q] = p.a + (int64_t)row * K + d_chunk * 8;
  }
#pragma unroll
  for (int q = 0; q < C::B_INS; ++q) {
    const int r = dma_row(wave, C::B_INS, q);
    const uint16_t* base = p.b0;
    int col = it.n0 + r;
    if (C::DUAL && r >= C::BN / 2) {
      base = p.b1;
      col = it.n0 + r - C::BN / 2;
    }
    col = min(col, p.N - 1);
    b_src[q] = base + ((int64_t)it.e * p.N + col) * K + d_chunk * 8;
  }
}

template <class C>
__device__ __forceinline__ void start(const FwdParams& p, uint32_t lds0, const Item& it) {
  const uint16_t* a_src[C::A_INS];
  const uint16_t* b_src[C::B_INS];
  sources<C>(p, it, a_src, b_src);
  tile::prologue<C>(lds0, a_src, b_src, p.K / tile::kBK);
}

template <class C>
__device__ __forceinline__ void epilogue(const FwdParams& p, const Item& it, const f32x4_t (&acc)[C::TM][C::TN]) {
  constexpr int TM = C::TM, TN = C::TN, WM = C::WM, WN = C::WN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N_, wn = wave % C::WAVES_N_;
  const int l16 = lane & 15, lg = lane >> 4;
  // lane holds row wm*WM + i*16 + l16, columns 4*lg .. 4*lg+3 of its
  // 16-column fragment
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = wm * WM + i * 16 + l16;
    if (it.m_start + m >= it.m1) continue;
    const int64_t row = it.m_start + m;
    if (!C::DUAL) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = it.n0 + wn * WN + j * 16 + 4 * lg;
        if (n >= p.N) continue;
        const f32x4_t a = acc[i][j];
        *reinterpret_cast<uint2*>(p.c0 + row * p.N + n) =
            make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
      }
    } else {
#pragma unroll
      for (int j = 0; j < TN / 2; ++j) {
        const int n = it.n0 + wn * (WN / 2) + j * 16 + 4 * lg;
        if (n >= p.N) continue;
        const f32x4_t a = acc[i][j], b = acc[i][j + TN / 2];
        const uint32_t gw0 = pack_bf16x2(a[0], a[1]), gw1 = pack_bf16x2(a[2], a[3]);
        const uint32_t uw0 = pack_bf16x2(b[0], b[1]), uw1 = pack_bf16x2(b[2], b[3]);
        const int64_t off = row * p.N + n;
        *reinterpret_cast<uint2*>(p.c0 + off) = make_uint2(gw0, gw1);
        *reinterpret_cast<uint2*>(p.c1 + off) = make_uint2(uw0, uw1);
        const float g0 = bf16lo(gw0), g1 = bf16hi(gw0), g2 = bf16lo(gw1), g3 = bf16hi(gw1);
        const float h0 = g0 * sigmoidf_(g0) * bf16lo(uw0);
        const float h1 = g1 * sigmoidf_(g1) * bf16hi(uw0);
        const float h2 = g2 * sigmoidf_(g2) * bf16lo(uw1);
        const float h3 = g3 * sigmoidf_(g3) * bf16hi(uw1);
        *reinterpret_cast<uint2*>(p.c2 + off) = make_uint2(pack_bf16x2(h0, h1), pack_bf16x2(h2, h3));
      }
    }
  }
}

// Run the current item (its prologue already issued), then claim the next
// one and issue its prologue before storing this item's outputs, so the
// loads of the next tile overlap this epilogue.
template <class C, bool DUAL>
__device__ __forceinline__ Item run_item(const FwdParams& p, const uint8_t* smem, uint32_t lds0, int* s_item,
                                         int& li, const Item& it) {
  const uint16_t* a_src[C::A_INS];
  const uint16_t* b_src[C::B_INS];
  sources<C>(p, it, a_src, b_src);
  f32x4_t acc[C::TM][C::TN];
  tile::mainloop<C>(smem, lds0, a_src, b_src, p.K / tile::kBK, acc);
  const Item next = claim<DUAL>(p, s_item, li);
  if (next.valid) {
    if (next.big) start<BigTile<DUAL>>(p, lds0, next);
    else start<SmallTile<DUAL>>(p, lds0, next);
  }
  epilogue<C>(p, it, acc);
  return next;
}

template <bool DUAL>
__global__ __launch_bounds__(512) void gemm_fwd_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLdsBytes];
  __shared__ int s_item;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  int li = 0;
  Item it = claim<DUAL>(p, &s_item, li);
  if (!it.valid) return;
  if (it.big) start<BigTile<DUAL>>(p, lds0, it);
  else start<SmallTile<DUAL>>(p, lds0, it);
  while (it.valid) {
    if (it.big) it = run_item<BigTile<DUAL>, DUAL>(p, smem, lds0, &s_item, li, it);
    else it = run_item<SmallTile<DUAL>, DUAL>(p, smem, lds0, &s_item, li, it);
  }
}

// Planner: one workgroup of 1024 threads (E <= 1024).  Each expert with rows
// gets ceil(rows / BM) * n_tiles items, BM by its tile class.  The experts of
// each class keep ascending id; the two classes are merged by the midpoint of
// each expert's items within its class, so both progress at the same rate.
__global__ __launch_bounds__(1024) void plan_fwd_kernel(const int32_t* __restrict__ offsets, int E, int n_tiles,
                                                        int32_t* __restrict__ plan, int32_t* __restrict__ head) {
  __shared__ int s_w0[16], s_w1[16], s_tot[2];
  __shared__ float s_key[1024];
  __shared__ int s_items[1024], s_ids[1024], s_pref[16];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  int items = 0, big = 0;
  if (t < E) {
    const int m = offsets[t + 1] - offsets[t];
    big = is_big(m);
    const int bm = big ? BigTile<true>::BM : SmallTile<true>::BM;
    items = m > 0 ? ((m + bm - 1) / bm) * n_tiles : 0;
  }
  int i0 = big ? 0 : items, i1 = big ? items : 0;   // per-class inclusive scans
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int a = __shfl_up(i0, o, 64), b = __shfl_up(i1, o, 64);
    if (lane >= o) { i0 += a; i1 += b; }
  }
  if (lane == 63) { s_w0[wv] = i0; s_w1[wv] = i1; }
  __syncthreads();
  if (t == 0) {
    int r0 = 0, r1 = 0;
    for (int w = 0; w < 16; ++w) {
      const int a = s_w0[w], b = s_w1[w];
      s_w0[w] = r0; s_w1[w] = r1;
      r0 += a; r1 += b;
    }
    s_tot[0] = r0; s_tot[1] = r1;
  }
  __syncthreads();
  const int pre = big ? (i1 - items + s_w1[wv]) : (i0 - items + s_w0[wv]);
  const int tot = s_tot[big];
  s_key[t] = (items > 0) ? ((float)pre + 0.5f * (float)items) / (float)tot : 2.0f;
  __syncthreads();
  if (items > 0) {
    const float k = s_key[t];
    int rank = 0;
    for (int f = 0; f < E; ++f) {
      const float kf = s_key[f];
      rank += (kf < k) || (kf == k && f < t);
    }
    s_items[rank] = items;
    s_ids[rank] = t;
  }
  const int L = __syncthreads_count(items > 0);
  // exclusive scan of the items in rank order
  const int v = t < L ? s_items[t] : 0;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int a = __shfl_up(inc, o, 64);
    if (lane >= o) inc += a;
  }
  if (lane == 63) s_pref[wv] = inc;
  __syncthreads();
  if (t == 0) {
    int r = 0;
    for (int w = 0; w < 16; ++w) { const int a = s_pref[w]; s_pref[w] = r; r += a; }
    plan[0] = r;
    plan[1] = L;
    plan[2 + E + L] = r;
    *head = 0;
  }
  __syncthreads();
  if (t < L) {
    plan[2 + t] = s_ids[t];
    plan[2 + E + t] = inc - v + s_pref[wv];
  }
}

template <bool DUAL>
hipError_t run_fwd(FwdParams p, int32_t* plan, hipStream_t s) {
  plan_fwd_kernel<<<1, 1024, 0, s>>>(p.offsets, p.E, p.n_tiles, plan, p.head);
  auto kern = gemm_fwd_kernel<DUAL>;
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err == hipSuccess) err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 512, 0);
  if (err != hipSuccess) return err;
  if (per_cu < 1) per_cu = 1;
  kern<<<cus * per_cu, 512, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

size_t gemm_fwd_plan_ints(int64_t E) { return (size_t)(4 + 2 * E + 64); }

bool gemm_fwd_fast_ok(int64_t k_dim, int64_t n_dim) { return k_dim % tile::kBK == 0 && n_dim % 16 == 0; }

hipError_t launch_gemm_fwd_fast(const GemmFwd& f, int32_t* ws, hipStream_t s) {
  FwdParams p{};
  p.offsets = f.offsets;
  p.E = (int)f.E;
  p.N = (int)f.n_dim;
  p.K = (int)f.k_dim;
  p.a = (const uint16_t*)f.a;
  p.b0 = (const uint16_t*)f.b0;
  p.b1 = (const uint16_t*)f.b1;
  p.c0 = (uint16_t*)f.c0;
  p.c1 = (uint16_t*)f.c1;
  p.c2 = (uint16_t*)f.act;
  p.head = ws;
  int32_t* plan = ws + 16;
  p.plan = plan;
  const int ncol = f.swiglu ? BigTile<true>::NCOL : BigTile<false>::NCOL;
  p.n_tiles = (p.N + ncol - 1) / ncol;
  return f.swiglu ? run_fwd<true>(p, plan, s) : run_fwd<false>(p, plan, s);
}

}  // namespace moe
