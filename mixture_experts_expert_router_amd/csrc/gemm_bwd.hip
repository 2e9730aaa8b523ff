// Persistent grouped GEMMs of the expert backward on bf16 MFMA (KOSMOS section
// 3.3.2; OLMo-core Appendix A, A.1 and A.13: the adjoints of the grouped
// forward products).  For a forward product c = a . b[e]^T per expert
// (a [rows][k_dim], b [E][n_dim][k_dim], c [rows][n_dim]):
//
//   dgrad  da[r][k] = sum_n dc[r][n] b[e][n][k]  (+ dc1[r][n] b1[e][n][k])
//          The weight is read k-major (its rows are the contraction), the
//          upstream gradient row-major; the optional second product
//          continues the same contraction (the gate/up dgrad sums
//          dG W_gate + dU W_up in one accumulator).  The SwiGLU-backward
//          epilogue turns dH into dG, dU with the saved G, U (down dgrad).
//   wgrad  db[e][n][k] = sum_{r in e} dc[r][n] a[r][k]
//          Both operands are contracted over the expert's rows, so both are
//          read k-major; the contraction length is the expert's row count.
//          The last step's rows past the segment reload its last row and the
//          B tile's copies are zeroed in LDS, so they add nothing.
//
// Both run on the shared tile engine (direct-to-LDS ring, k-major fragments
// through transposing LDS reads).  dgrad items are row blocks of expert
// segments and use the row scheduler of the forward GEMMs; wgrad items are
// (expert, output row tile, output column tile), experts with the most rows
// first so the longest items do not trail, on the same per-XCD queues.
#include "common.h"
#include "launch.h"
#include "mfma_tile.h"
#include "sched.h"
#include "permute_dev.h"
#include "router_dev.h"

namespace moe {

namespace {

using namespace sched;
using tile::kRB;

// ---------------------------------------------------------------- dgrad ----

struct DgradParams {
  const int32_t* offsets;   // [E+1]
  const int32_t* plan;      // row-scheduler plan
  int32_t* head;            // queue heads, kHeadStride apart
  int E, N, K;              // N output columns (forward k_dim), K contraction (forward n_dim)
  int nk, n_tiles;          // steps per product, ceil(N / 256)
  bool kcat;                // second product present
  const uint8_t* a0;        // dc0 [rows][K]
  const uint8_t* a1;        // dc1 [rows][K] (kcat)
  const uint8_t* b0;        // b0 [E][K][N]
  const uint8_t* b1;        // b1 [E][K][N] (kcat)
  uint16_t* c0;             // da, or dG [rows][N]
  uint16_t* c1;             // dU (SwiGLU backward)
  const uint16_t* g;        // saved G [rows][N] (SwiGLU backward)
  const uint16_t* u;        // saved U
};

using DgBig = tile::TileCfg<256, 256, 2, 4, 2, false, false, false, true>;     // 2 x 64 KB
using DgSmall = tile::TileCfg<128, 256, 3, 2, 4, false, false, false, true>;   // 3 x 48 KB
constexpr int kDgLds = DgSmall::LDS > DgBig::LDS ? DgSmall::LDS : DgBig::LDS;

template <class C>
__device__ __forceinline__ void sources_dg(const DgradParams& p, const Item& it, tile::SrcB<C>& src) {
  using namespace tile;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t RB = (int64_t)p.K * 2;
  const int d_chunk = dma_chunk();
  src.a[0] = uniform_ptr(p.a0 + (int64_t)it.m_start * RB);
  src.a[1] = uniform_ptr((p.kcat ? p.a1 : p.a0) + (int64_t)it.m_start * RB);
#pragma unroll
  for (int q = 0; q < C::A_INS; ++q) {
    const int row = min(it.m_start + dma_row(wave, C::A_INS, q), it.m1 - 1);
    src.a_off[q] = (uint32_t)((row - it.m_start) * RB + d_chunk * 16);
  }
  const int64_t ws = (int64_t)p.K * p.N * 2;   // bytes per expert's weight
  src.b[0] = uniform_ptr(p.b0 + (int64_t)it.e * ws);
  src.b[1] = uniform_ptr((p.kcat ? p.b1 : p.b0) + (int64_t)it.e * ws);
  src.b_rs = p.N * 2;
  src.b_lim = p.K - 1;
#pragma unroll
  for (int q = 0; q < C::B_INS; ++q) {
    const int g = wave * C::B_INS + q;
    const int x = min(it.n0 + (g >> 3) * 64 + tchunk_of(g) * 8, p.N - 8);
    src.b_off[q] = (uint32_t)(x * 2);
  }
  src.a_rs = 0;
  src.a_lim = 0;
  src.nk1 = p.nk;
}

template <class C, bool SWB>
__device__ __forceinline__ void epilogue_dg(const DgradParams& p, const Item& it, const f32x4_t (&acc)[C::TM][C::TN]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N_, wn = wave % C::WAVES_N_;
  const int l16 = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    const int64_t row = it.m_start + wm * C::WM + i * 16 + l16;
    if (row >= it.m1) continue;
    if constexpr (!SWB) {
      // 16-byte stores of fragment pairs (frag_pair_16b); N % 16 == 0
      static_assert(C::TN % 2 == 0, "fragment pairs");
      const bool odd = lg & 1;
#pragma unroll
      for (int j = 0; j < C::TN; j += 2) {
        const f32x4_t a = acc[i][j], b = acc[i][j + 1];
        const uint4 v = frag_pair_16b(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                                      pack_bf16x2(b[2], b[3]), odd);
        const int n = it.n0 + wn * C::WN + (j + (odd ? 1 : 0)) * 16 + 8 * (lg >> 1);
        if (n >= p.N) continue;
        *reinterpret_cast<uint4*>(p.c0 + row * p.N + n) = v;
      }
    } else {
      // fragment pairs in the 16-byte layout of frag_pair_16b: the lane's 8
      // columns of dH come from its own 4 and its partner's 4 (lane ^ 16),
      // and G, U, dG, dU move as 16 bytes per lane.  The saved G and U of the
      // whole fragment row are loaded first, so their loads overlap.
      static_assert(C::TN % 2 == 0, "fragment pairs");
      const bool odd = lg & 1;
      uint4 gv[C::TN / 2], uv[C::TN / 2];
#pragma unroll
      for (int jp = 0; jp < C::TN / 2; ++jp) {
        const int n = it.n0 + wn * C::WN + (2 * jp + (odd ? 1 : 0)) * 16 + 8 * (lg >> 1);
        gv[jp] = uv[jp] = make_uint4(0, 0, 0, 0);
        if (n < p.N) {
          gv[jp] = ldg16(p.g + row * p.N + n);
          uv[jp] = ldg16(p.u + row * p.N + n);
        }
      }
#pragma unroll
      for (int jp = 0; jp < C::TN / 2; ++jp) {
        const f32x4_t a = acc[i][2 * jp], b = acc[i][2 * jp + 1];
        float dh[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float r = __shfl_xor(odd ? a[q] : b[q], 16, 64);
          dh[q] = odd ? r : a[q];
          dh[4 + q] = odd ? b[q] : r;
        }
        const int n = it.n0 + wn * C::WN + (2 * jp + (odd ? 1 : 0)) * 16 + 8 * (lg >> 1);
        if (n >= p.N) continue;
        const uint32_t gw[4] = {gv[jp].x, gv[jp].y, gv[jp].z, gv[jp].w};
        const uint32_t uw[4] = {uv[jp].x, uv[jp].y, uv[jp].z, uv[jp].w};
        uint32_t dgw[4], duw[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // dH; dG = dH U s (1 + G (1 - s)), dU = dH G s with s = sigmoid(G)
          const float g0 = bf16lo(gw[w]), g1 = bf16hi(gw[w]), u0 = bf16lo(uw[w]), u1 = bf16hi(uw[w]);
          const float s0 = sigmoidf_(g0), s1 = sigmoidf_(g1);
          dgw[w] = pack_bf16x2(dh[2 * w] * u0 * s0 * (1.0f + g0 * (1.0f - s0)),
                               dh[2 * w + 1] * u1 * s1 * (1.0f + g1 * (1.0f - s1)));
          duw[w] = pack_bf16x2(dh[2 * w] * g0 * s0, dh[2 * w + 1] * g1 * s1);
        }
        const int64_t off = row * p.N + n;
        stg16(p.c0 + off, make_uint4(dgw[0], dgw[1], dgw[2], dgw[3]));
        stg16(p.c1 + off, make_uint4(duw[0], duw[1], duw[2], duw[3]));
      }
    }
  }
}

__device__ __forceinline__ Item claim_dg(const DgradParams& p, int* s_item, int& li, int xcd) {
  return claim_rows(p.plan, p.offsets, p.head, p.E, p.n_tiles, 256, s_item, li, xcd);
}

template <class C>
__device__ __forceinline__ void start_dg(const DgradParams& p, uint32_t lds0, const Item& it) {
  tile::SrcB<C> src;
  sources_dg<C>(p, it, src);
  tile::prologue_b<C>(lds0, src, p.kcat ? 2 * p.nk : p.nk);
}

template <class C, bool SWB>
__device__ __forceinline__ Item run_dg(const DgradParams& p, const uint8_t* smem, uint32_t lds0, int* s_item, int& li,
                                       int xcd, const Item& it) {
  tile::SrcB<C> src;
  sources_dg<C>(p, it, src);
  f32x4_t acc[C::TM][C::TN];
  tile::mainloop_b<C>(smem, lds0, src, p.kcat ? 2 * p.nk : p.nk, 64, acc);
  const Item next = claim_dg(p, s_item, li, xcd);
  if (next.valid) {
    if (next.big) start_dg<DgBig>(p, lds0, next);
    else start_dg<DgSmall>(p, lds0, next);
  }
  epilogue_dg<C, SWB>(p, it, acc);
  return next;
}

// A workgroup's share of a dgrad queue: items until the queue is empty.
template <bool SWB>
__device__ __forceinline__ void dgrad_loop(const DgradParams& p, const uint8_t* smem, uint32_t lds0, int* s_item) {
  const int xcd = xcd_id();
  int li = 0;
  Item it = claim_dg(p, s_item, li, xcd);
  if (!it.valid) return;
  if (it.big) start_dg<DgBig>(p, lds0, it);
  else start_dg<DgSmall>(p, lds0, it);
  while (it.valid) {
    if (it.big) it = run_dg<DgBig, SWB>(p, smem, lds0, s_item, li, xcd, it);
    else it = run_dg<DgSmall, SWB>(p, smem, lds0, s_item, li, xcd, it);
  }
}

template <bool SWB>
__global__ __launch_bounds__(512) void gemm_dgrad_kernel(DgradParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kDgLds];
  __shared__ int s_item;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  dgrad_loop<SWB>(p, smem, lds0, &s_item);
}

// ---------------------------------------------------------------- wgrad ----

struct WgradParams {
  const int32_t* offsets;   // [E+1]
  const int32_t* plan;      // [0] total items, [1 ..] expert order (most rows first)
  int32_t* head;            // queue heads, kHeadStride apart
  int E, M, N;              // per expert: output rows M (forward n_dim), columns N (forward k_dim)
  int m_tiles, n_tiles;
  const uint8_t* a;         // dc [rows][M]
  const uint8_t* b;         // forward operand [rows][N]
  void* c;                  // db [E][M][N], bf16 (or fp32 when f32)
  bool f32;
};

using WgTile = tile::TileCfg<256, 256, 2, 4, 2, false, false, true, true>;   // 2 x 64 KB

struct WgItem {
  int e, r0, rows, m0, n0, idx;   // idx: the item's index within its expert
  bool valid;
};

__device__ __forceinline__ WgItem claim_wg(const WgradParams& p, int* s_item, int xcd) {
  const int item = claim_global(p.head, p.plan[0], s_item, xcd);
  WgItem it{};
  if (item < 0) return it;
  const int per_e = p.m_tiles * p.n_tiles;
  const int ei = item / per_e;
  it.e = p.plan[1 + ei];
  it.r0 = p.offsets[it.e];
  it.rows = p.offsets[it.e + 1] - it.r0;
  int mt, nt;
  it.idx = item - ei * per_e;
  superblock_decode(it.idx, p.m_tiles, p.n_tiles, mt, nt);
  it.m0 = mt * WgTile::BM;
  it.n0 = nt * WgTile::BN;
  it.valid = true;
  return it;
}

__device__ __forceinline__ void sources_wg(const WgradParams& p, const WgItem& it, tile::SrcB<WgTile>& src) {
  using namespace tile;
  using C = WgTile;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  src.a[0] = src.a[1] = uniform_ptr(p.a + (int64_t)it.r0 * p.M * 2);
  src.b[0] = src.b[1] = uniform_ptr(p.b + (int64_t)it.r0 * p.N * 2);
  src.a_rs = p.M * 2;
  src.b_rs = p.N * 2;
  src.a_lim = src.b_lim = it.rows - 1;
#pragma unroll
  for (int q = 0; q < C::A_INS; ++q) {
    const int g = wave * C::A_INS + q;
    src.a_off[q] = (uint32_t)(min(it.m0 + (g >> 3) * 64 + tchunk_of(g) * 8, p.M - 8) * 2);
  }
#pragma unroll
  for (int q = 0; q < C::B_INS; ++q) {
    const int g = wave * C::B_INS + q;
    src.b_off[q] = (uint32_t)(min(it.n0 + (g >> 3) * 64 + tchunk_of(g) * 8, p.N - 8) * 2);
  }
  src.nk1 = 1 << 30;
}

__device__ __forceinline__ int wg_steps(const WgItem& it) { return (it.rows + 63) / 64; }

__device__ __forceinline__ void epilogue_wg(const WgradParams& p, const WgItem& it,
                                            const f32x4_t (&acc)[WgTile::TM][WgTile::TN]) {
  using C = WgTile;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N_, wn = wave % C::WAVES_N_;
  const int l16 = lane & 15, lg = lane >> 4;
  const int64_t cbase = (int64_t)it.e * p.M * p.N;
  if (p.f32) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      const int m = it.m0 + wm * C::WM + i * 16 + l16;
      if (m >= p.M) continue;
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        const int n = it.n0 + wn * C::WN + j * 16 + 4 * lg;
        if (n >= p.N) continue;
        const f32x4_t a = acc[i][j];
        *reinterpret_cast<float4*>(static_cast<float*>(p.c) + cbase + (int64_t)m * p.N + n) =
            make_float4(a[0], a[1], a[2], a[3]);
      }
    }
    return;
  }
  // bf16: 16-byte stores of fragment pairs (frag_pair_16b); N % 16 == 0, so
  // a fragment is all in or all out
  const bool odd = lg & 1;
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    const int m = it.m0 + wm * C::WM + i * 16 + l16;
#pragma unroll
    for (int j = 0; j < C::TN; j += 2) {
      const f32x4_t a = acc[i][j], b = acc[i][j + 1];
      const uint4 v = frag_pair_16b(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                                    pack_bf16x2(b[2], b[3]), odd);
      const int n = it.n0 + wn * C::WN + (j + (odd ? 1 : 0)) * 16 + 8 * (lg >> 1);
      if (m >= p.M || n >= p.N) continue;
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.c) + cbase + (int64_t)m * p.N + n) = v;
    }
  }
}

// An expert without rows has a zero gradient.  Its items do not store tiles:
// item idx clears bytes [idx, idx + 1) x (one tile's bytes) of the expert's
// dW as a flat range, 16 bytes per lane, so every wave writes whole
// contiguous kilobytes (the expert's items cover at least its M x N values).
__device__ __forceinline__ void zero_wg(const WgradParams& p, const WgItem& it) {
  const int64_t esz = p.f32 ? 4 : 2;
  const int64_t total = (int64_t)p.M * p.N * esz;   // a multiple of 32 bytes (N % 16 == 0)
  const int64_t chunk = (int64_t)WgTile::BM * WgTile::BN * esz;
  const int64_t c0 = (int64_t)it.idx * chunk;
  const int64_t c1 = min(c0 + chunk, total);
  uint8_t* base = static_cast<uint8_t*>(p.c) + (int64_t)it.e * total;
  for (int64_t off = c0 + (int64_t)threadIdx.x * 16; off < c1; off += (int64_t)blockDim.x * 16)
    *reinterpret_cast<uint4*>(base + off) = make_uint4(0, 0, 0, 0);
}

// Items are claimed one ahead and their steps stream through the ring
// without a drain between tiles: a tile with few rows (one or two steps)
// would otherwise pay a claim, a full load latency and its stores in series.
// Tiles of experts without rows have no steps: they issue no loads and clear
// a flat range of the expert's gradient, and the tile after one issues its
// own first step.
__device__ __forceinline__ void wgrad_loop(const WgradParams& p, const uint8_t* smem, uint32_t lds0, int* s_item) {
  const int xcd = xcd_id();
  WgItem it = claim_wg(p, s_item, xcd);
  if (!it.valid) return;
  __syncthreads();   // every wave has read s_item before it is reused
  WgItem next = claim_wg(p, s_item, xcd);
  tile::SrcB<WgTile> src;
  sources_wg(p, it, src);
  bool issued = false;   // step 0 of `it` is in the ring at position g0
  int g0 = 0;
  while (it.valid) {
    const int nk = wg_steps(it);
    // the stage at g0 was last read two steps back, before the previous
    // tile's last barrier, so it is free
    if (nk > 0 && !issued) tile::issue_step_b_at<WgTile>(lds0, src, 0, g0 & 1);
    const bool stream = nk > 0 && next.valid && wg_steps(next) > 0;
    tile::SrcB<WgTile> ns;
    if (next.valid) sources_wg(p, next, ns);
    f32x4_t acc[WgTile::TM][WgTile::TN];
    tile::mainloop_b_stream<WgTile>(smem, lds0, src, nk, it.rows - 64 * (nk - 1), ns, stream, g0, acc);
    // claim the tile after next while next's first step is in flight
    const WgItem after = next.valid ? claim_wg(p, s_item, xcd) : WgItem{};
    if (nk > 0) epilogue_wg(p, it, acc);
    else zero_wg(p, it);
    g0 += nk;
    issued = stream;
    it = next;
    src = ns;
    next = after;
  }
}

__global__ __launch_bounds__(512) void gemm_wgrad_kernel(WgradParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[WgTile::LDS];
  __shared__ int s_item;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  wgrad_loop(p, smem, lds0, &s_item);
}

// Expert order for wgrad: most rows first (ties: lower id), one workgroup
// (E <= its thread count); s_rows: one int of LDS per thread.
__device__ __forceinline__ void plan_wgrad_body(const int32_t* __restrict__ offsets, int E, int per_e,
                                                int32_t* __restrict__ plan, int32_t* __restrict__ head, int* s_rows) {
  const int t = threadIdx.x;
  const int rows = t < E ? offsets[t + 1] - offsets[t] : -1;
  s_rows[t] = rows;
  __syncthreads();
  if (t < E) {
    int rank = 0;
    for (int f = 0; f < E; ++f) {
      const int rf = s_rows[f];
      rank += (rf > rows) || (rf == rows && f < t);
    }
    plan[1 + rank] = t;
  }
  if (t == 0) plan[0] = E * per_e;
  if (t < kXcds) head[t * kHeadStride] = 0;
}

__global__ __launch_bounds__(1024) void plan_wgrad_kernel(const int32_t* __restrict__ offsets, int E, int per_e,
                                                          int32_t* __restrict__ plan, int32_t* __restrict__ head) {
  __shared__ int s_rows[1024];
  plan_wgrad_body(offsets, E, per_e, plan, head, s_rows);
}

// ---------------------------------------------------------- MXFP8 wgrad ----
// Native block-scaled weight gradient (OLMo-core Appendix A, A.15; KOSMOS
// section 3.3.2 step 1: the operands' column-wise copies quantized from their
// bf16 values):  db[e][m][n] = sum over the rows r of expert e of
// aT[m][r] bT[n][r] (eq. 87).  The copies hold one contiguous block per
// expert (quantize_cols_seg_kernel): expert e's aT is [M][len128] E4M3 at byte
// M * toff[e] with scales [M][len128 / 32] at M * toff[e] / 32 (bT likewise
// with N), len128 = its rows rounded up to 128, the columns past its rows
// zero, so whole 128-column steps contract exactly its rows.  Items are
// (expert, 256-row tile of db, 256-column tile) on the wgrad planner's order
// and queues; an expert without rows clears its db.

struct WgradMxParams {
  const int32_t* offsets;   // [E+1], row segments (multiples of 32)
  const int32_t* toff;      // [E+1], the copies' block offsets (columns)
  const int32_t* plan;      // wgrad planner output
  int32_t* head;            // queue heads
  int E, M, N, m_tiles, n_tiles;
  const uint8_t* aq;        // the copies of aT (width M) and bT (width N)
  const uint8_t* as;
  const uint8_t* bq;
  const uint8_t* bs;
  uint16_t* c;              // [E][M][N] bf16
};

using WmxTile = tile::TileCfg<256, 256, 2, 4, 2, false, true>;   // 2 x 64 KB ring + scale groups

struct WmxItem {
  int e, t0, len, m0, n0, idx;   // the expert's block: columns [t0, t0 + len) of the copies
  bool valid;
};

__device__ __forceinline__ WmxItem claim_wmx(const WgradMxParams& p, int* s_item, int xcd) {
  const int item = claim_global(p.head, p.plan[0], s_item, xcd);
  WmxItem it{};
  if (item < 0) return it;
  const int per_e = p.m_tiles * p.n_tiles;
  const int ei = item / per_e;
  it.e = p.plan[1 + ei];
  it.t0 = p.toff[it.e];
  it.len = p.toff[it.e + 1] - it.t0;
  int mt, nt;
  it.idx = item - ei * per_e;
  superblock_decode(it.idx, p.m_tiles, p.n_tiles, mt, nt);
  it.m0 = mt * WmxTile::BM;
  it.n0 = nt * WmxTile::BN;
  it.valid = true;
  return it;
}

__device__ __forceinline__ int wmx_steps(const WmxItem& it) { return it.len / tile::kRB; }

// DMA sources (rows past M or N reload the last row and are never stored);
// scale load q of a wave: A rows, then B rows, then padding rows that reload
// the tile's first A rows.
__device__ __forceinline__ void sources_wmx(const WgradMxParams& p, const WmxItem& it, tile::Src<WmxTile>& src) {
  using namespace tile;
  using C = WmxTile;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int d_chunk = dma_chunk();
  src.a = uniform_ptr(p.aq + (int64_t)p.M * it.t0);
  src.b = uniform_ptr(p.bq + (int64_t)p.N * it.t0);
#pragma unroll
  for (int q = 0; q < C::A_INS; ++q)
    src.a_off[q] = (uint32_t)(min(it.m0 + dma_row(wave, C::A_INS, q), p.M - 1) * it.len + d_chunk * 16);
#pragma unroll
  for (int q = 0; q < C::B_INS; ++q)
    src.b_off[q] = (uint32_t)(min(it.n0 + dma_row(wave, C::B_INS, q), p.N - 1) * it.len + d_chunk * 16);
  src.s_ks = it.len / 32;
#pragma unroll
  for (int q = 0; q < C::SCI; ++q) {
    const int r0 = wave * C::SRW + q * 16;
    if (r0 < C::BM || r0 >= C::BM + C::BN) {
      src.s[q] = uniform_ptr(p.as + (int64_t)p.M * it.t0 / 32);
      src.s_row0[q] = it.m0 + (r0 < C::BM ? r0 : 0);
      src.s_lim[q] = p.M - 1;
    } else {
      src.s[q] = uniform_ptr(p.bs + (int64_t)p.N * it.t0 / 32);
      src.s_row0[q] = __builtin_amdgcn_readfirstlane(it.n0 + r0 - C::BM);
      src.s_lim[q] = p.N - 1;
    }
  }
}

__device__ __forceinline__ void epilogue_wmx(const WgradMxParams& p, const WmxItem& it,
                                             const f32x4_t (&acc)[WmxTile::TM][WmxTile::TN]) {
  using C = WmxTile;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N_, wn = wave % C::WAVES_N_;
  const int l16 = lane & 15, lg = lane >> 4;
  const bool odd = lg & 1;
  uint16_t* cb = p.c + (int64_t)it.e * p.M * p.N;
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    const int m = it.m0 + wm * C::WM + i * 16 + l16;
#pragma unroll
    for (int j = 0; j < C::TN; j += 2) {
      const f32x4_t a = acc[i][j], b = acc[i][j + 1];
      const uint4 v = frag_pair_16b(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                                    pack_bf16x2(b[2], b[3]), odd);
      const int n = it.n0 + wn * C::WN + (j + (odd ? 1 : 0)) * 16 + 8 * (lg >> 1);
      if (m >= p.M || n >= p.N) continue;
      *reinterpret_cast<uint4*>(cb + (int64_t)m * p.N + n) = v;
    }
  }
}

// an expert without rows: item idx clears its share of the expert's db as a
// flat range (the expert's items cover at least its M x N values)
__device__ __forceinline__ void zero_wmx(const WgradMxParams& p, const WmxItem& it) {
  const int64_t total = (int64_t)p.M * p.N * 2;
  const int64_t chunk = (int64_t)WmxTile::BM * WmxTile::BN * 2;
  const int64_t c0 = (int64_t)it.idx * chunk;
  const int64_t c1 = min(c0 + chunk, total);
  uint8_t* base = reinterpret_cast<uint8_t*>(p.c) + (int64_t)it.e * total;
  for (int64_t off = c0 + (int64_t)threadIdx.x * 16; off < c1; off += (int64_t)blockDim.x * 16)
    *reinterpret_cast<uint4*>(base + off) = make_uint4(0, 0, 0, 0);
}

// Items are claimed one ahead: the claim of the item after next (an atomic
// round trip) overlaps the next item's first loads and this item's stores.
__global__ __launch_bounds__(512) void gemm_wgrad_mx_kernel(WgradMxParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[WmxTile::LDS];
  __shared__ int s_item;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  const int xcd = xcd_id();
  WmxItem it = claim_wmx(p, &s_item, xcd);
  if (!it.valid) return;
  __syncthreads();   // every wave has read s_item before it is reused
  WmxItem next = claim_wmx(p, &s_item, xcd);
  if (wmx_steps(it) > 0) {
    tile::Src<WmxTile> src;
    sources_wmx(p, it, src);
    tile::prologue<WmxTile>(lds0, src, wmx_steps(it));
  }
  while (it.valid) {
    const int nk = wmx_steps(it);
    f32x4_t acc[WmxTile::TM][WmxTile::TN];
    if (nk > 0) {
      tile::Src<WmxTile> src;
      sources_wmx(p, it, src);
      tile::mainloop_mx<WmxTile>(smem, lds0, src, nk, acc);   // ends with a barrier
    } else {
      __syncthreads();   // every wave has read s_item before the claim below rewrites it
    }
    if (next.valid && wmx_steps(next) > 0) {
      tile::Src<WmxTile> ns;
      sources_wmx(p, next, ns);
      tile::prologue<WmxTile>(lds0, ns, wmx_steps(next));
    }
    const WmxItem after = next.valid ? claim_wmx(p, &s_item, xcd) : WmxItem{};
    if (nk > 0) epilogue_wmx(p, it, acc);
    else zero_wmx(p, it);
    it = next;
    next = after;
  }
}

// ---------------------------------------------------------------------------
// Single-launch layer backward (KOSMOS section 3.3 and Figure 6: one launch
// per direction; section 3.3.2 steps 1-4), on one GPU.  One persistent
// workgroup per CU runs four phases, each ended by a grid barrier (every
// workgroup adds to a counter after an agent-scope release and waits,
// bounded, until all have):
//   0. the combine backward (dY_d rows and dprob), 8 tokens per item, and
//      the plans of the GEMM queues (a workgroup each);
//   1. the down dgrad queue (SwiGLU backward in its epilogue: dG, dU), the
//      down wgrad queue, then the router backward blocks (dlogits);
//   2. the gate/up dgrad queue (dX_d), the gate and up wgrad queues, the
//      router's dX_r and dW_r queues;
//   3. the router's dW_r and db_r reductions and the fold (dx, plus dX_r).
// A workgroup drains the queues of a phase one after another, so a queue's
// tail overlaps the next queue's items.  Each item computes what it does in
// its separate launch, so the gradients are bitwise the staged backward's.
// ---------------------------------------------------------------------------

struct SingleBwdParams {
  const uint16_t* dout;       // [N][D]
  const int32_t* dst_rows;    // [N][K]
  const float* topk_prob;     // [N][K]
  const uint16_t* y;          // saved Y [rows][D]
  int N, D, K, E;
  uint16_t* dyd;              // dY_d [rows][D]
  float* dprob;               // [N][K]
  DgradParams dg_dn, dg_gu, dg_rt;
  WgradParams wg_dn, wg_g, wg_u, wg_rt;
  int router;                 // the router backward is on
  int rt_split;               // dW_r through fp32 token-split partials
  const float* logits;
  const int32_t* topk_idx;
  int renorm;
  float* dl;                  // dlogits fp32 [N][E]
  uint16_t* dlb;              // and bf16
  float* colpart;             // [ceil(N / 64)][E]
  int32_t* offs;              // S + 1 token-split offsets
  int S;
  int32_t* offs1;             // {0, N}
  const int32_t* aux_counts;
  float aux_c;
  int rb_blocks;              // ceil(N / 64) router backward blocks
  uint16_t* dw_r;
  float* db_r;
  const uint16_t* dxd;        // dX_d [rows][D]
  uint16_t* dx;               // [N][D]
  const uint16_t* dxr;        // dX_r [N][D] or null
  int32_t* bar;               // [3] barriers, [3]: router block queue (zeroed before the launch)
  int32_t* status;
  int polls, publish;
};

constexpr int kSbLds = kDgLds > WgTile::LDS ? kDgLds : WgTile::LDS;
static_assert(kSbLds >= 2 * 4 * router::kRbMaxE * 4, "the router backward's LDS rows");

// after the workgroup's stores: thread 0 adds to *bar with an agent-scope
// release and waits (bounded, acquire loads) until every workgroup has;
// false if the wait expired
__device__ __forceinline__ bool bar_sync(const SingleBwdParams& p, int32_t* bar, int* s_flag) {
  __syncthreads();   // the workgroup's stores precede thread 0's release
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(bar, p.publish, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    bool ok = false;
    for (int it = 0; it < p.polls && !ok; ++it) {
      ok = __hip_atomic_load(bar, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) >= (int)gridDim.x;
      if (!ok) __builtin_amdgcn_s_sleep(2);
    }
    if (!ok && p.status) atomicOr(p.status, 1);
    *s_flag = ok;
  }
  __syncthreads();   // thread 0 acquired; the workgroup's loads follow
  return *s_flag != 0;
}

__global__ __launch_bounds__(512) void layer_bwd_single_kernel(SingleBwdParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSbLds];
  __shared__ int s_item;
  __shared__ int s_flag;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int nt8 = (p.N + 7) / 8;

  // ---- 0. combine backward; the GEMM plans -----------------------------------
  for (int it = blockIdx.x; it < nt8; it += gridDim.x) {
    const int t = __builtin_amdgcn_readfirstlane(it * 8 + wave);
    if (t < p.N)
      perm::combine_bwd_token<false>(t, p.dout, p.dst_rows, p.topk_prob, p.y, p.D, p.K, p.dyd, p.dprob, nullptr,
                                     nullptr, nullptr);
  }
  {
    int* w = reinterpret_cast<int*>(smem);
    const int nplans = p.router ? 7 : 5;
    for (int j = (int)gridDim.x - 1 - (int)blockIdx.x; j < nplans; j += gridDim.x) {
      __syncthreads();   // the LDS of the previous plan
      if (j == 0) sched::plan_rows_body<512>(p.dg_dn.offsets, p.dg_dn.E, p.dg_dn.n_tiles, const_cast<int32_t*>(p.dg_dn.plan),
                                             p.dg_dn.head, w, w + 16, w + 32, reinterpret_cast<float*>(w + 512),
                                             w + 1024, w + 1536, w + 48);
      else if (j == 1) sched::plan_rows_body<512>(p.dg_gu.offsets, p.dg_gu.E, p.dg_gu.n_tiles,
                                                  const_cast<int32_t*>(p.dg_gu.plan), p.dg_gu.head, w, w + 16, w + 32,
                                                  reinterpret_cast<float*>(w + 512), w + 1024, w + 1536, w + 48);
      else if (j < 5) {
        const WgradParams& q = j == 2 ? p.wg_dn : (j == 3 ? p.wg_g : p.wg_u);
        plan_wgrad_body(q.offsets, q.E, q.m_tiles * q.n_tiles, const_cast<int32_t*>(q.plan), q.head, w);
      } else {
        // the router's token splits (the router backward's first block writes the same)
        if (tid <= p.S) p.offs[tid] = (int)((int64_t)p.N * tid / p.S);
        if (tid < 2) p.offs1[tid] = tid ? p.N : 0;
        __syncthreads();
        if (j == 5) sched::plan_rows_body<512>(p.dg_rt.offsets, p.dg_rt.E, p.dg_rt.n_tiles,
                                               const_cast<int32_t*>(p.dg_rt.plan), p.dg_rt.head, w, w + 16, w + 32,
                                               reinterpret_cast<float*>(w + 512), w + 1024, w + 1536, w + 48);
        else plan_wgrad_body(p.wg_rt.offsets, p.wg_rt.E, p.wg_rt.m_tiles * p.wg_rt.n_tiles,
                             const_cast<int32_t*>(p.wg_rt.plan), p.wg_rt.head, w);
      }
    }
  }
  if (!bar_sync(p, p.bar + 0, &s_flag)) return;

  // ---- 1. down dgrad, down wgrad, router backward blocks ----------------------
  dgrad_loop<true>(p.dg_dn, smem, lds0, &s_item);
  __syncthreads();   // the ring and s_item are free
  wgrad_loop(p.wg_dn, smem, lds0, &s_item);
  __syncthreads();
  if (p.router) {
    float (*s_g)[router::kRbMaxE] = reinterpret_cast<float (*)[router::kRbMaxE]>(smem) + 4 * (tid >> 8);
    const int npairs = (p.rb_blocks + 1) / 2;
    for (;;) {
      if (tid == 0) s_item = atomicAdd(p.bar + 3, 1);
      __syncthreads();
      const int pr = s_item;
      __syncthreads();
      if (pr >= npairs) break;
      const int blk = 2 * pr + (tid >> 8);
      router::router_bwd_block(blk, blk < p.rb_blocks, tid & 255, s_g, p.logits, p.topk_idx, p.dprob, p.N, p.E, p.K,
                               p.renorm, p.dl, p.dlb, p.colpart, p.offs, p.S, p.offs1, p.aux_counts, p.aux_c);
    }
  }
  if (!bar_sync(p, p.bar + 1, &s_flag)) return;

  // ---- 2. gate/up dgrad, gate and up wgrad, the router's GEMMs ----------------
  dgrad_loop<false>(p.dg_gu, smem, lds0, &s_item);
  __syncthreads();
  wgrad_loop(p.wg_g, smem, lds0, &s_item);
  __syncthreads();
  wgrad_loop(p.wg_u, smem, lds0, &s_item);
  __syncthreads();
  if (p.router) {
    dgrad_loop<false>(p.dg_rt, smem, lds0, &s_item);
    __syncthreads();
    wgrad_loop(p.wg_rt, smem, lds0, &s_item);
  }
  if (!bar_sync(p, p.bar + 2, &s_flag)) return;

  // ---- 3. the router's reductions and the fold ---------------------------------
  if (p.router) {
    const int64_t ED = (int64_t)p.E * p.D;
    if (p.rt_split)
      for (int64_t i = (int64_t)blockIdx.x * 512 + tid; i < ED / 4; i += (int64_t)gridDim.x * 512)
        router::router_reduce_dw4(i, reinterpret_cast<const float*>(p.wg_rt.c), p.S, ED, p.dw_r);
    if (p.db_r)
      for (int e = blockIdx.x * 8 + wave; e < p.E; e += gridDim.x * 8)
        router::router_reduce_db(e, p.colpart, p.rb_blocks, p.E, p.db_r);
  }
  for (int it = blockIdx.x; it < nt8; it += gridDim.x) {
    const int t = __builtin_amdgcn_readfirstlane(it * 8 + wave);
    if (t < p.N) perm::combine_token<false>(t, p.dxd, p.dst_rows, nullptr, p.D, p.K, p.dx, p.dxr, nullptr);
  }
}

__global__ void single_bwd_reset_kernel(int32_t* bar, int n) {
  if ((int)threadIdx.x < n) bar[threadIdx.x] = 0;
}

hipError_t grid_for(const void* kern, int* grid) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err == hipSuccess) err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 512, 0);
  if (per_cu < 1) per_cu = 1;
  *grid = cus * per_cu;
  return err;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

// dgrad: contraction (forward n_dim) in whole 64-row steps, output columns
// (forward k_dim) a multiple of 16, 16-byte aligned operands, 32-bit offsets
bool gemm_dgrad_fast_ok(const GemmBwd& b) {
  if (b.n_dim % 64 || b.k_dim % 16 || b.k_dim < 16) return false;
  if (b.n_dim * b.k_dim * 2 >= (int64_t(1) << 31) || 256 * b.n_dim * 2 >= (int64_t(1) << 31)) return false;
  if (!aligned16(b.dc0) || !aligned16(b.b0) || (b.dc1 && (!aligned16(b.dc1) || !aligned16(b.b1)))) return false;
  if (b.swiglu_bwd ? (!aligned16(b.dg) || !aligned16(b.du) || !aligned16(b.g) || !aligned16(b.u)) : !aligned16(b.da))
    return false;
  return true;
}

namespace {
DgradParams dgrad_params(const GemmBwd& b, int32_t* ws) {
  DgradParams p{};
  p.offsets = b.offsets;
  p.E = (int)b.E;
  p.N = (int)b.k_dim;
  p.K = (int)b.n_dim;
  p.nk = (int)(b.n_dim / 64);
  p.n_tiles = (int)((b.k_dim + 255) / 256);
  p.kcat = b.dc1 != nullptr;
  p.a0 = (const uint8_t*)b.dc0;
  p.a1 = (const uint8_t*)b.dc1;
  p.b0 = (const uint8_t*)b.b0;
  p.b1 = (const uint8_t*)b.b1;
  p.c0 = (uint16_t*)(b.swiglu_bwd ? b.dg : b.da);
  p.c1 = (uint16_t*)b.du;
  p.g = (const uint16_t*)b.g;
  p.u = (const uint16_t*)b.u;
  p.head = ws;
  p.plan = ws + kGemmHeadInts;
  return p;
}

WgradParams wgrad_params(const GemmBwd& b, const void* dc, void* db, int32_t* ws, bool f32) {
  WgradParams p{};
  p.offsets = b.offsets;
  p.E = (int)b.E;
  p.M = (int)b.n_dim;
  p.N = (int)b.k_dim;
  p.m_tiles = (p.M + WgTile::BM - 1) / WgTile::BM;
  p.n_tiles = (p.N + WgTile::BN - 1) / WgTile::BN;
  p.a = (const uint8_t*)dc;
  p.b = (const uint8_t*)b.a;
  p.c = db;
  p.f32 = f32;
  p.head = ws;
  p.plan = ws + kGemmHeadInts;
  return p;
}
}  // namespace

hipError_t launch_gemm_dgrad_fast(const GemmBwd& b, int32_t* ws, hipStream_t s) {
  const DgradParams p = dgrad_params(b, ws);
  plan_rows_kernel<<<1, 1024, 0, s>>>(b.offsets, (int)b.E, p.n_tiles, ws + kGemmHeadInts, ws);
  const void* kern = b.swiglu_bwd ? (const void*)gemm_dgrad_kernel<true> : (const void*)gemm_dgrad_kernel<false>;
  int grid = 0;
  hipError_t err = grid_for(kern, &grid);
  if (err != hipSuccess) return err;
  if (b.swiglu_bwd) gemm_dgrad_kernel<true><<<grid, 512, 0, s>>>(p);
  else gemm_dgrad_kernel<false><<<grid, 512, 0, s>>>(p);
  return hipGetLastError();
}

// wgrad: both output dims multiples of 16 (at least 16), 16-byte aligned
// operands, a contraction step's 64 rows within 32-bit offsets
bool gemm_wgrad_fast_ok(const GemmBwd& b, const void* dc, const void* db) {
  if (b.n_dim % 16 || b.k_dim % 16 || b.n_dim < 16 || b.k_dim < 16) return false;
  const int64_t w = b.n_dim > b.k_dim ? b.n_dim : b.k_dim;
  if (65 * w * 2 >= (int64_t(1) << 31)) return false;
  return aligned16(dc) && aligned16(b.a) && aligned16(db);
}

hipError_t launch_gemm_wgrad_fast(const GemmBwd& b, const void* dc, void* db, int32_t* ws, hipStream_t s,
                                  bool f32) {
  const WgradParams p = wgrad_params(b, dc, db, ws, f32);
  plan_wgrad_kernel<<<1, 1024, 0, s>>>(b.offsets, p.E, p.m_tiles * p.n_tiles, ws + kGemmHeadInts, ws);
  int grid = 0;
  hipError_t err = grid_for((const void*)gemm_wgrad_kernel, &grid);
  if (err != hipSuccess) return err;
  gemm_wgrad_kernel<<<grid, 512, 0, s>>>(p);
  return hipGetLastError();
}

// plans and queue heads of the single-launch backward's seven GEMM queues,
// then its four barrier words
size_t layer_bwd_single_ints(int64_t E, int S) {
  const int64_t w = E > S ? E : S;
  return (size_t)(7 * (kGemmHeadInts + gemm_fwd_plan_ints(w)) + 64);
}

bool layer_bwd_single_ok(const LayerBwdSingle& a) {
  if (a.E > 512 || a.S > 512) return false;
  if (!gemm_dgrad_fast_ok(a.down) || !gemm_dgrad_fast_ok(a.gu)) return false;
  if (!gemm_wgrad_fast_ok(a.down, a.dyd, a.dw_down) || !gemm_wgrad_fast_ok(a.gu, a.gu.dc0, a.dw_gate) ||
      !gemm_wgrad_fast_ok(a.gu, a.gu.dc1, a.dw_up))
    return false;
  if (a.router && (!gemm_dgrad_fast_ok(a.rt) ||
                   !(a.split ? gemm_wgrad_fast_ok(a.rs, a.rs.dc0, a.part) : gemm_wgrad_fast_ok(a.rt, a.rt.dc0, a.dw_r))))
    return false;
  return true;
}

hipError_t launch_layer_bwd_single(const LayerBwdSingle& a, int32_t* ws, hipStream_t s) {
  if (!layer_bwd_single_ok(a)) return hipErrorInvalidValue;
  const int64_t w = a.E > a.S ? a.E : a.S;
  const int64_t q = kGemmHeadInts + (int64_t)gemm_fwd_plan_ints(w);
  SingleBwdParams p{};
  p.dout = (const uint16_t*)a.dout;
  p.dst_rows = a.dst_rows;
  p.topk_prob = a.topk_prob;
  p.y = (const uint16_t*)a.y;
  p.N = (int)a.N;
  p.D = (int)a.D;
  p.K = (int)a.K;
  p.E = (int)a.E;
  p.dyd = (uint16_t*)a.dyd;
  p.dprob = a.dprob;
  p.dg_dn = dgrad_params(a.down, ws + 0 * q);
  p.wg_dn = wgrad_params(a.down, a.dyd, a.dw_down, ws + 1 * q, false);
  p.dg_gu = dgrad_params(a.gu, ws + 2 * q);
  p.wg_g = wgrad_params(a.gu, a.gu.dc0, a.dw_gate, ws + 3 * q, false);
  p.wg_u = wgrad_params(a.gu, a.gu.dc1, a.dw_up, ws + 4 * q, false);
  p.router = a.router;
  if (a.router) {
    p.dg_rt = dgrad_params(a.rt, ws + 5 * q);
    p.rt_split = a.split;
    p.wg_rt = a.split ? wgrad_params(a.rs, a.rs.dc0, a.part, ws + 6 * q, true)
                      : wgrad_params(a.rt, a.rt.dc0, a.dw_r, ws + 6 * q, false);
    p.logits = a.logits;
    p.topk_idx = a.topk_idx;
    p.renorm = a.renorm;
    p.dl = a.dl;
    p.dlb = a.dlb;
    p.colpart = a.colpart;
    p.offs = a.offs;
    p.S = a.S;
    p.offs1 = a.offs1;
    p.aux_counts = a.aux_counts;
    p.aux_c = a.aux_c;
    p.rb_blocks = (int)((a.N + 63) / 64);
    p.dw_r = (uint16_t*)a.dw_r;
    p.db_r = a.db_r;
  }
  p.dxd = (const uint16_t*)a.dxd;
  p.dx = (uint16_t*)a.dx;
  p.dxr = (const uint16_t*)a.dxr;
  p.bar = ws + 7 * q;
  p.status = a.status;
  p.polls = a.test_polls > 0 ? a.test_polls : (1 << 22);
  p.publish = a.test_polls > 0 ? 0 : 1;
  int grid = 0;
  hipError_t err = grid_for((const void*)layer_bwd_single_kernel, &grid);
  if (err != hipSuccess) return err;
  single_bwd_reset_kernel<<<1, 64, 0, s>>>(p.bar, 4);
  layer_bwd_single_kernel<<<grid, 512, 0, s>>>(p);
  return hipGetLastError();
}

// MXFP8 wgrad: output dims % 32, 32-bit offsets into an expert's block of
// at most max_len columns
bool gemm_wgrad_mx_ok(int64_t M, int64_t N, int64_t max_len) {
  return M % 32 == 0 && N % 32 == 0 && M >= 32 && N >= 32 && M * max_len < (int64_t(1) << 31) &&
         N * max_len < (int64_t(1) << 31);
}

hipError_t launch_gemm_wgrad_mx(const int32_t* offsets, const int32_t* toff, int64_t E, int64_t M, int64_t N,
                                const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs, void* db,
                                int32_t* ws, hipStream_t s) {
  WgradMxParams p{};
  p.offsets = offsets;
  p.toff = toff;
  p.E = (int)E;
  p.M = (int)M;
  p.N = (int)N;
  p.m_tiles = (p.M + WmxTile::BM - 1) / WmxTile::BM;
  p.n_tiles = (p.N + WmxTile::BN - 1) / WmxTile::BN;
  p.aq = aq;
  p.as = as;
  p.bq = bq;
  p.bs = bs;
  p.c = (uint16_t*)db;
  p.head = ws;
  p.plan = ws + kGemmHeadInts;
  plan_wgrad_kernel<<<1, 1024, 0, s>>>(offsets, p.E, p.m_tiles * p.n_tiles, ws + kGemmHeadInts, ws);
  int grid = 0;
  hipError_t err = grid_for((const void*)gemm_wgrad_mx_kernel, &grid);
  if (err != hipSuccess) return err;
  gemm_wgrad_mx_kernel<<<grid, 512, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
