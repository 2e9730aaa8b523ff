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
// Tile engine.  Operand tiles go from global memory straight into an NS-stage
// LDS ring with global_load_lds_dwordx4 (each wave instruction writes 1 KB:
// 64 lanes x 16 bytes at consecutive LDS addresses from M0), so no registers
// stage the copies and NS-1 contraction steps are in flight while the MFMAs of
// the current one run.  The loads are issued from inline assembly and their
// completion is tracked here with explicit vmcnt waits: the vector-memory
// loads of a wave complete in issue order, so "at most n outstanding" after
// the loads of n later steps were issued means every older step has landed.
// LDS rows hold 64 bf16 (128 bytes); chunk c of row r sits at slot c ^ (r & 7),
// which, measured on gfx950, keeps the 16-row fragment reads (ds_read_b128)
// free of bank conflicts; each lane fetches the global chunk that belongs at
// its LDS slot.  Eight waves per workgroup (two per SIMD).  Operands are fed
// swapped (weight tile as the MFMA's first operand) so each lane's four
// accumulators are four consecutive output columns of one row.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kBK = 64;          // contraction step (bf16 elements)
constexpr int kRB = kBK * 2;     // bytes per LDS row
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

__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr), "v"(g) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait until at most n_after steps' loads of this wave are outstanding
template <int LPS, int KMAX>
__device__ __forceinline__ void wait_steps(int n_after) {
  if constexpr (KMAX > 0) {
    if (n_after >= KMAX) { wait_vmcnt<KMAX * LPS>(); return; }
    wait_steps<LPS, KMAX - 1>(n_after);
  } else {
    wait_vmcnt<0>();
  }
}

__device__ __forceinline__ int slot_of(int r, int c) { return c ^ (r & 7); }

template <int BM_, int BN_, int NS_, int WAVES_M, int WAVES_N, bool DUAL_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, NS = NS_;
  static constexpr bool DUAL = DUAL_;
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int WAVES_N_ = WAVES_N;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 16, TN = WN / 16;
  static constexpr int RPI = 1024 / kRB;                           // rows per DMA instruction
  static constexpr int A_BYTES = BM * kRB, STAGE = (BM + BN) * kRB;
  static constexpr int A_INS = BM / RPI / NW, B_INS = BN / RPI / NW;   // per wave per step
  static constexpr int LPS = A_INS + B_INS;
  static constexpr int NCOL = DUAL ? BN / 2 : BN;                  // output columns per tile
  static_assert(A_INS * RPI * NW == BM && B_INS * RPI * NW == BN, "even DMA split");
  static_assert(WM % 16 == 0 && WN % 16 == 0 && (!DUAL || TN % 2 == 0), "wave tile");
  static_assert(NS >= 2 && NS * STAGE <= 160 * 1024, "LDS ring");
};

// Row of the B tile that wave column wn, fragment j reads.  DUAL: gate rows
// [0, BN/2), up rows [BN/2, BN); a wave holds TN/2 gate and TN/2 up fragments
// of the same output columns.
template <class C>
__device__ __forceinline__ int b_row(int wn, int j) {
  if (!C::DUAL) return wn * C::WN + j * 16;
  constexpr int half = C::TN / 2;
  const int jj = j < half ? j : j - half;
  return (j < half ? 0 : C::BN / 2) + wn * (C::WN / 2) + jj * 16;
}

// One output tile: rows [m_start, min(m_start + BM, m1)) of expert e, columns
// [n0, n0 + NCOL).  Rows past the expert's segment (or columns past N) load a
// clamped valid row and are never stored.
template <class C>
__device__ __forceinline__ void run_tile(const FwdParams& p, const uint8_t* smem, uint32_t lds0, int e,
                                         int m_start, int m1, int n0) {
  constexpr int TM = C::TM, TN = C::TN, WM = C::WM, WN = C::WN, NS = C::NS;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N_, wn = wave % C::WAVES_N_;
  const int l16 = lane & 15, lg = lane >> 4;
  const int nk = p.K / kBK;
  const int64_t K = p.K;

  int a_off[TM][2], b_off[TN][2];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int r = wm * WM + i * 16 + l16;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) a_off[i][ks] = r * kRB + (slot_of(r, ks * 4 + lg) << 4);
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int r = b_row<C>(wn, j) + l16;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) b_off[j][ks] = C::A_BYTES + r * kRB + (slot_of(r, ks * 4 + lg) << 4);
  }

  // this lane's place in a DMA instruction: row within the 1 KB block and the
  // global chunk that belongs at its slot (slot_of is an involution in c)
  const int d_row = lane >> 3;
  const int d_chunk = slot_of(d_row, lane & 7);
  const uint16_t* a_src[C::A_INS];
  const uint16_t* b_src[C::B_INS];
#pragma unroll
  for (int q = 0; q < C::A_INS; ++q) {
    const int r = (wave * C::A_INS + q) * C::RPI + d_row;
    const int row = min(m_start + r, m1 - 1);
    a_src[q] = p.a + (int64_t)row * K + d_chunk * 8;
  }
#pragma unroll
  for (int q = 0; q < C::B_INS; ++q) {
    const int r = (wave * C::B_INS + q) * C::RPI + d_row;
    const uint16_t* base = p.b0;
    int col = n0 + r;
    if (C::DUAL && r >= C::BN / 2) {
      base = p.b1;
      col = n0 + r - C::BN / 2;
    }
    col = min(col, p.N - 1);
    b_src[q] = base + ((int64_t)e * p.N + col) * K + d_chunk * 8;
  }
  const uint32_t wave_a = (uint32_t)(wave * C::A_INS) * 1024u;
  const uint32_t wave_b = (uint32_t)C::A_BYTES + (uint32_t)(wave * C::B_INS) * 1024u;
  auto issue = [&](int kt) {
    const uint32_t st = lds0 + (uint32_t)((kt % NS) * C::STAGE);
    const int64_t ko = (int64_t)kt * kBK;
#pragma unroll
    for (int q = 0; q < C::A_INS; ++q)
      lds_dma16(a_src[q] + ko, __builtin_amdgcn_readfirstlane(st + wave_a + q * 1024u));
#pragma unroll
    for (int q = 0; q < C::B_INS; ++q)
      lds_dma16(b_src[q] + ko, __builtin_amdgcn_readfirstlane(st + wave_b + q * 1024u));
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue(s);
  for (int kt = 0; kt < nk; ++kt) {
    wait_steps<C::LPS, NS - 2>(min(NS - 2, nk - 1 - kt));
    __syncthreads();   // step kt landed for every wave; every wave is done with step kt-1
    if (kt + NS - 1 < nk) issue(kt + NS - 1);
    const uint8_t* st = smem + (kt % NS) * C::STAGE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const bf16x8_t*>(st + a_off[i][ks]);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = *reinterpret_cast<const bf16x8_t*>(st + b_off[j][ks]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
  }
  __syncthreads();   // every wave is done reading the ring before it is refilled

  // epilogue: lane holds row wm*WM + i*16 + l16, columns 4*lg .. 4*lg+3 of its
  // 16-column fragment
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = wm * WM + i * 16 + l16;
    if (m_start + m >= m1) continue;
    const int64_t row = m_start + m;
    if (!C::DUAL) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + j * 16 + 4 * lg;
        if (n >= p.N) continue;
        const f32x4_t a = acc[i][j];
        *reinterpret_cast<uint2*>(p.c0 + row * p.N + n) =
            make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
      }
    } else {
#pragma unroll
      for (int j = 0; j < TN / 2; ++j) {
        const int n = n0 + wn * (WN / 2) + j * 16 + 4 * lg;
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

// The two tile classes; both have BN = 256 (DUAL: 128 gate + 128 up columns).
template <bool DUAL>
using BigTile = TileCfg<256, 256, 2, 4, 2, DUAL>;     // 2 x 64 KB ring
template <bool DUAL>
using SmallTile = TileCfg<128, 256, 3, 2, 4, DUAL>;   // 3 x 48 KB ring
constexpr int kLdsBytes = 3 * (128 + 256) * kRB;     // the larger ring
static_assert(kLdsBytes >= 2 * (256 + 256) * kRB, "ring size");

__device__ __host__ __forceinline__ bool is_big(int rows) { return rows >= kBigRows; }

template <bool DUAL>
__global__ __launch_bounds__(512) void gemm_fwd_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLdsBytes];
  __shared__ int s_item;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  const int total = p.plan[0];
  const int L = p.plan[1];
  const int32_t* order = p.plan + 2;
  const int32_t* pref = p.plan + 2 + p.E;

  int li = 0;   // position in the expert list; each workgroup's claims increase
  for (;;) {
    if (threadIdx.x == 0) s_item = atomicAdd(p.head, 1);
    __syncthreads();
    const int item = s_item;
    if (item >= total) break;
    while (li + 1 < L && pref[li + 1] <= item) ++li;
    const int e = order[li];
    const int m0 = p.offsets[e], m1 = p.offsets[e + 1];
    const int w = item - pref[li];
    if (is_big(m1 - m0)) {
      using C = BigTile<DUAL>;
      const int nmb = (m1 - m0 + C::BM - 1) / C::BM;
      const int n_t = w / nmb, mb = w - n_t * nmb;
      run_tile<C>(p, smem, lds0, e, m0 + mb * C::BM, m1, n_t * C::NCOL);
    } else {
      using C = SmallTile<DUAL>;
      const int nmb = (m1 - m0 + C::BM - 1) / C::BM;
      const int n_t = w / nmb, mb = w - n_t * nmb;
      run_tile<C>(p, smem, lds0, e, m0 + mb * C::BM, m1, n_t * C::NCOL);
    }
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

bool gemm_fwd_fast_ok(int64_t k_dim, int64_t n_dim) { return k_dim % kBK == 0 && n_dim % 16 == 0; }

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
