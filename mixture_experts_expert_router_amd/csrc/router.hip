// Router logits L = X W_r^T + b on bf16 MFMA with fp32 accumulation (KOSMOS
// section 3.3.1 step 1: router logits in FP32 tiles; the router product has
// only as many columns as experts, so its tile is narrow).
//
// The product is skinny (N tokens x D, times D x E with E <= 1024), so one
// row block per workgroup would leave most CUs idle.  The contraction is
// split into S fixed ranges: item (row block, column tile, split) runs the
// shared MFMA tile engine over its range and writes an fp32 partial tile;
// a second kernel adds the S partials in ascending split order plus the bias.
// The split is a function of the shape only, so the result is bitwise the
// same run to run.  With S = 1 the tile kernel writes the logits directly.
// Every row block re-reads its column tile of W_r, so large N takes 128-row
// blocks (half the re-reads of 64-row ones).  The split is the fastest part
// of the item index: with 8 splits, workgroup b (on XCD b % 8) always reads
// the same slice of W_r, which stays in that XCD's L2.
//
// Shapes the engine does not take (D not a multiple of 64) use a direct
// kernel: one workgroup per 16 rows, operands read straight from global
// memory in 16-byte fragments, the contraction split over the waves when
// there are few column tiles.
#include "common.h"
#include "launch.h"
#include "mfma_tile.h"
#include "router_dev.h"

namespace moe {

namespace {

using router::RouterParams;
using router::RouterPlan;
using router::RouterTile;
using router::router_plan;
using router::router_tiled;

template <int BM, int BN>
__global__ __launch_bounds__(BM * 4) void router_tile_kernel(RouterParams p) {
  using C = RouterTile<BM, BN>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::NS * C::STAGE];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  router::router_tile_item<BM, BN>(p, blockIdx.x, smem, lds0);
}

// logits = sum over splits (ascending) of the partials, plus the bias; VEC:
// four adjacent logits per thread (E % 4 == 0), the same sums element by element
template <bool VEC>
__global__ __launch_bounds__(256) void router_reduce_kernel(const float* __restrict__ part, const float* __restrict__ bias,
                                                            int64_t NE, int E, int S, float* __restrict__ logits) {
  if constexpr (VEC) {
    const int64_t NE4 = NE >> 2;
    const f32x4_t* p4 = reinterpret_cast<const f32x4_t*>(part);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < NE4; i += (int64_t)gridDim.x * blockDim.x) {
      f32x4_t s = p4[i];
      for (int k = 1; k < S; ++k) s += p4[(int64_t)k * NE4 + i];
      if (bias) {
        const int e = (int)((i << 2) % E);
        s += f32x4_t{bias[e], bias[e + 1], bias[e + 2], bias[e + 3]};
      }
      reinterpret_cast<f32x4_t*>(logits)[i] = s;
    }
  } else {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < NE; i += (int64_t)gridDim.x * blockDim.x) {
      float s = part[i];
      for (int k = 1; k < S; ++k) s += part[(int64_t)k * NE + i];
      logits[i] = s + (bias ? bias[i % E] : 0.0f);
    }
  }
}

constexpr int kRouterMaxTiles = 16;   // column tiles per wave (E <= 1024)

__global__ __launch_bounds__(256) void router_direct_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ w,
                                                            const float* __restrict__ bias, int N,
                                                            int D, int E,
                                                            float* __restrict__ logits) {
  __shared__ float s_part[4][16][48];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int ntl = (E + 15) / 16;
  const int waves_n = ntl < 4 ? ntl : 4;
  const int waves_k = 4 / waves_n;
  const int wn = wv % waves_n, wk = wv / waves_n;
  if (wk >= waves_k) return;        // idle wave when ntl == 3 (no barrier follows for it)
  const int nq = (ntl - wn + waves_n - 1) / waves_n;
  const int ksteps = (D + 31) / 32;
  const int kper = (ksteps + waves_k - 1) / waves_k;
  const int kb = wk * kper, ke = min(ksteps, kb + kper);

  f32x4_t acc[kRouterMaxTiles];
#pragma unroll
  for (int q = 0; q < kRouterMaxTiles; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int xr = row0 + l16;
  const uint16_t* xrow = x + (int64_t)(xr < N ? xr : 0) * D;
  for (int ks = kb; ks < ke; ++ks) {
    const int k = ks * 32 + lg * 8;
    uint4 av = (xr < N && k < D) ? ldg16(xrow + k) : make_uint4(0, 0, 0, 0);
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
    for (int q = 0; q < kRouterMaxTiles; ++q) {
      if (q < nq) {
        const int n = (wn + q * waves_n) * 16 + l16;
        uint4 bv = (n < E && k < D) ? ldg16(w + (int64_t)n * D + k) : make_uint4(0, 0, 0, 0);
        acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, bv), acc[q], 0, 0, 0);
      }
    }
  }
  // lane holds rows 4*lg + r, column l16 of each tile
  if (waves_k > 1) {
    // ntl <= 3 here: partial sums to LDS, then wave 0 adds them in order wk = 0..
#pragma unroll
    for (int q = 0; q < 3; ++q)
      if (q < nq)
#pragma unroll
        for (int r = 0; r < 4; ++r) s_part[wk][4 * lg + r][(wn + q * waves_n) * 16 + l16] = acc[q][r];
    __syncthreads();
    if (wk != 0) return;
#pragma unroll
    for (int q = 0; q < 3; ++q)
      if (q < nq)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float s = 0.0f;
          for (int kk = 0; kk < waves_k; ++kk) s += s_part[kk][4 * lg + r][(wn + q * waves_n) * 16 + l16];
          acc[q][r] = s;
        }
  }
#pragma unroll
  for (int q = 0; q < kRouterMaxTiles; ++q) {
    if (q >= nq) continue;
    const int n = (wn + q * waves_n) * 16 + l16;
    if (n >= E) continue;
    const float b = bias ? bias[n] : 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + 4 * lg + r;
      if (row < N) logits[(int64_t)row * E + n] = acc[q][r] + b;
    }
  }
}

// tile height and width for the shape, and the number of contraction splits
}  // namespace

size_t router_workspace_bytes(int64_t N, int64_t D, int64_t E) {
  if (N <= 0 || !router_tiled(D, E)) return 0;
  const RouterPlan r = router_plan(N, D, E);
  return r.S > 1 ? (size_t)r.S * N * E * 4 : 0;
}

hipError_t launch_router_logits(const void* x, const void* w_r, const float* bias, int64_t N,
                                int64_t D, int64_t E, float* logits, void* ws, hipStream_t s) {
  if (N == 0) return hipSuccess;
  if (!router_tiled(D, E)) {
    router_direct_kernel<<<(unsigned)((N + 15) / 16), 256, 0, s>>>(
        (const uint16_t*)x, (const uint16_t*)w_r, bias, (int)N, (int)D, (int)E, logits);
    return hipGetLastError();
  }
  const RouterPlan r = router_plan(N, D, E);
  RouterParams p{(const uint16_t*)x, (const uint16_t*)w_r, bias, r.S > 1 ? (float*)ws : logits,
                 (int)N, (int)D, (int)E, r.S, r.mblocks, r.ntiles};
  const unsigned grid = (unsigned)((int64_t)r.mblocks * r.ntiles * r.S);
  if (r.bm == 128) {
    if (r.bn == 64) router_tile_kernel<128, 64><<<grid, 512, 0, s>>>(p);
    else if (r.bn == 128) router_tile_kernel<128, 128><<<grid, 512, 0, s>>>(p);
    else router_tile_kernel<128, 256><<<grid, 512, 0, s>>>(p);
  } else {
    if (r.bn == 64) router_tile_kernel<64, 64><<<grid, 256, 0, s>>>(p);
    else if (r.bn == 128) router_tile_kernel<64, 128><<<grid, 256, 0, s>>>(p);
    else router_tile_kernel<64, 256><<<grid, 256, 0, s>>>(p);
  }
  if (r.S > 1) {
    const int64_t NE = N * E;
    const bool vec = (E & 3) == 0;
    const int64_t nblk = ((vec ? NE / 4 : NE) + 255) / 256;
    const unsigned rg = (unsigned)(nblk < 4096 ? nblk : 4096);
    if (vec) router_reduce_kernel<true><<<rg, 256, 0, s>>>((const float*)ws, bias, NE, (int)E, r.S, logits);
    else router_reduce_kernel<false><<<rg, 256, 0, s>>>((const float*)ws, bias, NE, (int)E, r.S, logits);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router backward (KOSMOS section 3.3.2 step 2: the router's dX_r and dW_r).
// From the route-weight gradient dprob [N][K], token by token, with p the
// softmax of the saved logits and s_k = p[idx_k]:
//   ds_k = dprob_k, or (dprob_k - sum_j w_j dprob_j) / S with renormalised
//   weights w_k = s_k / S, S = sum_j s_j;
//   dL_e = p_e (g_e - sum_j p_j g_j), g_e = ds_k at e = idx_k, else 0, plus
//   aux_c counts_e for every e when the aux loss is on (its gradient with
//   the counts fixed).
// One wave per token (kRbTok tokens per wave, 4 waves per workgroup); g goes
// through a per-wave LDS row.  Each workgroup also writes the column sums of
// its 64 tokens' dL, added in wave order, for the bias gradient.  The GEMMs
// dX_r = dL W_r and dW_r = dL^T x run on the grouped-GEMM kernels.
// ---------------------------------------------------------------------------

using router::kRbMaxE;

__global__ __launch_bounds__(256) void router_bwd_kernel(const float* __restrict__ logits,
                                                         const int32_t* __restrict__ topk_idx,
                                                         const float* __restrict__ dprob, int N, int E, int K,
                                                         int renorm, float* __restrict__ dl,
                                                         uint16_t* __restrict__ dlb, float* __restrict__ colpart,
                                                         int32_t* __restrict__ offs, int S,
                                                         int32_t* __restrict__ offs1,
                                                         const int32_t* __restrict__ aux_counts, float aux_c) {
  __shared__ float s_g[4][kRbMaxE];
  router::router_bwd_block(blockIdx.x, true, threadIdx.x, s_g, logits, topk_idx, dprob, N, E, K, renorm, dl, dlb,
                           colpart, offs, S, offs1, aux_counts, aux_c);
}

__global__ __launch_bounds__(256) void router_bwd_reduce_kernel(const float* __restrict__ part, int S, int64_t ED,
                                                                uint16_t* __restrict__ dw_r,
                                                                const float* __restrict__ colpart, int64_t P,
                                                                int64_t E, float* __restrict__ db_r) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (part)
    for (int64_t i = tid; i < ED / 4; i += stride) router::router_reduce_dw4(i, part, S, ED, dw_r);
  if (db_r && blockIdx.x < E && threadIdx.x < 64) router::router_reduce_db(blockIdx.x, colpart, P, E, db_r);
}

// token splits of the router's wgrad: about 256 tiles, at least 64 rows each
int router_wgrad_splits(int64_t N, int64_t D, int64_t E) {
  const int64_t tiles = ((E + 255) / 256) * ((D + 255) / 256);
  int64_t S = (256 + tiles - 1) / tiles;
  S = S > 32 ? 32 : S;
  const int64_t cap = N / 64;
  S = S > cap ? cap : S;
  return (int)(S < 1 ? 1 : S);
}

hipError_t launch_router_bwd(const float* logits, const int32_t* topk_idx, const float* dprob, int64_t N,
                             int64_t E, int64_t K, int renorm, float* dl, uint16_t* dlb, float* colpart,
                             int32_t* offs, int S, int32_t* offs1, hipStream_t s, const int32_t* aux_counts,
                             float aux_c) {
  if (N == 0) return hipSuccess;
  router_bwd_kernel<<<(unsigned)((N + 63) / 64), 256, 0, s>>>(logits, topk_idx, dprob, (int)N, (int)E, (int)K,
                                                               renorm, dl, dlb, colpart, offs, S, offs1,
                                                               aux_counts, aux_c);
  return hipGetLastError();
}

hipError_t launch_router_bwd_reduce(const float* part, int S, int64_t ED, uint16_t* dw_r, const float* colpart,
                                    int64_t P, int64_t E, float* db_r, hipStream_t s) {
  router_bwd_reduce_kernel<<<1024, 256, 0, s>>>(part, S, ED, dw_r, colpart, P, E, db_r);   // E <= 1024 blocks
  return hipGetLastError();
}

}  // namespace moe
