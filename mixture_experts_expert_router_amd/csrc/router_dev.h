// Router tiles (KOSMOS section 3.3.1 step 1): the MFMA tile item of the
// router product and the shape rule that splits its contraction.  router.hip
// launches the items as a kernel; the single-launch layer runs them inside
// its persistent workgroups, with the same split, so the partial sums and
// the logits are the same bits either way.
#pragma once

#include "common.h"
#include "mfma_tile.h"

namespace moe {
namespace router {

template <int BM, int BN>
using RouterTile = tile::TileCfg<BM, BN, 3, BM / 64, 4, false>;   // 4 or 8 waves

struct RouterParams {
  const uint16_t* x;    // [N][D]
  const uint16_t* w;    // [E][D]
  const float* bias;    // [E] or null (added only when S == 1)
  float* out;           // S == 1: logits [N][E]; else partials [S][N][E]
  int N, D, E, S, mblocks, ntiles;
};

// One router item (row block, column tile, split) on a workgroup of BM * 4
// threads, its LDS ring at smem / lds0 (C::NS * C::STAGE bytes).
template <int BM, int BN>
__device__ __forceinline__ void router_tile_item(const RouterParams& p, int item, const uint8_t* smem,
                                                 uint32_t lds0) {
  using C = RouterTile<BM, BN>;
  using namespace tile;
  static_assert(C::NW * 64 == BM * 4, "block size");
  const int split = item % p.S;
  item /= p.S;
  const int mb = item % p.mblocks;
  const int nt = item / p.mblocks;
  const int nk = p.D / kBK;
  const int k0 = (int)((int64_t)nk * split / p.S), k1 = (int)((int64_t)nk * (split + 1) / p.S);
  const int m_start = mb * C::BM, n0 = nt * BN;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int d_chunk = dma_chunk();
  Src<C> src;
  const int64_t rb = (int64_t)p.D * 2;   // row bytes
  src.a = uniform_ptr(reinterpret_cast<const uint8_t*>(p.x + (int64_t)m_start * p.D + (int64_t)k0 * kBK));
  src.b = uniform_ptr(reinterpret_cast<const uint8_t*>(p.w + (int64_t)k0 * kBK));
#pragma unroll
  for (int q = 0; q < C::A_INS; ++q) {
    const int row = min(m_start + dma_row(wave, C::A_INS, q), p.N - 1);
    src.a_off[q] = (uint32_t)((row - m_start) * rb + d_chunk * 16);
  }
#pragma unroll
  for (int q = 0; q < C::B_INS; ++q) {
    const int col = min(n0 + dma_row(wave, C::B_INS, q), p.E - 1);
    src.b_off[q] = (uint32_t)(col * rb + d_chunk * 16);
  }
  f32x4_t acc[C::TM][C::TN];
  prologue<C>(lds0, src, k1 - k0);
  mainloop<C>(smem, lds0, src, k1 - k0, acc);

  // lane holds row wm*WM + i*16 + l16, columns wn*WN + j*16 + 4*lg + r
  const int l16 = lane & 15, lg = lane >> 4;
  const int wm = wave / C::WAVES_N_, wn = wave % C::WAVES_N_;
  float* out = p.out + (p.S > 1 ? (int64_t)split * p.N * p.E : 0);
  // rows of E floats start 16-byte aligned when E % 4 == 0 (outputs are 16-byte aligned)
  const bool vec4 = (p.E & 3) == 0;
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    const int row = m_start + wm * C::WM + i * 16 + l16;
    if (row >= p.N) continue;
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      const int n = n0 + wn * C::WN + j * 16 + 4 * lg;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = acc[i][j][r] + ((p.S == 1 && p.bias && n + r < p.E) ? p.bias[n + r] : 0.0f);
      if (vec4 && n < p.E) {   // the lane's 4 adjacent columns (n % 4 == 0) in one 16-byte store
        *reinterpret_cast<f32x4_t*>(out + (int64_t)row * p.E + n) = f32x4_t{v[0], v[1], v[2], v[3]};
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < p.E) out[(int64_t)row * p.E + n + r] = v[r];
      }
    }
  }
}

struct RouterPlan {
  int bm, bn, ntiles, mblocks, S;
};

inline RouterPlan router_plan(int64_t N, int64_t D, int64_t E) {
  RouterPlan r{};
  r.bm = N >= 2048 ? 128 : 64;
  r.bn = E <= 64 ? 64 : (E <= 128 ? 128 : 256);
  r.ntiles = (int)((E + r.bn - 1) / r.bn);
  r.mblocks = (int)((N + r.bm - 1) / r.bm);
  const int nk = (int)(D / tile::kBK);
  const int64_t base = (int64_t)r.mblocks * r.ntiles;
  const int64_t target = r.bm == 128 ? 256 : 512;   // about one (8-wave) or two (4-wave) items per CU
  int S = (int)((target + base - 1) / (base > 0 ? base : 1));
  S = S < 1 ? 1 : (S > nk ? nk : S);
  S = S > 16 ? 16 : S;
  r.S = S;
  return r;
}

inline bool router_tiled(int64_t D, int64_t E) { return D % tile::kBK == 0 && E >= 16; }

}  // namespace router
}  // namespace moe
