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


constexpr int kRbTok = 16;
constexpr int kRbMaxE = 1024;
constexpr int kRbCols = kRbMaxE / 64;   // logits per lane

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// One block of 64 tokens (4 waves of kRbTok tokens) of the router backward by
// 256 threads ltid = 0..255 of a workgroup, with their own LDS rows s_g[4]; a
// 512-thread workgroup runs two blocks at once.  The body calls
// __syncthreads() twice, so every thread of the workgroup makes the call;
// live == false (a block past the tokens) writes nothing.
__device__ __forceinline__ void router_bwd_block(int blk, bool live, int ltid, float (*s_g)[kRbMaxE],
                                                 const float* __restrict__ logits,
                                                 const int32_t* __restrict__ topk_idx,
                                                 const float* __restrict__ dprob, int N, int E, int K, int renorm,
                                                 float* __restrict__ dl, uint16_t* __restrict__ dlb,
                                                 float* __restrict__ colpart, int32_t* __restrict__ offs, int S,
                                                 int32_t* __restrict__ offs1, const int32_t* __restrict__ aux_counts,
                                                 float aux_c) {
  const int lane = ltid & 63, w = ltid >> 6;
  if (blk == 0 && live) {
    if (ltid <= S) offs[ltid] = (int)((int64_t)N * ltid / S);
    if (ltid < 2) offs1[ltid] = ltid ? N : 0;
  }
  const int nI = (E + 63) >> 6;
  float* g = s_g[w];
  float col[kRbCols];
#pragma unroll
  for (int i = 0; i < kRbCols; ++i) {
    col[i] = 0.0f;
    if (i < nI && lane + 64 * i < E) g[lane + 64 * i] = 0.0f;
  }
  // aux loss (optional): a_e = aux_c counts_e joins g for every expert
  float aj[kRbCols];
#pragma unroll
  for (int i = 0; i < kRbCols; ++i)
    aj[i] = (aux_counts && i < nI && lane + 64 * i < E) ? aux_c * (float)aux_counts[lane + 64 * i] : 0.0f;
  wave_lds_fence();
  const int t0 = blk * 64 + w * kRbTok;
  for (int j = 0; j < kRbTok; ++j) {
    const int t = t0 + j;
    if (t >= N) break;
    const float* Lr = logits + (int64_t)t * E;
    float l[kRbCols];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kRbCols; ++i) {
      const int e = lane + 64 * i;
      l[i] = (i < nI && e < E) ? Lr[e] : -INFINITY;
      m = fmaxf(m, l[i]);
    }
    m = wave_max(m);
    float z = 0.0f;
#pragma unroll
    for (int i = 0; i < kRbCols; ++i)
      if (i < nI && lane + 64 * i < E) z += expf(l[i] - m);
    z = wave_sum(z);
    const float rz = 1.0f / z;
    // the selected slots: lane k < K
    int ek = -1;
    float sk = 0.0f, dk = 0.0f;
    if (lane < K) {
      ek = topk_idx[(int64_t)t * K + lane];
      dk = dprob[(int64_t)t * K + lane];
      if (ek >= 0 && ek < E) sk = expf(Lr[ek] - m) * rz;
      else ek = -1;
    }
    float ds = dk;
    if (renorm) {
      const float tot = wave_sum(sk);
      const float c = wave_sum(sk * dk) / tot;   // sum_j w_j dprob_j
      ds = (dk - c) / tot;
    }
    float pa = 0.0f;
    if (aux_counts) {
#pragma unroll
      for (int i = 0; i < kRbCols; ++i)
        if (i < nI && lane + 64 * i < E) pa += expf(l[i] - m) * rz * aj[i];
    }
    const float dot = wave_sum(sk * ds + pa);
    if (ek >= 0) g[ek] = ds;
    wave_lds_fence();
    float* dlr = dl + (int64_t)t * E;
    uint16_t* dlbr = dlb + (int64_t)t * E;
#pragma unroll
    for (int i = 0; i < kRbCols; ++i) {
      const int e = lane + 64 * i;
      if (i < nI && e < E) {
        const float d = expf(l[i] - m) * rz * (g[e] + aj[i] - dot);
        dlr[e] = d;
        dlbr[e] = (uint16_t)(pack_bf16x2(d, 0.0f) & 0xFFFFu);
        col[i] += d;
      }
    }
    wave_lds_fence();
    if (ek >= 0) g[ek] = 0.0f;
    wave_lds_fence();
  }
  // column partials of this workgroup's tokens, added in wave order
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kRbCols; ++i)
    if (i < nI && lane + 64 * i < E) s_g[w][lane + 64 * i] = col[i];
  __syncthreads();
  if (live)
    for (int e = ltid; e < E; e += 256)
      colpart[(int64_t)blk * E + e] = ((s_g[0][e] + s_g[1][e]) + s_g[2][e]) + s_g[3][e];
}

// dw_r element block i (4 values): the S fp32 partials added in split order
__device__ __forceinline__ void router_reduce_dw4(int64_t i, const float* __restrict__ part, int S, int64_t ED,
                                                  uint16_t* __restrict__ dw_r) {
  float4 a = reinterpret_cast<const float4*>(part)[i];
  for (int sp = 1; sp < S; ++sp) {
    const float4 b = reinterpret_cast<const float4*>(part + (int64_t)sp * ED)[i];
    a.x += b.x;
    a.y += b.y;
    a.z += b.z;
    a.w += b.w;
  }
  reinterpret_cast<uint2*>(dw_r)[i] = make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w));
}

// db_r[e] by one wave: lane l adds the column partials l, l + 64, ... in
// order, then the lanes' sums are added by a fixed shuffle tree
__device__ __forceinline__ void router_reduce_db(int64_t e, const float* __restrict__ colpart, int64_t P, int64_t E,
                                                 float* __restrict__ db_r) {
  const int lane = threadIdx.x & 63;
  float a = 0.0f;
  for (int64_t b = lane; b < P; b += 64) a += colpart[b * E + e];
  a = wave_sum(a);
  if (lane == 0) db_r[e] = a;
}

}  // namespace router
}  // namespace moe
