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
// once; every workgroup claims items from atomic head counters until the work
// is done.  An item is (expert, row block, n-tile).  Experts with many rows
// use 256-row tiles, the others 128-row tiles (KOSMOS section 3.4 uses 256x256
// tiles; small expert batches would waste most of such a tile).  A
// one-workgroup planner builds the expert order and the item prefix sums on
// the device from the expert offsets (no host round trip), interleaving the
// two tile classes in proportion to their work so that weight-streaming tiles
// of small experts run beside the MFMA-bound tiles of large ones, and resets
// the queue heads.  Which workgroup computes an item never changes its result.
//
// Cache locality across the chip's eight XCDs (each with its own L2): the item
// sequence is cut into chunks of 32 consecutive items, and chunk c belongs to
// the queue of XCD c % 8, so the 32 CUs of an XCD work on neighbouring items
// at the same time and fetch their shared operand tiles once.  Inside an
// expert the items run in super-blocks of 4 row blocks x 8 n-tiles (m
// fastest), so a chunk of a large expert reads 4 A blocks and 8 weight tiles
// instead of a whole operand.  A workgroup claims from its own XCD's queue and,
// once that is empty, takes items from the other queues.
//
// The MFMA main loop (direct-to-LDS operand ring) is the shared tile engine;
// eight waves per workgroup (two per SIMD).
//
// The same kernel runs the block-scaled MXFP8 variant (OLMo-core Appendix A,
// A.5 eq. 87; KOSMOS section 2.2): E4M3 operands with one E8M0 scale per 32
// contraction elements of each row, on the scaled 16x16x128 MFMA, fp32
// accumulation and the same bf16 outputs; GEMM1's epilogue also stores H
// quantized row-wise along its columns (blocks of 32, KOSMOS section 3.3.1
// step 3), the A operand of the MXFP8 GEMM2.
//
// The MXFP8 data gradient of the down projection runs here too (KOSMOS
// section 3.3.2 step 2; OLMo-core Appendix A, A.13: dgrad on the scaled
// grouped GEMM with a right-hand operand prequantized for it): A = dY_d
// quantized along D, B = W_down^T quantized along D, so the accumulator is
// dH.  Its epilogue applies the SwiGLU backward with the saved G and U,
// stores dG and dU in bf16 and quantizes [dG | dU] row-wise in blocks of 32,
// the A operand of the gate/up data gradient (a plain single-B MXFP8 GEMM over
// 2H contraction elements).
#include "common.h"
#include "launch.h"
#include "mfma_tile.h"
#include "sched.h"
#include "permute_dev.h"
#include "route_dev.h"
#include "router_dev.h"

namespace moe {

namespace {

using namespace sched;

struct FwdParams {
  const int32_t* offsets;   // [E+1]
  const int32_t* plan;      // planner output (layout below)
  int32_t* head;            // queue head counters, kHeadStride apart
  int E, N, K;              // N output columns per weight, K contraction
  int nk;                   // contraction steps (128 bytes of a row each)
  int n_tiles;              // ceil(N / NCOL)
  const uint8_t* a;         // [rows][K]      bf16 or E4M3
  const uint8_t* b0;        // [E][N][K]
  const uint8_t* b1;        // DUAL: [E][N][K]
  const uint8_t* as;        // MX: E8M0 [rows][K/32]
  const uint8_t* bs0;       // MX: E8M0 [E][N][K/32]
  const uint8_t* bs1;       // MX, DUAL
  uint16_t* c0;             // [rows][N]  (G or Y), bf16
  uint16_t* c1;             // DUAL: U
  uint16_t* c2;             // DUAL: H
  uint8_t* hq;              // DUAL, optional: H as E4M3 [rows][N]; DSW: [dG | dU] [rows][2N]
  uint8_t* hs;              //   and its E8M0 scales [rows][N/32]; DSW: [rows][2N/32]
  const uint16_t* g;        // DSW: saved G and U [rows][N], bf16
  const uint16_t* u;
};

// The two tile classes; both have BN = 256 (DUAL: 128 gate + 128 up columns).
template <bool DUAL, bool MX = false>
using BigTile = tile::TileCfg<256, 256, 2, 4, 2, DUAL, MX>;     // 2 x 64 KB ring (+2 x 2 KB scales)
template <bool DUAL, bool MX = false>
using SmallTile = tile::TileCfg<128, 256, 3, 2, 4, DUAL, MX>;   // 3 x 48 KB ring (+ scale groups)
// experts with at most 64 rows: the same columns, half the A rows
template <bool DUAL, bool MX = false>
using TinyTile = tile::TileCfg<64, 256, 3, 2, 4, DUAL, MX>;     // 3 x 40 KB ring
// bf16 experts with at most 32 rows: waves 0-3 load the A rows, and the
// smaller stage leaves room for a fourth, so three steps are in flight
template <bool DUAL, bool MX = false>
using Tiny32Tile = tile::TileCfg<32, 256, 4, 2, 4, DUAL, MX>;   // 4 x 36 KB ring
template <bool MX>
constexpr int lds_bytes() {
  constexpr int s = SmallTile<true, MX>::LDS, s1 = SmallTile<false, MX>::LDS;
  constexpr int b = BigTile<true, MX>::LDS, b1 = BigTile<false, MX>::LDS;
  constexpr int t = TinyTile<true, MX>::LDS, t1 = TinyTile<false, MX>::LDS;
  constexpr int u = Tiny32Tile<true, false>::LDS, u1 = Tiny32Tile<false, false>::LDS;
  constexpr int m0 = s > b ? s : b, m1 = s1 > b1 ? s1 : b1, m2 = t > t1 ? t : t1, m3 = u > u1 ? u : u1;
  constexpr int m01 = m0 > m1 ? m0 : m1, m23 = m2 > m3 ? m2 : m3;
  return m01 > m23 ? m01 : m23;
}
constexpr int kLdsBytes = lds_bytes<false>();

// Claim the next item of the row scheduler and decode it.
template <bool DUAL>
__device__ __forceinline__ Item claim(const FwdParams& p, int* s_item, int& li, int xcd) {
  return claim_rows(p.plan, p.offsets, p.head, p.E, p.n_tiles, BigTile<DUAL>::NCOL, s_item, li, xcd);
}

// DMA sources of an item (rows past the expert's segment or columns past N
// load a clamped valid row and are never stored).  A rows are offsets from
// the item's first row; a wave's B rows all belong to one weight (gate or
// up), offsets from that expert's matrix.  MX: thread t loads stage scale row
// t (A rows, then B rows, then padding that reloads the item's first A row);
// each wave's 64 scale rows come from one operand.
template <class C>
__device__ __forceinline__ void sources(const FwdParams& p, const Item& it, tile::Src<C>& src) {
  using namespace tile;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t RB = (int64_t)p.K * (C::MX ? 1 : 2);   // row bytes
  const int d_chunk = dma_chunk();
  src.a = uniform_ptr(p.a + (int64_t)it.m_start * RB);
#pragma unroll
  for (int q = 0; q < C::A_INS; ++q) {
    const int row = min(it.m_start + dma_row(wave, C::A_INS, q), it.m1 - 1);
    src.a_off[q] = (uint32_t)((row - it.m_start) * RB + d_chunk * 16);
  }
  const bool up_w = C::DUAL && wave * C::B_INS * C::RPI >= C::BN / 2;
  src.b = uniform_ptr((up_w ? p.b1 : p.b0) + (int64_t)it.e * p.N * RB);
#pragma unroll
  for (int q = 0; q < C::B_INS; ++q) {
    const int col = min(it.n0 + dma_row(wave, C::B_INS, q) - (up_w ? C::BN / 2 : 0), p.N - 1);
    src.b_off[q] = (uint32_t)(col * RB + d_chunk * 16);
  }
  if constexpr (C::MX) {
    // scale load q of this wave: tile rows [wave*SRW + 16q, +16), one operand
    const int KS = p.K / 32;
    src.s_ks = KS;
    const uint8_t* a_sc = p.as + (int64_t)it.m_start * KS;
#pragma unroll
    for (int q = 0; q < C::SCI; ++q) {
      const int r0 = wave * C::SRW + q * 16;
      if (r0 < C::BM || r0 >= C::BM + C::BN) {   // A rows, or padding (reloads the item's A rows)
        src.s[q] = uniform_ptr(a_sc);
        src.s_row0[q] = r0 < C::BM ? r0 : 0;
        src.s_lim[q] = __builtin_amdgcn_readfirstlane(it.m1 - it.m_start - 1);
      } else {
        const bool up = C::DUAL && r0 >= C::BM + C::BN / 2;
        src.s[q] = uniform_ptr((up ? p.bs1 : p.bs0) + (int64_t)it.e * p.N * KS);
        src.s_row0[q] = __builtin_amdgcn_readfirstlane(it.n0 + r0 - C::BM - (up ? C::BN / 2 : 0));
        src.s_lim[q] = p.N - 1;
      }
    }
  }
}

template <class C>
__device__ __forceinline__ void start(const FwdParams& p, uint32_t lds0, const Item& it) {
  tile::Src<C> src;
  sources<C>(p, it, src);
  tile::prologue<C>(lds0, src, p.nk);
}

template <class C>
__device__ __forceinline__ void mainloop_any(const uint8_t* smem, uint32_t lds0, const tile::Src<C>& src, int nk,
                                             f32x4_t (&acc)[C::TM][C::TN]) {
  if constexpr (C::MX) tile::mainloop_mx<C>(smem, lds0, src, nk, acc);
  else tile::mainloop<C>(smem, lds0, src, nk, acc);
}

template <class C>
__device__ __forceinline__ void epilogue(const FwdParams& p, const Item& it, const f32x4_t (&acc)[C::TM][C::TN]) {
  constexpr int TM = C::TM, TN = C::TN, WM = C::WM, WN = C::WN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N_, wn = wave % C::WAVES_N_;
  const int l16 = lane & 15, lg = lane >> 4;
  static_assert(TN % 2 == 0 && (!C::DUAL || (TN / 2) % 2 == 0), "fragment pairs");
  // lane holds row wm*WM + i*16 + l16, columns 4*lg .. 4*lg+3 of its
  // 16-column fragment
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = wm * WM + i * 16 + l16;
    if (it.m_start + m >= it.m1) continue;
    const int64_t row = it.m_start + m;
    const bool odd = lg & 1;
    if (!C::DUAL) {
      // 16-byte stores of fragment pairs (frag_pair_16b); N % 16 == 0
#pragma unroll
      for (int j = 0; j < TN; j += 2) {
        const f32x4_t a = acc[i][j], b = acc[i][j + 1];
        const uint4 v = frag_pair_16b(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                                      pack_bf16x2(b[2], b[3]), odd);
        const int n = it.n0 + wn * WN + (j + (odd ? 1 : 0)) * 16 + 8 * (lg >> 1);
        if (n >= p.N) continue;
        *reinterpret_cast<uint4*>(p.c0 + row * p.N + n) = v;
      }
    } else {
      uint32_t gw[TN / 2][2], uw[TN / 2][2], hw[TN / 2][2];
#pragma unroll
      for (int j = 0; j < TN / 2; ++j) {
        const f32x4_t a = acc[i][j], b = acc[i][j + TN / 2];
        gw[j][0] = pack_bf16x2(a[0], a[1]);
        gw[j][1] = pack_bf16x2(a[2], a[3]);
        uw[j][0] = pack_bf16x2(b[0], b[1]);
        uw[j][1] = pack_bf16x2(b[2], b[3]);
        const float g0 = bf16lo(gw[j][0]), g1 = bf16hi(gw[j][0]), g2 = bf16lo(gw[j][1]), g3 = bf16hi(gw[j][1]);
        const float h0 = g0 * sigmoidf_(g0) * bf16lo(uw[j][0]);
        const float h1 = g1 * sigmoidf_(g1) * bf16hi(uw[j][0]);
        const float h2 = g2 * sigmoidf_(g2) * bf16lo(uw[j][1]);
        const float h3 = g3 * sigmoidf_(g3) * bf16hi(uw[j][1]);
        hw[j][0] = pack_bf16x2(h0, h1);
        hw[j][1] = pack_bf16x2(h2, h3);
      }
      // G, U and H as 16-byte stores of fragment pairs (frag_pair_16b)
#pragma unroll
      for (int j = 0; j < TN / 2; j += 2) {
        const uint4 gv = frag_pair_16b(gw[j][0], gw[j][1], gw[j + 1][0], gw[j + 1][1], odd);
        const uint4 uv = frag_pair_16b(uw[j][0], uw[j][1], uw[j + 1][0], uw[j + 1][1], odd);
        const uint4 hv = frag_pair_16b(hw[j][0], hw[j][1], hw[j + 1][0], hw[j + 1][1], odd);
        const int n = it.n0 + wn * (WN / 2) + (j + (odd ? 1 : 0)) * 16 + 8 * (lg >> 1);
        if (n >= p.N) continue;
        const int64_t off = row * p.N + n;
        *reinterpret_cast<uint4*>(p.c0 + off) = gv;
        *reinterpret_cast<uint4*>(p.c1 + off) = uv;
        if (p.c2) *reinterpret_cast<uint4*>(p.c2 + off) = hv;   // MXFP8 may keep H quantized only
      }
      if (p.hq) {
        // a 32-column block of H is fragments (j, j+1) over the four lane
        // groups of one row (N % 32 == 0, so a block is all in or all out)
#pragma unroll
        for (int j = 0; j < TN / 2; j += 2) {
          const float v[8] = {bf16lo(hw[j][0]),     bf16hi(hw[j][0]),     bf16lo(hw[j][1]),     bf16hi(hw[j][1]),
                              bf16lo(hw[j + 1][0]), bf16hi(hw[j + 1][0]), bf16lo(hw[j + 1][1]), bf16hi(hw[j + 1][1])};
          float amax = 0.0f;
#pragma unroll
          for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
          amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
          amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
          const int code = e8m0_code(amax);
          const uint32_t q0 = e4m3x4(v[0], v[1], v[2], v[3], code - 127);
          const uint32_t q1 = e4m3x4(v[4], v[5], v[6], v[7], code - 127);
          const int nb = it.n0 + wn * (WN / 2) + j * 16;
          if (nb >= p.N) continue;
          uint8_t* qrow = p.hq + row * p.N + nb + 4 * lg;
          *reinterpret_cast<uint32_t*>(qrow) = q0;
          *reinterpret_cast<uint32_t*>(qrow + 16) = q1;
          if (lg == 0) p.hs[row * (p.N / 32) + nb / 32] = (uint8_t)code;
        }
      }
    }
  }
}

// MX data gradient of the down projection: acc = dH [rows][N] (N = H).
// dG = dH U s (1 + G (1 - s)), dU = dH G s with s = sigmoid(G) from the saved
// bf16 G and U, stored bf16 in c0 / c1; the bf16 values are then quantized
// row-wise, dG into columns [0, N) and dU into [N, 2N) of hq / hs.  Fragment
// pairs are handled in the 16-byte layout of frag_pair_16b (each lane owns 8
// adjacent columns; its dH values come from its own fragment and its
// partner's, lane ^ 16).  A 32-column block is one pair over the four lane
// groups of a row, so a block's amax is two shuffles away (N % 32 == 0: a
// block is all in or all out).
template <class C>
__device__ __forceinline__ void epilogue_dsw(const FwdParams& p, const Item& it,
                                             const f32x4_t (&acc)[C::TM][C::TN]) {
  constexpr int TM = C::TM, TN = C::TN, WM = C::WM, WN = C::WN;
  static_assert(!C::DUAL && TN % 2 == 0, "single-B tile, fragment pairs");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N_, wn = wave % C::WAVES_N_;
  const int l16 = lane & 15, lg = lane >> 4;
  const bool odd = lg & 1;
  const int64_t N2 = 2 * (int64_t)p.N;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = wm * WM + i * 16 + l16;
    if (it.m_start + m >= it.m1) continue;
    const int64_t row = it.m_start + m;
    // two pairs (64 columns) at a time: their G and U loads are issued
    // together, and fewer values stay live beside the accumulators
#pragma unroll
    for (int j0 = 0; j0 < TN / 2; j0 += 2) {
      constexpr int kPairs = 2;
      static_assert((TN / 2) % kPairs == 0, "whole pair groups");
      uint4 gv[kPairs], uv[kPairs];
#pragma unroll
      for (int jj = 0; jj < kPairs; ++jj) {
        const int n = it.n0 + wn * WN + (2 * (j0 + jj) + (odd ? 1 : 0)) * 16 + 8 * (lg >> 1);
        gv[jj] = uv[jj] = make_uint4(0, 0, 0, 0);
        if (n < p.N) {
          gv[jj] = ldg16(p.g + row * p.N + n);
          uv[jj] = ldg16(p.u + row * p.N + n);
        }
      }
#pragma unroll
      for (int jj = 0; jj < kPairs; ++jj) {
        const int jp = j0 + jj;
        const f32x4_t a = acc[i][2 * jp], b = acc[i][2 * jp + 1];
        float dh[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float r = __shfl_xor(odd ? a[q] : b[q], 16, 64);
          dh[q] = odd ? r : a[q];
          dh[4 + q] = odd ? b[q] : r;
        }
        const uint32_t gw[4] = {gv[jj].x, gv[jj].y, gv[jj].z, gv[jj].w};
        const uint32_t uw[4] = {uv[jj].x, uv[jj].y, uv[jj].z, uv[jj].w};
        uint32_t dgw[4], duw[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float g0 = bf16lo(gw[w]), g1 = bf16hi(gw[w]), u0 = bf16lo(uw[w]), u1 = bf16hi(uw[w]);
          const float s0 = sigmoidf_(g0), s1 = sigmoidf_(g1);
          dgw[w] = pack_bf16x2(dh[2 * w] * u0 * s0 * (1.0f + g0 * (1.0f - s0)),
                               dh[2 * w + 1] * u1 * s1 * (1.0f + g1 * (1.0f - s1)));
          duw[w] = pack_bf16x2(dh[2 * w] * g0 * s0, dh[2 * w + 1] * g1 * s1);
        }
        // quantize the bf16 values: a 32-column block spans the row's four lane groups
        uint2 qv[2];
        int code[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t* w = h ? duw : dgw;
          const float v[8] = {bf16lo(w[0]), bf16hi(w[0]), bf16lo(w[1]), bf16hi(w[1]),
                              bf16lo(w[2]), bf16hi(w[2]), bf16lo(w[3]), bf16hi(w[3])};
          float amax = 0.0f;
#pragma unroll
          for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
          amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
          amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
          code[h] = e8m0_code(amax);
          qv[h] = make_uint2(e4m3x4(v[0], v[1], v[2], v[3], code[h] - 127),
                             e4m3x4(v[4], v[5], v[6], v[7], code[h] - 127));
        }
        const int nb = it.n0 + wn * WN + 2 * jp * 16;   // the block's first column
        if (nb >= p.N) continue;
        const int n = nb + (odd ? 16 : 0) + 8 * (lg >> 1);
        const int64_t off = row * p.N + n;
        stg16(p.c0 + off, make_uint4(dgw[0], dgw[1], dgw[2], dgw[3]));
        stg16(p.c1 + off, make_uint4(duw[0], duw[1], duw[2], duw[3]));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          *reinterpret_cast<uint2*>(p.hq + row * N2 + h * p.N + n) = qv[h];
          if (lg == 0) p.hs[row * (N2 / 32) + (h * p.N + nb) / 32] = (uint8_t)code[h];
        }
      }
    }
  }
}

// Run the current item (its prologue already issued), then claim the next
// one and issue its prologue before storing this item's outputs, so the
// loads of the next tile overlap this epilogue.
template <class C, bool DUAL, bool DSW = false>
__device__ __forceinline__ Item run_item(const FwdParams& p, const uint8_t* smem, uint32_t lds0, int* s_item,
                                         int& li, int xcd, const Item& it) {
  tile::Src<C> src;
  sources<C>(p, it, src);
  f32x4_t acc[C::TM][C::TN];
  mainloop_any<C>(smem, lds0, src, p.nk, acc);
  const Item next = claim<DUAL>(p, s_item, li, xcd);
  if (next.valid) {
    if (next.big) start<BigTile<DUAL, C::MX>>(p, lds0, next);
    else if (!C::MX && next.tiny32) start<Tiny32Tile<DUAL, false>>(p, lds0, next);
    else if (next.tiny) start<TinyTile<DUAL, C::MX>>(p, lds0, next);
    else start<SmallTile<DUAL, C::MX>>(p, lds0, next);
  }
  if constexpr (DSW) epilogue_dsw<C>(p, it, acc);
  else epilogue<C>(p, it, acc);
  return next;
}

template <bool DUAL, bool MX, bool DSW = false>
__global__ __launch_bounds__(512) void gemm_fwd_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[lds_bytes<MX>()];
  __shared__ int s_item;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  using Big = BigTile<DUAL, MX>;
  using Small = SmallTile<DUAL, MX>;
  using Tiny = TinyTile<DUAL, MX>;
  using Tiny32 = Tiny32Tile<DUAL, false>;
  const int xcd = xcd_id();
  int li = 0;
  Item it = claim<DUAL>(p, &s_item, li, xcd);
  if (!it.valid) return;
  if (it.big) start<Big>(p, lds0, it);
  else if (!MX && it.tiny32) start<Tiny32>(p, lds0, it);
  else if (it.tiny) start<Tiny>(p, lds0, it);
  else start<Small>(p, lds0, it);
  while (it.valid) {
    if (it.big) it = run_item<Big, DUAL, DSW>(p, smem, lds0, &s_item, li, xcd, it);
    else if (!MX && it.tiny32) it = run_item<Tiny32, DUAL, DSW>(p, smem, lds0, &s_item, li, xcd, it);
    else if (it.tiny) it = run_item<Tiny, DUAL, DSW>(p, smem, lds0, &s_item, li, xcd, it);
    else it = run_item<Small, DUAL, DSW>(p, smem, lds0, &s_item, li, xcd, it);
  }
}

template <bool DUAL, bool MX, bool DSW = false>
hipError_t run_fwd(FwdParams p, int32_t* plan, hipStream_t s) {
  plan_rows_kernel<<<1, 1024, 0, s>>>(p.offsets, p.E, p.n_tiles, plan, p.head);
  auto kern = gemm_fwd_kernel<DUAL, MX, DSW>;
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err == hipSuccess) err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 512, 0);
  if (err != hipSuccess) return err;
  if (per_cu < 1) per_cu = 1;
  kern<<<cus * per_cu, 512, 0, s>>>(p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused expert forward: dispatch -> GEMM1 -> GEMM2 in one persistent launch,
// each tile gated on data readiness (KOSMOS section 3.1.1 and section 3.3.1
// steps 3-4, on one GPU).  A workgroup runs, in order:
//   1. its share of the dispatch: each token row read once and written to
//      its routes' rows of X_d (as the dispatch launch does; MXFP8: quantized
//      on the way, a wave per row segment, after the share's experts'
//      padding rows are zeroed), then one release adding the share to a
//      count;
//   2. GEMM1 tiles (MXFP8: block-scaled, H stored quantized) from the
//      staged launch's per-XCD queues, in its order
//      (the two tile classes interleaved in proportion to their work,
//      super-blocks of neighbouring tiles on one XCD's L2); a workgroup's
//      first tile waits until every workgroup's share is counted;
//   3. GEMM2 tiles the same way (a plan of their own); each waits until
//      every GEMM1 n-tile of its (expert, row block) has stored H, so GEMM2
//      starts on the row blocks GEMM1 finished while its last tiles run.
// The dispatch shares never wait, and a workgroup goes from GEMM1 to GEMM2
// when its claims come back empty, so every GEMM1 tile is claimed, by a
// running workgroup, before any GEMM2 tile: items only wait on earlier
// steps, and the queue drains whatever the grid size.  On one GPU the rows
// of an expert come from tokens all over the batch, so an expert is complete
// only when nearly the whole dispatch is.  Two per-expert readiness orders
// were measured slower than this (DeepSeek-V3 bf16 forward 5.10-5.42 ms
// against 4.3 here): GEMM tiles claimed in the order dispatch completed the
// experts gave phases of only weight-streaming and of only MFMA-bound tiles
// and lost the per-XCD L2 sharing, and an expert-major gather (a wave per
// X_d row) read each token row K times.
// A writer workgroup ends its stores with a workgroup barrier, then its
// thread 0 publishes with an agent-scope release (the release covers the
// whole workgroup's stores, which the barrier ordered before it); a reader's
// thread 0 waits with agent-scope acquire loads and a workgroup barrier
// orders the other threads' loads after that acquire.  Each release is a
// write-back of the L2, so there is one per published item (GEMM1 tiles:
// one per batch, flush_g1), never one per wave.
// Waits are bounded: a wait that expires or-s MOE_STATUS_WAIT_EXPIRED into
// the caller's status word and the item that waited is skipped (no load, no
// store), so no wave can hang and nothing is computed from unpublished data.
// ---------------------------------------------------------------------------

constexpr int kSpinLimit = 1 << 22;

struct FusedParams {
  FwdParams g1, g2;             // g1: X_d -> G, U, H;  g2: H -> Y (plans and queue heads in each)
  const uint16_t* x;            // [N][D] token rows
  const int32_t* dst_rows;      // [N][K] row of each route in X_d, -1 if none
  const int32_t* counts;        // MXFP8: [E] rows of each expert (the rest of its segment is padding)
  int N, K;                     // tokens, routes per token
  int32_t* st;                  // queue state (zeroed by the planner)
  const int32_t* fplan;         // fused plan
  int nt1, nt2;                 // n-tiles of GEMM1 / GEMM2
  int32_t* status;              // optional caller status word
  int polls;                    // bound of every wait
  int publish;                  // 0: readiness withheld (testing the bound)
};

// queue state layout (int32 units; 128-byte aligned): the GEMM2 queue heads,
// then the counters and per-expert and per-row-block words
__device__ __host__ __forceinline__ int st_err() { return kGemmHeadInts + 1; }
__device__ __host__ __forceinline__ int st_disp_done() { return kGemmHeadInts + 2; }  // dispatch items stored
__device__ __host__ __forceinline__ int st_g1_done() { return kGemmHeadInts + 3; }    // [row block]
__device__ __host__ __forceinline__ int st_ints(int max_mb) { return kGemmHeadInts + 3 + max_mb; }

// fused plan layout (int32 units): each expert's first row block in the
// planner's order [E], then the GEMM2 plan (the GEMM planner's layout:
// items, L, order, item prefix)
__device__ __host__ __forceinline__ int fp_plan2(int E) { return E; }
__device__ __host__ __forceinline__ int fp_ints(int E) { return E + (int)gemm_fwd_plan_ints(E) + 8; }

__device__ __forceinline__ int ld_acquire(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}

// thread 0: wait until *p >= target (bounded); false if the bound expired,
// which is recorded in the queue state and the caller's status word
__device__ __forceinline__ bool wait_ge(const FusedParams& f, const int32_t* p, int target) {
  for (int it = 0; it < f.polls; ++it) {
    if (ld_acquire(p) >= target) return true;
    __builtin_amdgcn_s_sleep(2);
  }
  atomicOr(f.st + st_err(), 1);
  if (f.status) atomicOr(f.status, 1);
  return false;
}

__device__ __forceinline__ int rows_bm(int rows) { return is_big(rows) ? 256 : 128; }

// row block of a claimed tile within its expert (blocks of the expert's own
// size, 256 or 128 rows, whatever tile class runs the last one)
__device__ __forceinline__ int claimed_block(const FwdParams& p, const Item& it) {
  const int m0 = p.offsets[it.e];
  return (it.m_start - m0) / rows_bm(it.m1 - m0);
}

// thread 0: the readiness word of a claimed tile and the value it waits
// for: GEMM1 the count of stored dispatch items, GEMM2 its GEMM1 row
// block's count of stored n-tiles
template <bool DUAL>
__device__ __forceinline__ const int32_t* gate_word(const FusedParams& f, const int32_t* mbase, const Item& it,
                                                    int* target) {
  if (DUAL) {
    *target = (int)gridDim.x;   // every workgroup's share of the dispatch
    return f.st + st_disp_done();
  }
  *target = f.nt1;
  return f.st + st_g1_done() + mbase[it.e] + claimed_block(f.g2, it);
}

// thread 0: is the tile ready?  One acquire load (block = false), or a
// bounded wait (block = true; false if it expired, reported).
template <bool DUAL>
__device__ __forceinline__ bool gate(const FusedParams& f, const int32_t* mbase, const Item& it, bool block) {
  int target = 0;
  const int32_t* w = gate_word<DUAL>(f, mbase, it, &target);
  return block ? wait_ge(f, w, target) : ld_acquire(w) >= target;
}

template <bool DUAL, bool MX>
__device__ __forceinline__ void start_claimed(const FwdParams& p, uint32_t lds0, const Item& it) {
  if (it.big) start<BigTile<DUAL, MX>>(p, lds0, it);
  else if (!MX && it.tiny32) start<Tiny32Tile<DUAL, false>>(p, lds0, it);
  else if (it.tiny) start<TinyTile<DUAL, MX>>(p, lds0, it);
  else start<SmallTile<DUAL, MX>>(p, lds0, it);
}

// GEMM1 tiles are published to their row blocks' counts in batches: thread
// 0 lists each stored tile's row block (s_info[4 ..], kPend entries) and a
// flush makes them all visible with one agent-scope release fence, then adds
// them to the counts with relaxed atomics.  On gfx950 an agent-scope release
// writes back the L2, so one per batch instead of one per tile; every count
// is a read-modify-write, so a reader that acquires the complete count
// synchronizes with each contributor's fence.  A workgroup flushes when its
// list is full, and after every tile once its claims reach the last two
// tiles a workgroup of the queue (GEMM2 tiles start while those run, and
// must not wait for tiles stored long before but held in a list).
constexpr int kPend = 16;
constexpr int kInfoInts = 4 + kPend;   // s_info: 4 words, then the pending list

// every thread, npend the same in all: publish the listed GEMM1 tiles
__device__ __forceinline__ void flush_g1(const FusedParams& f, int* s_info, int& npend) {
  __syncthreads();   // the workgroup's stores precede thread 0's release fence
  if (threadIdx.x == 0 && npend > 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    for (int i = 0; i < npend; ++i)
      __hip_atomic_fetch_add(f.st + st_g1_done() + s_info[4 + i], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  npend = 0;
}

// Run a claimed tile whose prologue is issued, as the staged engine does:
// after its main loop, claim the next tile and, if that one is already
// ready, issue its prologue before this tile's stores, so its loads overlap
// them.  A GEMM1 tile then joins the pending list (npend: the same count in
// every thread).  Returns the next tile; *next_started says whether its
// prologue is issued.
template <class C, bool DUAL>
__device__ __forceinline__ Item fused_tile(const FusedParams& f, const FwdParams& p, const uint8_t* smem,
                                           uint32_t lds0, int* s_info, int& li, int xcd, bool* gated,
                                           const int32_t* mbase, const Item& it, bool* next_started, int& npend) {
  tile::Src<C> src;
  sources<C>(p, it, src);
  f32x4_t acc[C::TM][C::TN];
  mainloop_any<C>(smem, lds0, src, p.nk, acc);
  const Item next = claim_rows(p.plan, p.offsets, p.head, p.E, p.n_tiles, BigTile<DUAL>::NCOL, s_info, li, xcd);
  // s_info[0] still holds the claim's place in the queue (-1: none left)
  const bool late = !next.valid || s_info[0] >= p.plan[0] - 2 * (int)gridDim.x;
  bool started = false;
  if (next.valid) {
    if (DUAL && *gated) {
      started = true;   // GEMM1's gate is the same for every tile: acquired once
    } else {
      if (threadIdx.x == 0) s_info[3] = gate<DUAL>(f, mbase, next, false);
      __syncthreads();   // thread 0 acquired; the workgroup's loads follow
      started = s_info[3] != 0;
      if (DUAL && started) *gated = true;
    }
    if (started) start_claimed<DUAL, C::MX>(p, lds0, next);
  }
  epilogue<C>(p, it, acc);
  if (DUAL) {
    if (threadIdx.x == 0) s_info[4 + npend] = mbase[it.e] + claimed_block(p, it);
    if (++npend == kPend || late) flush_g1(f, s_info, npend);
  }
  *next_started = started;
  return next;
}

// Every tile of one GEMM from its per-XCD queues, each after its readiness
// word; a tile whose bounded wait expires is skipped (reported).
template <bool DUAL, bool MX>
__device__ __forceinline__ void gemm_phase(const FusedParams& f, const FwdParams& p, const uint8_t* smem,
                                           uint32_t lds0, int* s_info, int xcd, const int32_t* mbase) {
  int li = 0, npend = 0;
  bool gated = false;   // GEMM1's gate acquired (the same in every thread)
  Item it = claim_rows(p.plan, p.offsets, p.head, p.E, p.n_tiles, BigTile<DUAL>::NCOL, s_info, li, xcd);
  bool started = false;
  while (it.valid) {
    if (!started) {
      if (!(DUAL && gated)) {
        if (threadIdx.x == 0) s_info[3] = gate<DUAL>(f, mbase, it, true);
        __syncthreads();   // thread 0 acquired; the workgroup's loads follow
        if (!s_info[3]) {   // the wait expired: skip the tile
          it = claim_rows(p.plan, p.offsets, p.head, p.E, p.n_tiles, BigTile<DUAL>::NCOL, s_info, li, xcd);
          continue;
        }
        if (DUAL) gated = true;
      }
      start_claimed<DUAL, MX>(p, lds0, it);
    }
    if (it.big)
      it = fused_tile<BigTile<DUAL, MX>, DUAL>(f, p, smem, lds0, s_info, li, xcd, &gated, mbase, it, &started,
                                               npend);
    else if (!MX && it.tiny32)
      it = fused_tile<Tiny32Tile<DUAL, false>, DUAL>(f, p, smem, lds0, s_info, li, xcd, &gated, mbase, it,
                                                     &started, npend);
    else if (it.tiny)
      it = fused_tile<TinyTile<DUAL, MX>, DUAL>(f, p, smem, lds0, s_info, li, xcd, &gated, mbase, it, &started,
                                                npend);
    else
      it = fused_tile<SmallTile<DUAL, MX>, DUAL>(f, p, smem, lds0, s_info, li, xcd, &gated, mbase, it, &started,
                                                 npend);
  }
  if (DUAL) flush_g1(f, s_info, npend);   // the rest of this workgroup's GEMM1 tiles
}

// The fold after the fused queue (single-launch layer): items of 8 tokens, a
// wave per token.  Every workgroup publishes once, when it has claimed its
// last GEMM2 tile (each of its GEMM2 tiles then is stored), and a fold item
// waits until all of them have: the fold reads Y rows of any expert.
struct FoldArgs {
  const int32_t* dst_rows;   // [N][K]
  const float* weight;       // [N][K] route weights
  int N;
  uint16_t* out;             // [N][D]
  int32_t* passed;           // workgroups past the GEMM2 tiles (zeroed before the launch)
};

// The readiness-gated queue: dispatch items, GEMM1 and GEMM2 tiles, then the
// fold when fold != nullptr (bf16 only).  MX: the dispatch quantizes each
// token row (the MXFP8 dispatch launch's body) and zeroes the padding rows
// of the 32-row groups, and the GEMMs run on the block-scaled tiles.
// s_info: kInfoInts ints of LDS.
template <bool MX>
__device__ __forceinline__ void fused_items(const FusedParams& f, const uint8_t* smem, uint32_t lds0, int* s_info,
                                            const FoldArgs* fold) {
  const int E = f.g1.E;
  int32_t* st = f.st;
  const int32_t* mbase = f.fplan;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int xcd = xcd_id();

  // ---- 1. dispatch: each token row read once, written to its routes' rows ------
  // Workgroup b takes the token groups b, b + G, ... of 8 tokens (G the grid
  // size), a wave one token a group.  Its loop keeps the next token's row in
  // flight while it stores the current one's K copies: vector memory
  // operations complete in order, so loads issued after the stores would
  // wait for them.
  {
    constexpr int VB = 16;   // vectors a lane of a row in one pass (rows up to 8192 elements)
    const int D = f.g1.K, nvec = D >> 3;
    uint16_t* xd = reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(f.g1.a));
    const int step = (int)gridDim.x * 8;
    int t = (int)blockIdx.x * 8 + wave;
    if (MX) {
      // padding rows of experts blockIdx.x, + G, ...; then the token rows
      for (int e = blockIdx.x; e < f.g1.E; e += gridDim.x)
        perm::zero_pad_rows_mx(e, f.counts, f.g1.offsets, D, const_cast<uint8_t*>(f.g1.a),
                               const_cast<uint8_t*>(f.g1.as), 8);
      // a wave per row segment of a token
      const int nseg = perm::mx_dispatch_segs(D);
      const int nitems = f.N * nseg;
      for (int i = t; i < nitems; i += step) {
        const int tt = i / nseg;
        perm::dispatch_mx_token(tt, i - tt * nseg, f.x, f.dst_rows, D, f.K, -1, const_cast<uint8_t*>(f.g1.a),
                                const_cast<uint8_t*>(f.g1.as));
      }
    } else if (nvec <= VB * 64) {
      uint4 cur[VB], nxt[VB];
      auto load = [&](uint4 (&r)[VB], int tok) {
        const uint16_t* src = f.x + (int64_t)tok * D;
#pragma unroll
        for (int j = 0; j < VB; ++j) {
          const int v = lane + j * 64;
          if (v < nvec) r[j] = ldg16(src + v * 8);
        }
      };
      if (t < f.N) load(cur, t);
      for (; t < f.N; t += step) {
        if (t + step < f.N) load(nxt, t + step);
        for (int k = 0; k < f.K; ++k) {
          const int dk = f.dst_rows[(int64_t)t * f.K + k];
          if (dk < 0) continue;
#pragma unroll
          for (int j = 0; j < VB; ++j) {
            const int v = lane + j * 64;
            if (v < nvec) stg16(xd + (int64_t)dk * D + v * 8, cur[j]);
          }
        }
#pragma unroll
        for (int j = 0; j < VB; ++j) cur[j] = nxt[j];
      }
    } else {
      for (; t < f.N; t += step) {
        const uint16_t* src = f.x + (int64_t)t * D;
        for (int v0 = 0; v0 < nvec; v0 += VB * 64) {
          uint4 r[VB];
#pragma unroll
          for (int j = 0; j < VB; ++j) {
            const int v = v0 + lane + j * 64;
            if (v < nvec) r[j] = ldg16(src + v * 8);
          }
          for (int k = 0; k < f.K; ++k) {
            const int dk = f.dst_rows[(int64_t)t * f.K + k];
            if (dk < 0) continue;
#pragma unroll
            for (int j = 0; j < VB; ++j) {
              const int v = v0 + lane + j * 64;
              if (v < nvec) stg16(xd + (int64_t)dk * D + v * 8, r[j]);
            }
          }
        }
      }
    }
    __syncthreads();   // the workgroup's stores precede thread 0's release below
    if (tid == 0) __hip_atomic_fetch_add(st + st_disp_done(), f.publish, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- 2. GEMM1 tiles, each after its expert is ready --------------------------
  gemm_phase<true, MX>(f, f.g1, smem, lds0, s_info, xcd, mbase);
  // ---- 3. GEMM2 tiles, each after its GEMM1 row block ---------------------------
  gemm_phase<false, MX>(f, f.g2, smem, lds0, s_info, xcd, mbase);
  if (MX || !fold) return;

  // ---- 4. the fold: out[t] = sum over k of w[t,k] Y[dst[t,k]] -------------------
  // after every workgroup has passed its GEMM2 tiles; a wave per row segment
  // of a token (the combine launch's items), wave w of the grid taking
  // segments w, w + 8G, ...: no claims, and the waves of a workgroup run
  // independently
  __syncthreads();   // the workgroup's stores precede thread 0's release below
  if (tid == 0) {
    __hip_atomic_fetch_add(fold->passed, f.publish, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    s_info[3] = wait_ge(f, fold->passed, (int)gridDim.x);
  }
  __syncthreads();   // thread 0 acquired; the workgroup's loads follow
  if (!s_info[3]) return;   // the wait expired (reported): no fold
  const int nseg = perm::combine_segs(f.g2.N >> 3);
  const int64_t nitems = (int64_t)fold->N * nseg;
  for (int64_t w = (int64_t)blockIdx.x * 8 + wave; w < nitems; w += (int64_t)gridDim.x * 8) {
    const int t = (int)(w / nseg);
    perm::combine_seg<true>(t, (int)(w - (int64_t)t * nseg), nseg, f.g2.c0, fold->dst_rows, fold->weight, f.g2.N,
                            f.K, fold->out, nullptr, nullptr);
  }
}

template <bool MX>
__global__ __launch_bounds__(512) void experts_fwd_fused_kernel(FusedParams f) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[lds_bytes<MX>()];
  __shared__ int s_info[kInfoInts];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  fused_items<MX>(f, smem, lds0, s_info, nullptr);
}

// Fused planner: one workgroup, after the GEMM1 plan (gplan): each expert's
// first row block in the planner's order, the GEMM2 plan in the same expert
// order (fp_* above), and zeroes the queue state (the GEMM2 queue heads
// included) for this launch.  LDS: s_m [THREADS / 64] ints.
template <int THREADS>
__device__ __forceinline__ void plan_fused_body(const int32_t* __restrict__ offsets, int E, int max_mb, int nt2,
                                                const int32_t* __restrict__ gplan, int32_t* __restrict__ fplan,
                                                int32_t* __restrict__ st, int* s_m) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int L = gplan[1];
  int mbs = 0;
  if (t < L) {
    const int e = gplan[2 + t];
    const int m = offsets[e + 1] - offsets[e];
    mbs = (m + rows_bm(m) - 1) / rows_bm(m);
  }
  int incm = mbs;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int b = __shfl_up(incm, o, 64);
    if (lane >= o) incm += b;
  }
  if (lane == 63) s_m[wv] = incm;
  for (int i = t; i < st_ints(max_mb); i += THREADS) st[i] = 0;
  __syncthreads();
  if (t == 0) {
    int rm = 0;
    for (int w = 0; w < THREADS / 64; ++w) {
      const int b = s_m[w];
      s_m[w] = rm;
      rm += b;
    }
    int32_t* plan2 = fplan + fp_plan2(E);
    plan2[0] = rm * nt2;
    plan2[1] = L;
    plan2[2 + E + L] = rm * nt2;
  }
  __syncthreads();
  if (t < L) {
    const int e = gplan[2 + t];
    const int mb0 = incm - mbs + s_m[wv];   // the expert's first row block in planner order
    fplan[e] = mb0;
    int32_t* plan2 = fplan + fp_plan2(E);
    plan2[2 + t] = e;
    plan2[2 + E + t] = mb0 * nt2;
  }
}

__global__ __launch_bounds__(1024) void plan_fused_kernel(const int32_t* __restrict__ offsets, int E, int max_mb,
                                                          int nt2, const int32_t* __restrict__ gplan,
                                                          int32_t* __restrict__ fplan, int32_t* __restrict__ st) {
  __shared__ int s_m[16];
  plan_fused_body<1024>(offsets, E, max_mb, nt2, gplan, fplan, st, s_m);
}

// ---------------------------------------------------------------------------
// Single-launch layer forward (KOSMOS section 3.3 and Figure 6: one launch
// from route to fold; section 3.3.1 steps 1-5), on one GPU.  One persistent
// workgroup per CU runs, in order:
//   1. the router tiles (the same items and contraction split as the router
//      launch, so the same partial sums), and marks every row unused;
//   2. per chunk of 16 tokens: the logits (partials added in split order,
//      then the bias), softmax and top-K, the in-chunk ranks and histogram;
//   3. the histogram scan, one expert a workgroup: each chunk's first row of
//      the expert within its segment, and the expert's count;
//   4. every workgroup the segment offsets from the counts; workgroup 0
//      stores them and builds the GEMM and queue plans while the others
//      scatter every route to its row;
//   5. the readiness-gated queue: the dispatch, GEMM1 tiles after it, GEMM2
//      tiles as their GEMM1 row blocks complete, then the fold, 8 tokens per
//      item.
// Steps 1-4 end at a grid barrier: a counter every workgroup adds to after an
// agent-scope release, waited on (bounded) and acquired.  Every workgroup is
// resident (one per CU), so each barrier is reached by all; a wait that
// expires reports MOE_STATUS_WAIT_EXPIRED and the workgroup stops.  Each
// step computes what its separate launch computes, so the outputs are
// bitwise those of the staged launches.
// ---------------------------------------------------------------------------

struct SingleFwdParams {
  FusedParams f;                // dispatch, GEMM1, GEMM2 (queue state and plans in the workspace)
  FoldArgs fold;
  router::RouterParams rp;      // out: partials [S][N][E] when S > 1, else the logits
  int rbn, r_items;             // router column tile, router items
  const float* bias;            // [E] or null
  float* logits;                // [N][E]
  const uint8_t* drop;          // [N][K] or null
  int N, E, K, renorm, npl, nchunks, align;
  int64_t rows_cap;
  int32_t *topk_idx, *counts, *offsets, *dst_rows, *row_route;
  float* topk_prob;
  int32_t *hist, *rank;         // route workspace: histogram / chunk bases, in-chunk ranks
  int32_t *gplan, *head;        // GEMM plan and queue heads
  int max_mb;
  int32_t* bar;                 // grid barrier counters [4] (zeroed before the launch)
};

// every workgroup: after its stores, add to *bar and wait until all have
__device__ __forceinline__ bool grid_sync(const FusedParams& f, int32_t* bar, int* s_info) {
  __syncthreads();   // the workgroup's stores precede thread 0's release
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(bar, f.publish, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    s_info[3] = wait_ge(f, bar, (int)gridDim.x);
  }
  __syncthreads();   // thread 0 acquired; the workgroup's loads follow
  return s_info[3] != 0;
}

template <int NPL>
__device__ __forceinline__ void topk_single(const SingleFwdParams& p, int c, int* s_sel, int* s_hist) {
  route::topk_chunk<NPL, 512>(c, p.logits, p.drop, p.N, p.E, p.K, p.renorm, p.topk_idx, p.topk_prob, p.hist,
                              p.rank, 0, 0, nullptr, p.f.status, s_sel, s_hist, nullptr);
}

__global__ __launch_bounds__(512) void layer_fwd_single_kernel(SingleFwdParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLdsBytes];
  __shared__ int s_info[kInfoInts];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  const FusedParams& f = p.f;
  const int tid = threadIdx.x;
  const int64_t gthreads = (int64_t)gridDim.x * 512;

  // ---- 1. router tiles; every row unused until the scatter --------------------
  for (int64_t i = (int64_t)blockIdx.x * 512 + tid; i < p.rows_cap; i += gthreads) p.row_route[i] = -1;
  for (int it = blockIdx.x; it < p.r_items; it += gridDim.x) {
    if (p.rbn == 64) router::router_tile_item<128, 64>(p.rp, it, smem, lds0);
    else if (p.rbn == 128) router::router_tile_item<128, 128>(p.rp, it, smem, lds0);
    else router::router_tile_item<128, 256>(p.rp, it, smem, lds0);
  }
  if (!grid_sync(f, p.bar + 0, s_info)) return;

  // ---- 2. logits and top-K, a chunk of 16 tokens at a time ---------------------
  int* s_sel = reinterpret_cast<int*>(smem);
  int* s_hist = s_sel + route::kChunk * 32;
  const int S = p.rp.S;
  for (int c = blockIdx.x; c < p.nchunks; c += gridDim.x) {
    __syncthreads();   // the previous chunk is done with the LDS
    if (S > 1) {
      // the router's reduce, element by element: partials in split order, then the bias
      const int t0 = c * route::kChunk;
      const int nt = min(route::kChunk, p.N - t0);
      const int64_t NE = (int64_t)p.N * p.E;
      if ((p.E & 3) == 0) {
        // four adjacent logits a thread, the same sums element by element
        const int64_t o4 = (int64_t)t0 * p.E / 4, NE4 = NE / 4;
        const f32x4_t* p4 = reinterpret_cast<const f32x4_t*>(p.rp.out);
        for (int i = tid; i < nt * p.E / 4; i += 512) {
          f32x4_t v = p4[o4 + i];
          for (int k = 1; k < S; ++k) v += p4[(int64_t)k * NE4 + o4 + i];
          if (p.bias) {
            const int e = (4 * i) % p.E;
            v += f32x4_t{p.bias[e], p.bias[e + 1], p.bias[e + 2], p.bias[e + 3]};
          }
          reinterpret_cast<f32x4_t*>(p.logits)[o4 + i] = v;
        }
      } else {
        for (int i = tid; i < nt * p.E; i += 512) {
          const int64_t o = (int64_t)t0 * p.E + i;
          float v = p.rp.out[o];
          for (int k = 1; k < S; ++k) v += p.rp.out[(int64_t)k * NE + o];
          if (p.bias) v += p.bias[i % p.E];
          p.logits[o] = v;
        }
      }
      __syncthreads();   // the chunk's logits are visible to every wave of the workgroup
    }
    if (p.npl == 1) topk_single<1>(p, c, s_sel, s_hist);
    else if (p.npl == 2) topk_single<2>(p, c, s_sel, s_hist);
    else if (p.npl == 4) topk_single<4>(p, c, s_sel, s_hist);
    else topk_single<8>(p, c, s_sel, s_hist);
  }
  if (!grid_sync(f, p.bar + 1, s_info)) return;

  // ---- 3. the histogram scan, an expert a workgroup ------------------------------
  {
    int* s_w = reinterpret_cast<int*>(smem);
    for (int e = blockIdx.x; e < p.E; e += gridDim.x)
      route::scan_expert<512>(p.hist, p.nchunks, p.E, e, p.counts, s_w);
  }
  if (!grid_sync(f, p.bar + 2, s_info)) return;

  // ---- 4. segment offsets (every workgroup), the scatter; workgroup 0 the plans --
  {
    int* w = reinterpret_cast<int*>(smem);
    int *s_off = w, *s_wsum = w + 1024;
    route::offsets_of<512>(p.counts, p.E, p.align, s_off, s_wsum);
    if (blockIdx.x == 0) {
      for (int e = tid; e <= p.E; e += 512) p.offsets[e] = s_off[e];
      __syncthreads();   // offsets written by this workgroup, read by its planners below
      int *s_w0 = w + 2048, *s_w1 = w + 2064, *s_tot2 = w + 2080, *s_pref = w + 2096;
      float* s_key = reinterpret_cast<float*>(w + 2560);
      int *s_items = w + 3072, *s_ids = w + 3584;
      sched::plan_rows_body<512>(p.offsets, p.E, f.nt1, p.gplan, p.head, s_w0, s_w1, s_tot2, s_key, s_items,
                                 s_ids, s_pref);
      __syncthreads();   // the GEMM plan, read by the queue plan
      plan_fused_body<512>(p.offsets, p.E, p.max_mb, f.nt2, p.gplan, const_cast<int32_t*>(f.fplan), f.st,
                           w + 4112);
    }
    // the other workgroups scatter every route to its row (all of them when
    // the grid is one workgroup)
    const int g0 = gridDim.x > 1 ? 1 : 0;
    const int64_t NK = (int64_t)p.N * p.K;
    const int64_t nth = (int64_t)(gridDim.x - g0) * 512;
    if ((int)blockIdx.x >= g0)
      for (int64_t r = (int64_t)(blockIdx.x - g0) * 512 + tid; r < NK; r += nth)
        route::scatter_route_seg(r, p.topk_idx, p.drop, p.hist, s_off, p.rank, p.K, p.E, p.dst_rows,
                                 p.row_route);
  }
  if (!grid_sync(f, p.bar + 3, s_info)) return;

  // ---- 5. dispatch, GEMM1, GEMM2 by readiness, then the fold ------------------
  fused_items<false>(f, smem, lds0, s_info, &p.fold);
}

__global__ void single_reset_kernel(int32_t* bar, int n, int32_t* status) {
  if ((int)threadIdx.x < n) bar[threadIdx.x] = 0;
  if (threadIdx.x == 0 && status) *status = 0;
}

}  // namespace

size_t gemm_fwd_plan_ints(int64_t E) { return (size_t)(4 + 2 * E + 64); }

namespace {
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
}  // namespace

// bf16: K % 64 == 0 (whole 128-byte steps), N % 16 == 0; MXFP8: K % 128 == 0,
// N % 32 == 0.  One expert's weight matrix under 2 GiB (32-bit DMA offsets);
// operands 16-byte aligned, scales 4-byte aligned.
bool gemm_fwd_fast_ok(const GemmFwd& f, bool mx) {
  if (f.k_dim % (mx ? 128 : 64) || f.n_dim % (mx ? 32 : 16)) return false;
  if (f.dswiglu && (!mx || f.swiglu || !aligned(f.g, 8) || !aligned(f.u, 8) || !aligned(f.c0, 8) ||
                    !aligned(f.c1, 8) || !aligned(f.act_q, 4)))
    return false;
  if (f.n_dim * f.k_dim * (mx ? 1 : 2) >= (int64_t(1) << 31)) return false;   // 32-bit DMA offsets
  if (!aligned(f.a, 16) || !aligned(f.b0, 16) || (f.swiglu && !aligned(f.b1, 16))) return false;
  if (mx && (!aligned(f.a_scales, 4) || !aligned(f.b0_scales, 4) || (f.swiglu && !aligned(f.b1_scales, 4))))
    return false;
  return true;
}

bool gemm_fwd_fast_ok(int64_t k_dim, int64_t n_dim) {
  return k_dim % tile::kBK == 0 && n_dim % 16 == 0 && n_dim * k_dim * 2 < (int64_t(1) << 31);
}

hipError_t launch_gemm_fwd_fast(const GemmFwd& f, bool mx, int32_t* ws, hipStream_t s) {
  FwdParams p{};
  p.offsets = f.offsets;
  p.E = (int)f.E;
  p.N = (int)f.n_dim;
  p.K = (int)f.k_dim;
  p.nk = (int)(f.k_dim * (mx ? 1 : 2) / tile::kRB);
  p.a = (const uint8_t*)f.a;
  p.b0 = (const uint8_t*)f.b0;
  p.b1 = (const uint8_t*)f.b1;
  p.as = f.a_scales;
  p.bs0 = f.b0_scales;
  p.bs1 = f.b1_scales;
  p.c0 = (uint16_t*)f.c0;
  p.c1 = (uint16_t*)f.c1;
  p.c2 = (uint16_t*)f.act;
  p.hq = (mx && (f.swiglu || f.dswiglu)) ? f.act_q : nullptr;   // bf16 callers quantize H separately
  p.hs = (mx && (f.swiglu || f.dswiglu)) ? f.act_scales : nullptr;
  p.g = (const uint16_t*)f.g;
  p.u = (const uint16_t*)f.u;
  p.head = ws;
  int32_t* plan = ws + kGemmHeadInts;
  p.plan = plan;
  const int ncol = f.swiglu ? BigTile<true>::NCOL : BigTile<false>::NCOL;
  p.n_tiles = (p.N + ncol - 1) / ncol;
  if (mx && f.dswiglu) return run_fwd<false, true, true>(p, plan, s);
  if (mx) return f.swiglu ? run_fwd<true, true>(p, plan, s) : run_fwd<false, true>(p, plan, s);
  return f.swiglu ? run_fwd<true, false>(p, plan, s) : run_fwd<false, false>(p, plan, s);
}

// Workspace of the fused forward: GEMM plan, fused plan and queue state.
size_t experts_fused_ws_ints(int64_t rows_cap, int64_t E) {
  const int64_t max_mb = rows_cap / 128 + E + 1;
  return (size_t)(kGemmHeadInts + gemm_fwd_plan_ints(E) + fp_ints((int)E) + st_ints((int)max_mb) + 96);
}

namespace {
// the fused queue's parameters and the places of its plans in the workspace
void fused_params(const ExpertsFwd& x, int32_t* ws, FusedParams& f, int32_t** gplan_out, int* max_mb_out,
                  int32_t** bar_out) {
  f = FusedParams{};
  FwdParams& g1 = f.g1;
  g1.offsets = x.offsets;
  g1.E = (int)x.E;
  g1.N = (int)x.H;
  g1.K = (int)x.D;
  g1.nk = (int)(x.D * 2 / tile::kRB);
  g1.a = (const uint8_t*)x.xd;
  g1.b0 = (const uint8_t*)x.w_gate;
  g1.b1 = (const uint8_t*)x.w_up;
  g1.c0 = (uint16_t*)x.g;
  g1.c1 = (uint16_t*)x.u;
  g1.c2 = (uint16_t*)x.h;
  FwdParams& g2 = f.g2;
  g2.offsets = x.offsets;
  g2.E = (int)x.E;
  g2.N = (int)x.D;
  g2.K = (int)x.H;
  g2.nk = (int)(x.H * 2 / tile::kRB);
  g2.a = (const uint8_t*)x.h;
  g2.b0 = (const uint8_t*)x.w_down;
  g2.c0 = (uint16_t*)x.y;
  if (x.mx) {
    // E4M3 operands (a step is 128 values), E8M0 scales; GEMM1 stores G, U
    // and H quantized (no bf16 H), GEMM2 reads the quantized H
    g1.nk = (int)(x.D / tile::kRB);
    g1.as = x.xd_s;
    g1.bs0 = x.wg_s;
    g1.bs1 = x.wu_s;
    g1.c2 = nullptr;
    g1.hq = x.h_q;
    g1.hs = x.h_s;
    g2.nk = (int)(x.H / tile::kRB);
    g2.a = x.h_q;
    g2.as = x.h_s;
    g2.bs0 = x.wd_s;
  }
  f.x = (const uint16_t*)x.x;
  f.dst_rows = x.dst_rows;
  f.counts = x.counts;
  f.N = (int)x.N_tokens;
  f.K = (int)x.K;
  f.nt1 = (int)((x.H + BigTile<true>::NCOL - 1) / BigTile<true>::NCOL);
  f.nt2 = (int)((x.D + BigTile<false>::NCOL - 1) / BigTile<false>::NCOL);
  // workspace: GEMM1 queue heads, GEMM1 plan, fused plan (GEMM2 plan in it),
  // queue state (GEMM2 queue heads first, 128-byte aligned), then the single
  // launch's barrier words
  int32_t* gplan = ws + kGemmHeadInts;
  int32_t* fplan = gplan + gemm_fwd_plan_ints(x.E);
  int32_t* st = fplan + fp_ints((int)x.E);
  st = (int32_t*)(((uintptr_t)st + 127) & ~(uintptr_t)127);
  const int max_mb = (int)(x.rows_cap / 128 + x.E + 1);
  g1.plan = gplan;
  g1.head = ws;
  g2.plan = fplan + fp_plan2((int)x.E);
  g2.head = st;
  g1.n_tiles = f.nt1;
  g2.n_tiles = f.nt2;
  f.st = st;
  f.fplan = fplan;
  f.status = x.status;
  f.polls = x.test_polls > 0 ? x.test_polls : kSpinLimit;
  f.publish = x.test_polls > 0 ? 0 : 1;
  *gplan_out = gplan;
  *max_mb_out = max_mb;
  // the single launch's barrier words: after the queue state, in the
  // workspace's slack (experts_fused_ws_ints)
  int32_t* bar = st + st_ints(max_mb);
  *bar_out = (int32_t*)(((uintptr_t)bar + 31) & ~(uintptr_t)31);
}

hipError_t resident_grid(const void* kern, int* grid) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err == hipSuccess) err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 512, 0);
  if (per_cu < 1) per_cu = 1;
  *grid = cus * per_cu;
  return err;
}
}  // namespace

hipError_t launch_experts_fwd_fused(const ExpertsFwd& x, int32_t* ws, hipStream_t s) {
  FusedParams f;
  int32_t* gplan = nullptr;
  int32_t* bar = nullptr;
  int max_mb = 0;
  fused_params(x, ws, f, &gplan, &max_mb, &bar);
  plan_rows_kernel<<<1, 1024, 0, s>>>(x.offsets, (int)x.E, f.nt1, gplan, ws);
  plan_fused_kernel<<<1, 1024, 0, s>>>(x.offsets, (int)x.E, max_mb, f.nt2, gplan, const_cast<int32_t*>(f.fplan),
                                       f.st);
  int grid = 0;
  const void* kern = x.mx ? (const void*)experts_fwd_fused_kernel<true> : (const void*)experts_fwd_fused_kernel<false>;
  hipError_t err = resident_grid(kern, &grid);
  if (err != hipSuccess) return err;
  if (x.mx) experts_fwd_fused_kernel<true><<<grid, 512, 0, s>>>(f);
  else experts_fwd_fused_kernel<false><<<grid, 512, 0, s>>>(f);
  return hipGetLastError();
}

bool layer_fwd_single_ok(int64_t D, int64_t E, int64_t K) {
  return router::router_tiled(D, E) && E <= 512 && K <= 32;
}

hipError_t launch_layer_fwd_single(const LayerFwdSingle& a, int32_t* ws, void* route_ws, void* router_ws,
                                   hipStream_t s) {
  const ExpertsFwd& x = a.x;
  if (!layer_fwd_single_ok(x.D, x.E, x.K)) return hipErrorInvalidValue;
  SingleFwdParams p{};
  int32_t* bar = nullptr;
  fused_params(x, ws, p.f, &p.gplan, &p.max_mb, &bar);
  p.head = ws;
  p.bar = bar;
  const router::RouterPlan r = router::router_plan(x.N_tokens, x.D, x.E);
  p.rp = router::RouterParams{(const uint16_t*)a.x_tokens, (const uint16_t*)a.w_r, a.bias,
                              r.S > 1 ? (float*)router_ws : a.logits, (int)x.N_tokens, (int)x.D, (int)x.E, r.S,
                              (int)((x.N_tokens + 127) / 128), r.ntiles};
  p.rbn = r.bn;
  p.r_items = (int)(((x.N_tokens + 127) / 128) * r.ntiles * r.S);
  p.bias = a.bias;
  p.logits = a.logits;
  p.drop = a.drop;
  p.N = (int)x.N_tokens;
  p.E = (int)x.E;
  p.K = (int)x.K;
  p.renorm = a.renorm;
  int npl = 1;
  while (npl * kWave < x.E) npl <<= 1;
  p.npl = npl;
  p.nchunks = (int)((x.N_tokens + route::kChunk - 1) / route::kChunk);
  p.align = 1;
  p.rows_cap = x.rows_cap;
  p.topk_idx = a.topk_idx;
  p.topk_prob = a.topk_prob;
  p.counts = a.counts;
  p.offsets = const_cast<int32_t*>(x.offsets);
  p.dst_rows = a.dst_rows;
  p.row_route = const_cast<int32_t*>(x.row_route);
  p.hist = (int32_t*)route_ws;
  p.rank = (int32_t*)((char*)route_ws + route::hist_bytes(x.N_tokens, x.E));
  p.fold = FoldArgs{a.dst_rows, a.topk_prob, (int)x.N_tokens, (uint16_t*)a.out, bar + 4};
  int grid = 0;
  hipError_t err = resident_grid((const void*)layer_fwd_single_kernel, &grid);
  if (err != hipSuccess) return err;
  single_reset_kernel<<<1, 64, 0, s>>>(bar, 5, x.status);
  layer_fwd_single_kernel<<<grid, 512, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
