// Shared MFMA tile engine of the grouped GEMMs and the router GEMM (gfx950).
//
// Operand tiles go from global memory straight into an NS-stage LDS ring with
// global_load_lds_dwordx4 (each wave instruction writes 1 KB: 64 lanes x 16
// bytes at consecutive LDS addresses from M0), so no registers stage the
// copies and NS-1 contraction steps are in flight while the MFMAs of the
// current one run.  The loads are issued from inline assembly and their
// completion is tracked with explicit vmcnt waits: the vector-memory loads of
// a wave complete in issue order, so "at most n outstanding" after the loads
// of n later steps were issued means every older step has landed.  LDS rows
// hold 64 bf16 (128 bytes); chunk c of row r sits at slot c ^ (r & 7), which,
// measured on gfx950, keeps the 16-row fragment reads (ds_read_b128) free of
// bank conflicts; each lane fetches the global chunk that belongs at its LDS
// slot.  MFMA operands are fed swapped (B tile as the instruction's first
// operand), so each lane's four accumulators are four consecutive output
// columns of one row.
//
// The same ring carries MXFP8 operands (TileCfg MX): an LDS row is then 128
// E4M3 values, one step of the scaled 16x16x128 MFMA, and a lane's two
// 16-byte chunks (lg and 4 + lg) are exactly that instruction's bytes 0..15
// and 16..31.  Each stage also holds the E8M0 scales of the step: 4 bytes
// (blocks of 32) per tile row, loaded with one global_load_lds_dword per wave
// (64 rows each, A rows first, then B rows, then unused padding up to 512).
#pragma once

#include "common.h"

namespace moe {
namespace tile {

constexpr int kBK = 64;          // contraction step (bf16 elements)
constexpr int kRB = kBK * 2;     // bytes per LDS row (also 128 E4M3 values)
constexpr int kScRows = 512;     // rows of the per-stage scale area (MX)

__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr), "v"(g) : "memory");
}

// 4 bytes per lane: LDS address M0 + 4 * lane
__device__ __forceinline__ void lds_dma4(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_addr), "v"(g) : "memory");
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

template <int BM_, int BN_, int NS_, int WAVES_M, int WAVES_N, bool DUAL_, bool MX_ = false>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, NS = NS_;
  static constexpr bool DUAL = DUAL_, MX = MX_;
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int WAVES_N_ = WAVES_N;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 16, TN = WN / 16;
  static constexpr int RPI = 1024 / kRB;                           // rows per DMA instruction
  static constexpr int A_BYTES = BM * kRB, SC_OFF = (BM + BN) * kRB;
  static constexpr int STAGE = SC_OFF + (MX ? kScRows * 4 : 0);
  static constexpr int A_INS = BM / RPI / NW, B_INS = BN / RPI / NW;   // per wave per step
  static constexpr int LPS = A_INS + B_INS + (MX ? 1 : 0);
  static constexpr int NCOL = DUAL ? BN / 2 : BN;                  // output columns per tile
  static_assert(A_INS * RPI * NW == BM && B_INS * RPI * NW == BN, "even DMA split");
  static_assert(WM % 16 == 0 && WN % 16 == 0 && (!DUAL || TN % 2 == 0), "wave tile");
  static_assert(NS >= 2 && NS * STAGE <= 160 * 1024, "LDS ring");
  static_assert(!MX || (NW * 64 == kScRows && BM + BN <= kScRows), "one scale load per wave");
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

// This lane's place in a DMA instruction: the tile row of the q-th load of
// wave `wave` (ROWS_PER_WAVE = INS * RPI rows per wave) and the global chunk
// that belongs at its slot (slot_of is an involution in c).
__device__ __forceinline__ int dma_row(int wave, int ins, int q) { return (wave * ins + q) * (1024 / kRB) + ((threadIdx.x & 63) >> 3); }
__device__ __forceinline__ int dma_chunk() {
  const int lane = threadIdx.x & 63;
  return slot_of(lane >> 3, lane & 7);
}

// Issue the DMA loads of contraction step kt into its ring stage.
// a_src[q] / b_src[q] point at this lane's 16-byte chunk of its q-th DMA row
// at the first step; step kt reads kt * kRB bytes further.  MX: s_src points
// at the 4 scale bytes of this lane's scale row at the first step.
template <class C>
__device__ __forceinline__ void issue_step(uint32_t lds0, const uint8_t* const* a_src, const uint8_t* const* b_src,
                                           const uint8_t* s_src, int kt) {
  const int wave = threadIdx.x >> 6;
  const uint32_t st = lds0 + (uint32_t)((kt % C::NS) * C::STAGE);
  const uint32_t wave_a = st + (uint32_t)(wave * C::A_INS) * 1024u;
  const uint32_t wave_b = st + (uint32_t)C::A_BYTES + (uint32_t)(wave * C::B_INS) * 1024u;
  const int64_t ko = (int64_t)kt * kRB;
#pragma unroll
  for (int q = 0; q < C::A_INS; ++q) lds_dma16(a_src[q] + ko, __builtin_amdgcn_readfirstlane(wave_a + q * 1024u));
#pragma unroll
  for (int q = 0; q < C::B_INS; ++q) lds_dma16(b_src[q] + ko, __builtin_amdgcn_readfirstlane(wave_b + q * 1024u));
  if constexpr (C::MX)
    lds_dma4(s_src + (int64_t)kt * 4, __builtin_amdgcn_readfirstlane(st + (uint32_t)C::SC_OFF + wave * 256u));
}

// Issue the first NS-1 steps (the ring must be free).
template <class C>
__device__ __forceinline__ void prologue(uint32_t lds0, const uint8_t* const* a_src, const uint8_t* const* b_src,
                                         const uint8_t* s_src, int nk) {
#pragma unroll
  for (int s = 0; s < C::NS - 1; ++s)
    if (s < nk) issue_step<C>(lds0, a_src, b_src, s_src, s);
}

// Main loop: acc = A[rows, k] . B[cols, k]^T over nk contraction steps, the
// prologue already issued.  The ring is free again when this returns; vector
// stores issued after the prologue only make the first waits stricter.
template <class C>
__device__ __forceinline__ void mainloop(const uint8_t* smem, uint32_t lds0, const uint8_t* const* a_src,
                                         const uint8_t* const* b_src, int nk,
                                         f32x4_t (&acc)[C::TM][C::TN]) {
  static_assert(!C::MX, "bf16 tiles");
  constexpr int TM = C::TM, TN = C::TN, WM = C::WM, NS = C::NS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N_, wn = wave % C::WAVES_N_;
  const int l16 = lane & 15, lg = lane >> 4;
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
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int kt = 0; kt < nk; ++kt) {
    wait_steps<C::LPS, NS - 2>(min(NS - 2, nk - 1 - kt));
    __syncthreads();   // step kt landed for every wave; every wave is done with step kt-1
    if (kt + NS - 1 < nk) issue_step<C>(lds0, a_src, b_src, nullptr, kt + NS - 1);
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
}

// MXFP8 main loop: one scaled MFMA per fragment pair per step.  Tile rows
// that differ by a multiple of 8 share a swizzle, so every fragment offset is
// a per-lane base plus a constant.  Lane group lg reads chunks lg and 4 + lg
// of its row (slots s and s ^ 4) and the scale byte of block lg.
template <class C>
__device__ __forceinline__ void mainloop_mx(const uint8_t* smem, uint32_t lds0, const uint8_t* const* a_src,
                                            const uint8_t* const* b_src, const uint8_t* s_src, int nk,
                                            f32x4_t (&acc)[C::TM][C::TN]) {
  static_assert(C::MX, "MXFP8 tiles");
  constexpr int TM = C::TM, TN = C::TN, WM = C::WM, NS = C::NS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N_, wn = wave % C::WAVES_N_;
  const int l16 = lane & 15, lg = lane >> 4;
  const int sw = (lg ^ (l16 & 7)) << 4;
  const int a_base = (wm * WM + l16) * kRB + sw;
  const int b_base = C::A_BYTES + l16 * kRB + sw;
  const int as_base = C::SC_OFF + (wm * WM + l16) * 4 + lg;
  const int bs_base = C::SC_OFF + (C::BM + l16) * 4 + lg;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int kt = 0; kt < nk; ++kt) {
    wait_steps<C::LPS, NS - 2>(min(NS - 2, nk - 1 - kt));
    __syncthreads();   // step kt landed for every wave; every wave is done with step kt-1
    if (kt + NS - 1 < nk) issue_step<C>(lds0, a_src, b_src, s_src, kt + NS - 1);
    const uint8_t* st = smem + (kt % NS) * C::STAGE;
    i32x8_t af[TM];
    int sa[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int off = a_base + i * 16 * kRB;
      const uint4 lo = *reinterpret_cast<const uint4*>(st + off);
      const uint4 hi = *reinterpret_cast<const uint4*>(st + (off ^ 64));
      af[i] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      sa[i] = st[as_base + i * 64];
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int br = b_row<C>(wn, j);
      const int off = b_base + br * kRB;
      const uint4 lo = *reinterpret_cast<const uint4*>(st + off);
      const uint4 hi = *reinterpret_cast<const uint4*>(st + (off ^ 64));
      const i32x8_t bf{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      const int sb = st[bs_base + br * 4];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af[i], acc[i][j], 0, 0, 0, sb, 0, sa[i]);
    }
  }
  __syncthreads();   // every wave is done reading the ring before it is refilled
}

}  // namespace tile
}  // namespace moe
