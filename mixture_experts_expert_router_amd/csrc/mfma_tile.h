// Shared MFMA tile engine of the grouped GEMMs and the router GEMM (gfx950).
//
// Operand tiles go from global memory straight into an NS-stage LDS ring with
// global_load_lds_dwordx4 (each wave instruction writes 1 KB: 64 lanes x 16
// bytes at consecutive LDS addresses from M0), so no registers stage the
// copies and NS-1 contraction steps are in flight while the MFMAs of the
// current one run.  The loads are issued from inline assembly and their
// completion is tracked with explicit vmcnt waits: the vector-memory loads of
// a wave complete in issue order, so "at most n outstanding" after the loads
// of n later steps were issued means every older step has landed.  Each load
// takes a wave-uniform 64-bit base in SGPRs (advanced by one step with a
// scalar add) and a 32-bit per-lane byte offset, which keeps the address
// registers of a tile to one VGPR per load.
//
// LDS rows hold 128 bytes (64 bf16); chunk c of row r sits at slot
// c ^ (r & 7), which, measured on gfx950, keeps the 16-row fragment reads
// (ds_read_b128) free of bank conflicts; each lane fetches the global chunk
// that belongs at its LDS slot.  Fragment rows are 16-row aligned, so every
// fragment address is one per-lane base plus a compile-time offset.  MFMA
// operands are fed swapped (B tile as the instruction's first operand), so
// each lane's four accumulators are four consecutive output columns of one
// row.
//
// The same ring carries MXFP8 operands (TileCfg MX): an LDS row is then 128
// E4M3 values, one step of the scaled 16x16x128 MFMA, and a lane's two
// 16-byte chunks (lg and 4 + lg) are exactly that instruction's bytes 0..15
// and 16..31.  The E8M0 scales (4 bytes, blocks of 32, per tile row and step)
// travel in groups of 4 steps: 16 bytes per tile row, A rows then B rows,
// loaded with global_load_lds_dword (4 lanes per row, 16 rows per wave
// instruction, so an instruction touches 16 rows instead of 64) into two
// alternating group buffers after the ring.  The group of steps 4g..4g+3 is
// issued with step 4g's loads and lands with them.
#pragma once

#include "common.h"

namespace moe {
namespace tile {

constexpr int kBK = 64;          // contraction step (bf16 elements)
constexpr int kRB = kBK * 2;     // bytes per LDS row (also 128 E4M3 values)
constexpr int kScG = 4;          // steps per MXFP8 scale group

// 16 bytes per lane: LDS address M0 + 16 * lane
__device__ __forceinline__ void lds_dma16(const uint8_t* base, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_addr), "v"(off), "s"(base)
               : "memory");
}

// 4 bytes per lane: LDS address M0 + 4 * lane
__device__ __forceinline__ void lds_dma4(const uint8_t* base, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds_addr), "v"(off), "s"(base)
               : "memory");
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

// a pointer every lane holds the same value of, moved to SGPRs
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int slot_of(int r, int c) { return c ^ (r & 7); }

template <int BM_, int BN_, int NS_, int WAVES_M, int WAVES_N, bool DUAL_, bool MX_ = false, bool AT_ = false,
          bool BT_ = false>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, NS = NS_;
  static constexpr bool DUAL = DUAL_, MX = MX_;
  static constexpr bool AT = AT_, BT = BT_;   // operand stored k-major (transposed), see below
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int WAVES_N_ = WAVES_N;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 16, TN = WN / 16;
  static constexpr int WNB = DUAL ? WN / 2 : WN;                   // B rows per wave per half
  static constexpr int RPI = 1024 / kRB;                           // rows per DMA instruction
  static constexpr int A_BYTES = BM * kRB, STAGE = (BM + BN) * kRB;
  // A rows are loaded by A_WAVES waves: all of them, unless the tile has fewer
  // A rows than one DMA instruction per wave covers (a 32-row tile: waves
  // 0-3 load A, waves 4-7 only B)
  static constexpr int A_WAVES = (BM / RPI) < NW ? BM / RPI : NW;
  static constexpr int A_INS = BM / RPI / A_WAVES, B_INS = BN / RPI / NW;   // per loading wave per step
  static constexpr int LPS = A_INS + B_INS;                        // loads per step of a wave that loads A
  static constexpr int LPS_NOA = B_INS;                            // of a wave that does not
  // MX scale groups: 16 bytes per tile row (rows past BM + BN are padding
  // that reloads an A row), SCI loads of 16 rows per wave
  static constexpr int SC_ROWS = (BM + BN + NW * 16 - 1) / (NW * 16) * (NW * 16);
  static constexpr int SG_BYTES = SC_ROWS * 16;
  static constexpr int SRW = SC_ROWS / NW;                         // scale rows per wave
  static constexpr int SCI = MX ? SRW / 16 : 0;
  static constexpr int SC_BASE = NS * STAGE;                        // group buffers after the ring
  static constexpr int LDS = NS * STAGE + (MX ? 2 * SG_BYTES : 0);
  static constexpr int NCOL = DUAL ? BN / 2 : BN;                  // output columns per tile
  static_assert(A_WAVES >= 1 && A_INS * RPI * A_WAVES == BM && B_INS * RPI * NW == BN, "even DMA split");
  static_assert(WM % 16 == 0 && WN % 16 == 0 && (!DUAL || TN % 2 == 0), "wave tile");
  static_assert(!DUAL || (BN / 2) % (B_INS * RPI) == 0, "a wave's B rows are all gate or all up");
  static_assert(NS >= 2 && LDS <= 160 * 1024 - 64, "LDS ring");
  static_assert(!MX || (SRW % 16 == 0 && BM % 16 == 0 && (BN / 2) % 16 == 0 && NS <= 3),
                "whole 16-row scale loads, each from one operand; at most one step in flight past the current");
  static_assert((!AT || BM % 64 == 0) && (!BT || BN % 64 == 0) && !((AT || BT) && (MX || DUAL)),
                "k-major tiles: whole 64-column blocks, bf16, single B");
};

// Row of the B tile that B fragment j of a wave reads, less the wave's own
// offset wn * WNB.  DUAL: gate rows [0, BN/2), up rows [BN/2, BN); a wave
// holds TN/2 gate and TN/2 up fragments of the same output columns.
template <class C>
constexpr int b_frag_row(int j) {
  if (!C::DUAL) return j * 16;
  return j < C::TN / 2 ? j * 16 : C::BN / 2 + (j - C::TN / 2) * 16;
}

// This lane's place in a DMA instruction: the tile row of the q-th load of
// wave `wave` (ins loads per wave per operand) and the global chunk that
// belongs at its slot (slot_of is an involution in c).
__device__ __forceinline__ int dma_row(int wave, int ins, int q) { return (wave * ins + q) * (1024 / kRB) + ((threadIdx.x & 63) >> 3); }
__device__ __forceinline__ int dma_chunk() {
  const int lane = threadIdx.x & 63;
  return slot_of(lane >> 3, lane & 7);
}

// DMA sources of one tile at its first contraction step: wave-uniform bases
// and this lane's byte offsets from them (A rows, this wave's B rows, and
// for MX this thread's scale row).
template <class C>
struct Src {
  const uint8_t* a;
  const uint8_t* b;
  uint32_t a_off[C::A_INS];
  uint32_t b_off[C::B_INS];
  // MX: per scale load q of this wave (uniform): base, the row of lane group
  // 0 relative to it, the last valid row (later rows reload it), row bytes
  const uint8_t* s[C::SCI > 0 ? C::SCI : 1];
  int s_row0[C::SCI > 0 ? C::SCI : 1];
  int s_lim[C::SCI > 0 ? C::SCI : 1];
  int s_ks;
};

// Issue the DMA loads of contraction step kt into its ring stage (MX: with
// the scale group of steps kt..kt+3 first when kt % 4 == 0; a lane's dword
// past the last step reloads the last step's).
template <class C>
__device__ __forceinline__ void issue_step(uint32_t lds0, const Src<C>& src, int kt, int nk) {
  const int wave = threadIdx.x >> 6;
  if constexpr (C::MX) {
    if (kt % kScG == 0) {
      const int lane = threadIdx.x & 63;
      const int g = kt / kScG;
      const uint32_t dst = lds0 + (uint32_t)(C::SC_BASE + (g & 1) * C::SG_BYTES + wave * C::SRW * 16);
      const int d = min(g * kScG + (lane & 3), nk - 1);
#pragma unroll
      for (int q = 0; q < C::SCI; ++q) {
        const int row = min(src.s_row0[q] + (lane >> 2), src.s_lim[q]);
        lds_dma4(src.s[q], (uint32_t)(row * src.s_ks + d * 4), __builtin_amdgcn_readfirstlane(dst + q * 256u));
      }
    }
  }
  const uint32_t st = lds0 + (uint32_t)((kt % C::NS) * C::STAGE);
  const uint32_t wave_a = st + (uint32_t)(wave * C::A_INS) * 1024u;
  const uint32_t wave_b = st + (uint32_t)C::A_BYTES + (uint32_t)(wave * C::B_INS) * 1024u;
  const int64_t ko = (int64_t)kt * kRB;
  const uint8_t* a = src.a + ko;
  const uint8_t* b = src.b + ko;
  // a wave-uniform (scalar) test, so a wave that loads no A rows issues no
  // A instruction at all and its vmcnt counts only its B loads
  if (C::A_WAVES == C::NW || __builtin_amdgcn_readfirstlane(wave) < C::A_WAVES) {
#pragma unroll
    for (int q = 0; q < C::A_INS; ++q) lds_dma16(a, src.a_off[q], __builtin_amdgcn_readfirstlane(wave_a + q * 1024u));
  }
#pragma unroll
  for (int q = 0; q < C::B_INS; ++q) lds_dma16(b, src.b_off[q], __builtin_amdgcn_readfirstlane(wave_b + q * 1024u));
}

// Issue the first NS-1 steps (the ring must be free).
template <class C>
__device__ __forceinline__ void prologue(uint32_t lds0, const Src<C>& src, int nk) {
#pragma unroll
  for (int s = 0; s < C::NS - 1; ++s)
    if (s < nk) issue_step<C>(lds0, src, s, nk);
}

// Per-lane LDS fragment bases: chunk lg (lo) and chunk 4 + lg (hi) of the
// lane's first A row and first B row; the two differ in bit 6 only.
template <class C>
struct FragBase {
  uint32_t a_lo, a_hi, b_lo, b_hi;
  __device__ __forceinline__ FragBase() {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / C::WAVES_N_, wn = wave % C::WAVES_N_;
    const int l16 = lane & 15, lg = lane >> 4;
    const uint32_t sw = (uint32_t)((lg ^ (l16 & 7)) << 4);
    a_lo = (uint32_t)((wm * C::WM + l16) * kRB) + sw;
    b_lo = (uint32_t)(C::A_BYTES + (wn * C::WNB + l16) * kRB) + sw;
    a_hi = a_lo ^ 64u;
    b_hi = b_lo ^ 64u;
  }
};

// Main loop: acc = A[rows, k] . B[cols, k]^T over nk contraction steps, the
// prologue already issued.  The ring is free again when this returns; vector
// stores issued after the prologue only make the first waits stricter.
template <class C>
__device__ __forceinline__ void mainloop(const uint8_t* smem, uint32_t lds0, const Src<C>& src, int nk,
                                         f32x4_t (&acc)[C::TM][C::TN]) {
  static_assert(!C::MX, "bf16 tiles");
  constexpr int TM = C::TM, TN = C::TN, NS = C::NS;
  const FragBase<C> fb;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bool loads_a = C::A_WAVES == C::NW || __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) < C::A_WAVES;
  for (int kt = 0; kt < nk; ++kt) {
    if (loads_a) wait_steps<C::LPS, NS - 2>(min(NS - 2, nk - 1 - kt));
    else wait_steps<C::LPS_NOA, NS - 2>(min(NS - 2, nk - 1 - kt));
    __syncthreads();   // step kt landed for every wave; every wave is done with step kt-1
    if (kt + NS - 1 < nk) issue_step<C>(lds0, src, kt + NS - 1, nk);
    const uint8_t* st = smem + (kt % NS) * C::STAGE;
    // dual-B tiles: MFMAs at raised wave priority, so the other wave of the
    // SIMD issues its fragment reads while these run (measured +3% on the
    // gate/up GEMM, -3% on single-B tiles)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint8_t* sa = st + (ks ? fb.a_hi : fb.a_lo);
      const uint8_t* sb = st + (ks ? fb.b_hi : fb.b_lo);
      bf16x8_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const bf16x8_t*>(sa + i * 16 * kRB);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = *reinterpret_cast<const bf16x8_t*>(sb + b_frag_row<C>(j) * kRB);
      if constexpr (C::DUAL) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
      if constexpr (C::DUAL) __builtin_amdgcn_s_setprio(0);
    }
  }
  __syncthreads();   // every wave is done reading the ring before it is refilled
}

__device__ __forceinline__ i32x8_t load_frag8(const uint8_t* lo, const uint8_t* hi) {
  const uint4 l = *reinterpret_cast<const uint4*>(lo);
  const uint4 h = *reinterpret_cast<const uint4*>(hi);
  return i32x8_t{(int)l.x, (int)l.y, (int)l.z, (int)l.w, (int)h.x, (int)h.y, (int)h.z, (int)h.w};
}

// Wait until step kt of an MXFP8 tile has landed (NS <= 3: at most step
// kt+1 was issued after it, with its scale group when kt+1 starts one).
template <class C>
__device__ __forceinline__ void wait_step_mx(int kt, int nk) {
  if (C::NS == 2 || kt + 1 >= nk) wait_vmcnt<0>();
  else if ((kt + 1) % kScG == 0) wait_vmcnt<C::LPS + C::SCI>();
  else wait_vmcnt<C::LPS>();
}

// MXFP8 main loop: one scaled MFMA per fragment pair per step.  Lane group
// lg reads chunks lg and 4 + lg of its row and the scale byte of block lg.
// All A fragments of the step are read first; B fragments are read one
// ahead of the MFMAs that use them.
template <class C>
__device__ __forceinline__ void mainloop_mx(const uint8_t* smem, uint32_t lds0, const Src<C>& src, int nk,
                                            f32x4_t (&acc)[C::TM][C::TN]) {
  static_assert(C::MX, "MXFP8 tiles");
  static_assert(C::A_WAVES == C::NW, "every wave loads A rows");
  constexpr int TM = C::TM, TN = C::TN, NS = C::NS;
  const FragBase<C> fb;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N_, wn = wave % C::WAVES_N_;
  const int l16 = lane & 15, lg = lane >> 4;
  const uint32_t as_b = (uint32_t)(C::SC_BASE + (wm * C::WM + l16) * 16 + lg);
  const uint32_t bs_b = (uint32_t)(C::SC_BASE + (C::BM + wn * C::WNB + l16) * 16 + lg);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int kt = 0; kt < nk; ++kt) {
    wait_step_mx<C>(kt, nk);
    __syncthreads();   // step kt landed for every wave; every wave is done with step kt-1
    if (kt + NS - 1 < nk) issue_step<C>(lds0, src, kt + NS - 1, nk);
    const uint8_t* st = smem + (kt % NS) * C::STAGE;
    const uint8_t* alo = st + fb.a_lo;
    const uint8_t* ahi = st + fb.a_hi;
    const uint8_t* blo = st + fb.b_lo;
    const uint8_t* bhi = st + fb.b_hi;
    const int sgo = ((kt / kScG) & 1) * C::SG_BYTES + (kt % kScG) * 4;
    const uint8_t* sa_p = smem + as_b + sgo;
    const uint8_t* sb_p = smem + bs_b + sgo;
    i32x8_t af[TM];
    int sa[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      af[i] = load_frag8(alo + i * 16 * kRB, ahi + i * 16 * kRB);
      sa[i] = sa_p[i * 16 * 16];
    }
    i32x8_t bcur = load_frag8(blo + b_frag_row<C>(0) * kRB, bhi + b_frag_row<C>(0) * kRB);
    int scur = sb_p[b_frag_row<C>(0) * 16];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      i32x8_t bnext = bcur;
      int snext = scur;
      if (j + 1 < TN) {
        bnext = load_frag8(blo + b_frag_row<C>(j + 1) * kRB, bhi + b_frag_row<C>(j + 1) * kRB);
        snext = sb_p[b_frag_row<C>(j + 1) * 16];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bcur, af[i], acc[i][j], 0, 0, 0, scur, 0, sa[i]);
      bcur = bnext;
      scur = snext;
    }
  }
  __syncthreads();   // every wave is done reading the ring before it is refilled
}

// ---------------------------------------------------------------------------
// k-major (transposed-storage) operands, for the backward GEMMs: the operand
// is stored with its contraction index k as the row and the tile's own index
// x contiguous (a weight read as W^T, or activations contracted over rows).
// A k-major tile of X columns holds X/64 column blocks of 64 k-rows x 128
// bytes; DMA instruction g (0 .. X/8-1) writes column block g/8, k-rows
// (g%8)*8 .. +7 at LDS byte g*1024 (the same places as a row-major tile's
// instructions), and chunk c of k-row r sits at slot c ^ tswz(r).  Fragments
// are read with ds_read_b64_tr_b16, which, per 16-lane group, hands output
// lane i the element i%4 of the 8 bytes addressed by source lane 4j + i/4 as
// its j-th value (measured on gfx950).  Lane (l16 = s, lg) therefore points at
// k-row 8 lg + s/4 (+4 for the second read) and columns x0 + 4 (s%4): both
// reads give it row x0 + l16 of the fragment at k = 8 lg .. 8 lg + 7, the
// MFMA operand layout.  With tswz the 8 k-rows one 32-lane pass reads fall on
// 8 distinct bank ranges (checked by a bank model of every fragment).
// ---------------------------------------------------------------------------

typedef short v4i16_t __attribute__((ext_vector_type(4)));

__device__ __host__ __forceinline__ int tswz(int r) { return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2); }

// k-row within its 64-row step, and the 16-byte column chunk, that this lane
// loads in DMA instruction g of a k-major tile
__device__ __forceinline__ int trow_of(int g) { return ((g & 7) << 3) + ((threadIdx.x & 63) >> 3); }
__device__ __forceinline__ int tchunk_of(int g) {
  const int lane = threadIdx.x & 63;
  return (lane & 7) ^ tswz(((g & 7) << 3) + (lane >> 3));
}

// Per-lane parts of a k-major fragment address.
struct TBase {
  uint32_t tb, G;
  __device__ __forceinline__ TBase() {
    const int lane = threadIdx.x & 63;
    const int s = lane & 15, lg = lane >> 4;
    tb = (uint32_t)((8 * lg + (s >> 2)) * kRB + (s & 1) * 8);
    G = (uint32_t)(((((s >> 3) & 1) << 1) | ((lg & 1) << 2) | ((s >> 1) & 1)) << 4);
  }
};

// Fragment of a k-major tile at tile byte offset `tile`: rows x0 .. x0+15 (x0
// a multiple of 16), contraction substep ks (32 k each).
__device__ __forceinline__ bf16x8_t tfrag(const uint8_t* smem, uint32_t tile, const TBase& t, int x0, int ks) {
  const uint32_t off = tile + (uint32_t)((x0 >> 6) * 8192 + ks * 4096) + t.tb + ((uint32_t)(((x0 & 63) >> 3) << 4) ^ t.G);
  typedef __attribute__((address_space(3))) v4i16_t* lp;
  const __attribute__((address_space(3))) uint8_t* l = (const __attribute__((address_space(3))) uint8_t*)smem;
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(l + off));
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(l + off + 512));
  const v4i16_t both[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8_t, both);
}

// DMA sources of a backward tile.  K may be the concatenation of two
// products (bases [0] for steps < nk1, [1] after; same offsets).  Row-major
// operands: offsets at step 0, advanced kRB bytes a step through the base.
// k-major operands: the column byte offset of the lane's chunk; its k-row
// (step * 64 + trow) is clamped to `lim` (rows past it reload it) and scaled
// by the row stride `rs` when issued.
template <class C>
struct SrcB {
  const uint8_t* a[2];
  const uint8_t* b[2];
  int nk1;
  uint32_t a_off[C::A_INS];
  uint32_t b_off[C::B_INS];
  int a_rs, b_rs, a_lim, b_lim;
};

template <class C>
__device__ __forceinline__ void issue_step_b_at(uint32_t lds0, const SrcB<C>& src, int kt, int stage) {
  static_assert(C::A_WAVES == C::NW, "every wave loads A rows");
  const int wave = threadIdx.x >> 6;
  const uint32_t st = lds0 + (uint32_t)(stage * C::STAGE);
  const uint32_t wave_a = st + (uint32_t)(wave * C::A_INS) * 1024u;
  const uint32_t wave_b = st + (uint32_t)C::A_BYTES + (uint32_t)(wave * C::B_INS) * 1024u;
  const bool second = kt >= src.nk1;
  const int kk = second ? kt - src.nk1 : kt;
  const uint8_t* a = second ? src.a[1] : src.a[0];
  const uint8_t* b = second ? src.b[1] : src.b[0];
  // k-major operands: the step's first row in the 64-bit base, so a lane's
  // 32-bit offset spans only the step's 64 rows (an expert's rows may span
  // more than 4 GiB of k-major bytes)
  const uint8_t* ak = C::AT ? uniform_ptr(a + (int64_t)kk * 64 * src.a_rs) : a;
  const uint8_t* bk = C::BT ? uniform_ptr(b + (int64_t)kk * 64 * src.b_rs) : b;
#pragma unroll
  for (int q = 0; q < C::A_INS; ++q) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(wave_a + q * 1024u);
    if constexpr (C::AT) {
      const int row = min(trow_of(wave * C::A_INS + q), src.a_lim - kk * 64);
      lds_dma16(ak, (uint32_t)row * (uint32_t)src.a_rs + src.a_off[q], dst);
    } else {
      lds_dma16(a + (int64_t)kk * kRB, src.a_off[q], dst);
    }
  }
#pragma unroll
  for (int q = 0; q < C::B_INS; ++q) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(wave_b + q * 1024u);
    if constexpr (C::BT) {
      const int row = min(trow_of(wave * C::B_INS + q), src.b_lim - kk * 64);
      lds_dma16(bk, (uint32_t)row * (uint32_t)src.b_rs + src.b_off[q], dst);
    } else {
      lds_dma16(b + (int64_t)kk * kRB, src.b_off[q], dst);
    }
  }
}

template <class C>
__device__ __forceinline__ void issue_step_b(uint32_t lds0, const SrcB<C>& src, int kt) {
  issue_step_b_at<C>(lds0, src, kt, kt % C::NS);
}

template <class C>
__device__ __forceinline__ void prologue_b(uint32_t lds0, const SrcB<C>& src, int nk) {
#pragma unroll
  for (int s = 0; s < C::NS - 1; ++s)
    if (s < nk) issue_step_b<C>(lds0, src, s);
}

// Zero the B tile's k-rows past b_tail (< 64) of the step in ring stage
// `stage` after it landed, so clamped reloads of the last valid row add nothing.
template <class C>
__device__ __forceinline__ void zero_b_tail(const uint8_t* smem, int stage, int b_tail) {
  uint8_t* bt = const_cast<uint8_t*>(smem) + stage * C::STAGE + C::A_BYTES;
  const int n16 = (64 - b_tail) * 8;   // 16-byte pieces per column block
  for (int idx = threadIdx.x; idx < n16 * (C::BN / 64); idx += C::NW * 64) {
    const int cb = idx / n16, w = idx - cb * n16;
    *reinterpret_cast<uint4*>(bt + cb * 8192 + (b_tail + (w >> 3)) * kRB + (w & 7) * 16) = make_uint4(0, 0, 0, 0);
  }
}

// MFMAs of one landed step in ring stage `stage`.
template <class C>
__device__ __forceinline__ void compute_step_b(const uint8_t* smem, int stage, const FragBase<C>& fb, const TBase& tbase,
                                               int wm, int wn, f32x4_t (&acc)[C::TM][C::TN]) {
  constexpr int TM = C::TM, TN = C::TN;
  const uint32_t so = (uint32_t)(stage * C::STAGE);
  const uint8_t* st = smem + so;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    bf16x8_t af[TM], bfr[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if constexpr (C::AT) af[i] = tfrag(smem, so, tbase, wm * C::WM + i * 16, ks);
      else af[i] = *reinterpret_cast<const bf16x8_t*>(st + (ks ? fb.a_hi : fb.a_lo) + i * 16 * kRB);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if constexpr (C::BT) bfr[j] = tfrag(smem, so + C::A_BYTES, tbase, wn * C::WNB + b_frag_row<C>(j), ks);
      else bfr[j] = *reinterpret_cast<const bf16x8_t*>(st + (ks ? fb.b_hi : fb.b_lo) + b_frag_row<C>(j) * kRB);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
  }
}

template <class C>
__device__ __forceinline__ void zero_acc(f32x4_t (&acc)[C::TM][C::TN]) {
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// Backward main loop over nk steps.  b_tail < 64: only the first b_tail
// k-rows of the last step are valid, and the B tile's other k-rows are zeroed
// after they land, so clamped reloads of the last valid row add nothing.
template <class C>
__device__ __forceinline__ void mainloop_b(const uint8_t* smem, uint32_t lds0, const SrcB<C>& src, int nk, int b_tail,
                                           f32x4_t (&acc)[C::TM][C::TN]) {
  constexpr int NS = C::NS;
  const FragBase<C> fb;
  const TBase tbase;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N_, wn = wave % C::WAVES_N_;
  zero_acc<C>(acc);
  for (int kt = 0; kt < nk; ++kt) {
    wait_steps<C::LPS, NS - 2>(min(NS - 2, nk - 1 - kt));
    __syncthreads();   // step kt landed for every wave; every wave is done with step kt-1
    if constexpr (C::BT) {
      if (kt == nk - 1 && b_tail < 64) {
        zero_b_tail<C>(smem, kt % NS, b_tail);
        __syncthreads();
      }
    }
    if (kt + NS - 1 < nk) issue_step_b<C>(lds0, src, kt + NS - 1);
    compute_step_b<C>(smem, kt % NS, fb, tbase, wm, wn, acc);
  }
  __syncthreads();   // every wave is done reading the ring before it is refilled
}

// The same loop for a sequence of tiles fed through the two-stage ring as one
// stream of steps: step 0 of this tile sits at ring position g0, and during
// this tile's last step the first step of the next tile (nsrc, when has_next)
// is issued, so its loads overlap this tile's last MFMAs and its epilogue
// instead of following them.  The caller issues the first tile's step 0.
template <class C>
__device__ __forceinline__ void mainloop_b_stream(const uint8_t* smem, uint32_t lds0, const SrcB<C>& src, int nk,
                                                  int b_tail, const SrcB<C>& nsrc, bool has_next, int g0,
                                                  f32x4_t (&acc)[C::TM][C::TN]) {
  static_assert(C::NS == 2, "one step in flight past the current one");
  const FragBase<C> fb;
  const TBase tbase;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N_, wn = wave % C::WAVES_N_;
  zero_acc<C>(acc);
  for (int kt = 0; kt < nk; ++kt) {
    const int stage = (g0 + kt) & 1;
    wait_vmcnt<0>();
    __syncthreads();   // step kt landed for every wave; every wave is done with the step before it
    if constexpr (C::BT) {
      if (kt == nk - 1 && b_tail < 64) {
        zero_b_tail<C>(smem, stage, b_tail);
        __syncthreads();
      }
    }
    if (kt + 1 < nk) issue_step_b_at<C>(lds0, src, kt + 1, stage ^ 1);
    else if (has_next) issue_step_b_at<C>(lds0, nsrc, 0, stage ^ 1);
    compute_step_b<C>(smem, stage, fb, tbase, wm, wn, acc);
  }
}

}  // namespace tile
}  // namespace moe
