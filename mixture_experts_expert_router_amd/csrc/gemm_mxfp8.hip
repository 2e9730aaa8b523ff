// Block-scaled MXFP8 grouped GEMM (forward) on gfx950's scaled MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4: E4M3 operands, one E8M0 scale per 32
// contraction elements of each row, fp32 accumulation, bf16 epilogue
// (OLMo-core Appendix A, A.5 eq. 87; KOSMOS section 2.2 and section 3.3.1
// step 3: GEMM1 with SwiGLU and the row-wise quantization of its output for
// GEMM2).
//
// Operand layout per MFMA (16 rows x 128 contraction), measured on gfx950:
// lane l supplies row l % 16; its bytes 0..15 are contraction indices
// 16*(l/16) .. +15 and its bytes 16..31 are 64 + 16*(l/16) .. +15, while the
// E8M0 byte it passes scales contraction block l/16 (indices 32*(l/16) ..
// +31) of its row, whichever lanes hold that block's data.
// Tiles are staged through LDS double-buffered like the bf16 kernel; the
// weight tile is fed as the first operand so each lane ends with four
// consecutive output columns of one row.
#include "common.h"
#include "launch.h"

namespace moe {

struct MxParams {
  const int32_t* offsets;
  const int32_t* mtiles;
  int E, N, K, n_tiles;
  const uint8_t* a; const uint8_t* as;          // [rows][K], [rows][K/32]
  const uint8_t* b0; const uint8_t* bs0;        // [E][N][K], [E][N][K/32]
  const uint8_t* b1; const uint8_t* bs1;
  uint16_t* c0; uint16_t* c1; uint16_t* c2;     // bf16 [rows][N]
  uint8_t* hq; uint8_t* hs;                     // optional MXFP8 copy of c2 along N
};

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool DUAL>
__global__ __launch_bounds__(WAVES_M* WAVES_N * 64) void gemm_mxfp8_kernel(MxParams p) {
  constexpr int NT = WAVES_M * WAVES_N * 64;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int LDB = BK + 16;                  // padded LDS row (bytes)
  constexpr int SB = BK / 32;                   // scale bytes per row per tile
  constexpr int A_BYTES = BM * LDB, B_BYTES = BN * LDB;
  constexpr int AS_BYTES = BM * SB, BS_BYTES = BN * SB;
  constexpr int STAGE = A_BYTES + NB * B_BYTES + AS_BYTES + NB * BS_BYTES;
  static_assert(BK % 128 == 0 && STAGE % 16 == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int l16 = lane & 15, lg = lane >> 4;

  const int total_m = p.mtiles[0];
  const int t = blockIdx.x;
  if (t >= total_m * p.n_tiles) return;
  constexpr int GM = 8;
  const int group = t / (GM * p.n_tiles);
  const int first = group * GM;
  const int gsz = min(GM, total_m - first);
  const int w = t - group * GM * p.n_tiles;
  const int mb = first + w % gsz;
  const int n0 = (w / gsz) * BN;
  const int e = p.mtiles[2 + 2 * mb];
  const int m_start = p.mtiles[3 + 2 * mb];
  const int m_valid = min(BM, p.offsets[e + 1] - m_start);
  const int n_valid = min(BN, p.N - n0);
  const int K = p.K, KS = K / 32;
  const uint8_t* Bq[2] = {p.b0 + (int64_t)e * p.N * K, DUAL ? p.b1 + (int64_t)e * p.N * K : nullptr};
  const uint8_t* Bsc[2] = {p.bs0 + (int64_t)e * p.N * KS, DUAL ? p.bs1 + (int64_t)e * p.N * KS : nullptr};
  const int nk = (K + BK - 1) / BK;

  constexpr int A_CH = BM * BK / 16, B_CH = BN * BK / 16;
  constexpr int A_IT = (A_CH + NT - 1) / NT, B_IT = (B_CH + NT - 1) / NT;
  constexpr int AS_IT = (BM * SB + NT - 1) / NT, BS_IT = (BN * SB + NT - 1) / NT;
  uint4 ra[A_IT];
  uint4 rb[NB][B_IT];
  uint8_t rsa[AS_IT];
  uint8_t rsb[NB][BS_IT];

  auto load_tiles = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < A_IT; ++i) {
      const int c = tid + i * NT;
      const int r = c / (BK / 16), kc = c % (BK / 16);
      const int gk = k0 + kc * 16;
      ra[i] = (c < A_CH && r < m_valid && gk < K) ? ldg16(p.a + (int64_t)(m_start + r) * K + gk)
                                                  : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < AS_IT; ++i) {
      const int c = tid + i * NT;
      const int r = c / SB, kb = c % SB;
      const int gkb = k0 / 32 + kb;
      rsa[i] = (c < BM * SB && r < m_valid && gkb < KS) ? p.as[(int64_t)(m_start + r) * KS + gkb] : 0;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int i = 0; i < B_IT; ++i) {
        const int c = tid + i * NT;
        const int r = c / (BK / 16), kc = c % (BK / 16);
        const int gk = k0 + kc * 16;
        rb[nb][i] = (c < B_CH && r < n_valid && gk < K) ? ldg16(Bq[nb] + (int64_t)(n0 + r) * K + gk)
                                                        : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < BS_IT; ++i) {
        const int c = tid + i * NT;
        const int r = c / SB, kb = c % SB;
        const int gkb = k0 / 32 + kb;
        rsb[nb][i] = (c < BN * SB && r < n_valid && gkb < KS) ? Bsc[nb][(int64_t)(n0 + r) * KS + gkb] : 0;
      }
    }
  };

  auto store_tiles = [&](int buf) {
    uint8_t* st = smem + buf * STAGE;
    uint8_t* As = st;
    uint8_t* Ass = st + A_BYTES + NB * B_BYTES;
#pragma unroll
    for (int i = 0; i < A_IT; ++i) {
      const int c = tid + i * NT;
      if (c < A_CH) *reinterpret_cast<uint4*>(As + (c / (BK / 16)) * LDB + (c % (BK / 16)) * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < AS_IT; ++i) {
      const int c = tid + i * NT;
      if (c < BM * SB) Ass[c] = rsa[i];
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      uint8_t* Bs = As + A_BYTES + nb * B_BYTES;
      uint8_t* Bss = Ass + AS_BYTES + nb * BS_BYTES;
#pragma unroll
      for (int i = 0; i < B_IT; ++i) {
        const int c = tid + i * NT;
        if (c < B_CH) *reinterpret_cast<uint4*>(Bs + (c / (BK / 16)) * LDB + (c % (BK / 16)) * 16) = rb[nb][i];
      }
#pragma unroll
      for (int i = 0; i < BS_IT; ++i) {
        const int c = tid + i * NT;
        if (c < BN * SB) Bss[c] = rsb[nb][i];
      }
    }
  };

  f32x4_t acc[NB][TM][TN];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[nb][i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (nk > 0) {
    load_tiles(0);
    store_tiles(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) load_tiles(kt + 1);
      const uint8_t* st = smem + buf * STAGE;
      const uint8_t* As = st;
      const uint8_t* Ass = st + A_BYTES + NB * B_BYTES;
#pragma unroll
      for (int ks = 0; ks < BK / 128; ++ks) {
        i32x8_t af[TM];
        int sa[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int r = wm * WM + i * 16 + l16;
          const uint4 lo = *reinterpret_cast<const uint4*>(As + r * LDB + ks * 128 + lg * 16);
          const uint4 hi = *reinterpret_cast<const uint4*>(As + r * LDB + ks * 128 + 64 + lg * 16);
          af[i] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          sa[i] = Ass[r * SB + ks * 4 + lg];
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint8_t* Bs = As + A_BYTES + nb * B_BYTES;
          const uint8_t* Bss = Ass + AS_BYTES + nb * BS_BYTES;
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int r = wn * WN + j * 16 + l16;
            const uint4 lo = *reinterpret_cast<const uint4*>(Bs + r * LDB + ks * 128 + lg * 16);
            const uint4 hi = *reinterpret_cast<const uint4*>(Bs + r * LDB + ks * 128 + 64 + lg * 16);
            const i32x8_t bf{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            const int sb = Bss[r * SB + ks * 4 + lg];
#pragma unroll
            for (int i = 0; i < TM; ++i)
              acc[nb][i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af[i], acc[nb][i][j], 0, 0,
                                                                               0, sb, 0, sa[i]);
          }
        }
      }
      if (kt + 1 < nk) store_tiles(buf ^ 1);
      __syncthreads();
    }
  }

  // epilogue: lane holds row m = wm*WM + i*16 + l16, cols n = wn*WN + j*16 + 4*lg + {0..3}
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = wm * WM + i * 16 + l16;
    const bool mok = m < m_valid;
    const int64_t row = m_start + m;
    uint32_t hw[TN][2];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = wn * WN + j * 16 + 4 * lg;
      const bool ok = mok && n < n_valid;
      const int64_t off = row * p.N + n0 + n;
      const f32x4_t a = acc[0][i][j];
      if (!DUAL) {
        if (ok) *reinterpret_cast<uint2*>(p.c0 + off) = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
        hw[j][0] = hw[j][1] = 0;
      } else {
        const f32x4_t b = acc[NB - 1][i][j];
        const uint32_t gw0 = pack_bf16x2(a[0], a[1]), gw1 = pack_bf16x2(a[2], a[3]);
        const uint32_t uw0 = pack_bf16x2(b[0], b[1]), uw1 = pack_bf16x2(b[2], b[3]);
        const float g0 = bf16lo(gw0), g1 = bf16hi(gw0), g2 = bf16lo(gw1), g3 = bf16hi(gw1);
        hw[j][0] = pack_bf16x2(g0 * sigmoidf_(g0) * bf16lo(uw0), g1 * sigmoidf_(g1) * bf16hi(uw0));
        hw[j][1] = pack_bf16x2(g2 * sigmoidf_(g2) * bf16lo(uw1), g3 * sigmoidf_(g3) * bf16hi(uw1));
        if (ok) {
          *reinterpret_cast<uint2*>(p.c0 + off) = make_uint2(gw0, gw1);
          *reinterpret_cast<uint2*>(p.c1 + off) = make_uint2(uw0, uw1);
          if (p.c2) *reinterpret_cast<uint2*>(p.c2 + off) = make_uint2(hw[j][0], hw[j][1]);
        }
      }
    }
    if (DUAL && p.hq) {
      // a 32-column block is tiles (j, j+1) over the 4 lane groups of one row
#pragma unroll
      for (int j = 0; j < TN; j += 2) {
        float v[8] = {bf16lo(hw[j][0]), bf16hi(hw[j][0]), bf16lo(hw[j][1]), bf16hi(hw[j][1]),
                      bf16lo(hw[j + 1][0]), bf16hi(hw[j + 1][0]), bf16lo(hw[j + 1][1]), bf16hi(hw[j + 1][1])};
        float amax = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        const int code = e8m0_code(amax);
        const uint32_t q0 = e4m3x4(v[0], v[1], v[2], v[3], code - 127);
        const uint32_t q1 = e4m3x4(v[4], v[5], v[6], v[7], code - 127);
        const int n = wn * WN + j * 16 + 4 * lg;
        if (mok && n < n_valid) {
          uint8_t* qrow = p.hq + row * p.N + n0;
          *reinterpret_cast<uint32_t*>(qrow + n) = q0;
          *reinterpret_cast<uint32_t*>(qrow + n + 16) = q1;
          if (lg == 0) p.hs[row * (p.N / 32) + (n0 + wn * WN + j * 16) / 32] = (uint8_t)code;
        }
      }
    }
  }
}

hipError_t launch_gemm_fwd_mxfp8(const GemmFwd& f, int32_t* table, hipStream_t s) {
  const int BM = (f.rows_cap / (f.E > 0 ? f.E : 1)) < 256 ? 64 : 128;
  hipError_t err = launch_build_mtiles(f.offsets, f.E, BM, table, s);
  if (err != hipSuccess) return err;
  MxParams p{};
  p.offsets = f.offsets;
  p.mtiles = table;
  p.E = (int)f.E;
  p.N = (int)f.n_dim;
  p.K = (int)f.k_dim;
  p.a = (const uint8_t*)f.a;
  p.as = f.a_scales;
  p.b0 = (const uint8_t*)f.b0;
  p.bs0 = f.b0_scales;
  p.b1 = (const uint8_t*)f.b1;
  p.bs1 = f.b1_scales;
  p.c0 = (uint16_t*)f.c0;
  p.c1 = (uint16_t*)f.c1;
  p.c2 = (uint16_t*)f.act;
  p.hq = f.act_q;
  p.hs = f.act_scales;
  constexpr int BN = 128;
  p.n_tiles = (int)((f.n_dim + BN - 1) / BN);
  const int64_t max_mb = f.rows_cap / BM + f.E + 1;
  const unsigned grid = (unsigned)(max_mb * p.n_tiles);
  if (grid == 0) return hipSuccess;
  if (f.swiglu) {
    if (BM == 64) gemm_mxfp8_kernel<64, BN, 128, 2, 2, true><<<grid, 256, 0, s>>>(p);
    else gemm_mxfp8_kernel<128, BN, 128, 2, 2, true><<<grid, 256, 0, s>>>(p);
  } else {
    if (BM == 64) gemm_mxfp8_kernel<64, BN, 128, 2, 2, false><<<grid, 256, 0, s>>>(p);
    else gemm_mxfp8_kernel<128, BN, 128, 2, 2, false><<<grid, 256, 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace moe
