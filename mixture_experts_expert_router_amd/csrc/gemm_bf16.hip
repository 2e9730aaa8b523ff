// Grouped GEMMs of the expert layer on bf16 MFMA (gfx950 v_mfma_f32_16x16x32_bf16),
// fp32 accumulation, LDS-staged double-buffered tiles (KOSMOS section 3.3.1
// steps 3-4: GEMM1 with SwiGLU fused in its epilogue storing the
// pre-activations, GEMM2; section 3.3.2: dgrad2 with the SwiGLU backward in its
// epilogue, wgrad2, dgrad1, wgrad1; OLMo-core Appendix A, A.8 eq. 92 for the
// work of each product).
//
// One kernel template covers every product of the layer:
//   ROWS kind (forward and dgrad): the M dimension is an expert's row segment
//     [offsets[e], offsets[e+1]); A is the activation rows (contraction
//     contiguous); B is the expert weight, contraction-contiguous (forward) or
//     output-contiguous (dgrad, loaded through an 8x8 register transpose).
//     DUAL: two weights share the A tile (gate and up) -> two accumulators.
//     KCAT: two (A, B) pairs summed into one accumulator (dgrad of gate/up).
//   WGRAD kind: per expert, output [n_dim][k_dim] and the contraction runs
//     over the expert's rows in ascending order; both operands are
//     row-contiguous in memory and go through the register transpose.
//
// MFMA operands are fed swapped (weight tile as the "A" operand) so that each
// lane's four accumulator values are four consecutive output columns of one
// row: epilogue stores are 8-byte vectors.
#include "common.h"
#include "launch.h"

namespace moe {

enum { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_SWIGLU_BWD = 2 };

struct GemmParams {
  const int32_t* offsets;   // [E+1]
  const int32_t* mtiles;    // ROWS kind: [0] = count; then (expert, first row) pairs
  int E;
  int N;                    // output columns
  int K;                    // contraction length (ROWS kind)
  int M_fixed;              // WGRAD kind: output rows (n_dim of the forward)
  int n_tiles;              // ceil(N / BN)
  int m_tiles_fixed;        // WGRAD kind: ceil(M_fixed / BM)
  // operand 0
  const uint16_t* a0; int64_t lda0;
  const uint16_t* b0; int64_t ldb0; int64_t sb0;   // sb = per-expert stride (elements)
  // operand 1 (DUAL: second weight; KCAT: second pair)
  const uint16_t* a1; int64_t lda1;
  const uint16_t* b1; int64_t ldb1; int64_t sb1;
  // outputs
  uint16_t* c0; uint16_t* c1; uint16_t* c2; int64_t ldc; int64_t sc;
  const uint16_t* g; const uint16_t* u;            // SWIGLU_BWD saved pre-activations
};

__device__ __forceinline__ uint4 zero4() { return make_uint4(0, 0, 0, 0); }

// 8x8 transpose of bf16: v[j] holds 8 consecutive "rows" r=0..7 of memory row j
// (contraction index j); out[i] = the 8 contraction values of row i.
__device__ __forceinline__ void transpose8x8(const uint4 (&v)[8], uint4 (&o)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t d[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4& A = v[2 * q];
      const uint4& B = v[2 * q + 1];
      uint32_t a = (i >> 1) == 0 ? A.x : (i >> 1) == 1 ? A.y : (i >> 1) == 2 ? A.z : A.w;
      uint32_t b = (i >> 1) == 0 ? B.x : (i >> 1) == 1 ? B.y : (i >> 1) == 2 ? B.z : B.w;
      d[q] = (i & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
    }
    o[i] = make_uint4(d[0], d[1], d[2], d[3]);
  }
}

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool A_KMAJ, bool B_KMAJ, bool DUAL,
          bool KCAT, int EPI, bool WGRAD>
__global__ __launch_bounds__(WAVES_M* WAVES_N * 64) void gemm_bf16_kernel(GemmParams p) {
  constexpr int NT = WAVES_M * WAVES_N * 64;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int LDK = BK + 8;                       // padded LDS row (bf16 elements)
  constexpr int A_ELEMS = BM * LDK, B_ELEMS = BN * LDK;
  constexpr int STAGE = A_ELEMS + NB * B_ELEMS;
  static_assert(BK % 32 == 0 && WM % 16 == 0 && WN % 16 == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // ---------------- tile -> (expert, rows, cols, contraction range) --------------
  int e, m_start, m_valid, n0;
  int64_t k_begin, k_end;                // contraction range (rows for WGRAD)
  {
    const int t = blockIdx.x;
    if (!WGRAD) {
      const int total_m = p.mtiles[0];
      if (t >= total_m * p.n_tiles) return;
      constexpr int GM = 8;               // m-blocks per swizzle group
      const int group = t / (GM * p.n_tiles);
      const int first = group * GM;
      const int gsz = min(GM, total_m - first);
      const int w = t - group * GM * p.n_tiles;
      const int mb = first + w % gsz;
      n0 = (w / gsz) * BN;
      e = p.mtiles[2 + 2 * mb];
      m_start = p.mtiles[3 + 2 * mb];
      m_valid = min(BM, p.offsets[e + 1] - m_start);
      k_begin = 0;
      k_end = p.K;
    } else {
      const int per_e = p.m_tiles_fixed * p.n_tiles;
      e = t / per_e;
      if (e >= p.E) return;
      const int w = t - e * per_e;
      m_start = (w % p.m_tiles_fixed) * BM;
      n0 = (w / p.m_tiles_fixed) * BN;
      m_valid = min(BM, p.M_fixed - m_start);
      k_begin = p.offsets[e];
      k_end = p.offsets[e + 1];
    }
  }
  const int n_valid = min(BN, p.N - n0);

  // per-pair operand bases
  const uint16_t* A[2];
  const uint16_t* B[2];
  int64_t lda[2], ldb[2];
  A[0] = p.a0; lda[0] = p.lda0; B[0] = p.b0 + (int64_t)e * p.sb0; ldb[0] = p.ldb0;
  A[1] = p.a1; lda[1] = p.lda1; B[1] = (p.b1 ? p.b1 + (int64_t)e * p.sb1 : nullptr); ldb[1] = p.ldb1;

  const int64_t klen = k_end - k_begin;
  const int nk0 = (int)((klen + BK - 1) / BK);
  const int nk = KCAT ? 2 * nk0 : nk0;

  // ---------------- global -> register staging ----------------------------------
  // K-major tile: R rows x BK, 16-byte chunks (8 contraction values)
  // MN-major tile: (R/8) x (BK/8) blocks of 8x8, each thread loads 8 rows of
  // memory (8 contraction indices) x 8 contiguous tile rows, then transposes.
  constexpr int A_CH = BM * BK / 8;
  constexpr int B_CH = BN * BK / 8;
  constexpr int A_IT = A_KMAJ ? (A_CH + NT - 1) / NT : (A_CH / 8 + NT - 1) / NT;
  constexpr int B_IT = B_KMAJ ? (B_CH + NT - 1) / NT : (B_CH / 8 + NT - 1) / NT;
  constexpr int A_REG = A_KMAJ ? A_IT : A_IT * 8;
  constexpr int B_REG = B_KMAJ ? B_IT : B_IT * 8;
  uint4 ra[A_REG];
  uint4 rb[NB][B_REG];

  auto load_tiles = [&](int kt) {
    const int pair = (KCAT && kt >= nk0) ? 1 : 0;
    const int64_t k0 = k_begin + (int64_t)(kt - pair * nk0) * BK;
    // ---- A ----
    const uint16_t* Ab = A[pair];
    const int64_t la = lda[pair];
    if (A_KMAJ) {
#pragma unroll
      for (int i = 0; i < A_IT; ++i) {
        const int c = tid + i * NT;
        const int r = c / (BK / 8), kc = c % (BK / 8);
        const int64_t gk = k0 + kc * 8;
        ra[i] = (c < A_CH && r < m_valid && gk < k_end)
                    ? ldg16(Ab + (int64_t)(m_start + r) * la + gk) : zero4();
      }
    } else {
#pragma unroll
      for (int i = 0; i < A_IT; ++i) {
        const int b = tid + i * NT;
        const int rc = b % (BM / 8), kb = b / (BM / 8);
        const bool ok = b < A_CH / 8 && rc * 8 < m_valid;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int64_t gk = k0 + kb * 8 + j;
          ra[i * 8 + j] = (ok && gk < k_end) ? ldg16(Ab + gk * la + m_start + rc * 8) : zero4();
        }
      }
    }
    // ---- B ----
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint16_t* Bb = (DUAL && nb == 1) ? B[1] : B[pair];
      const int64_t lb = (DUAL && nb == 1) ? ldb[1] : ldb[pair];
      if (B_KMAJ) {
#pragma unroll
        for (int i = 0; i < B_IT; ++i) {
          const int c = tid + i * NT;
          const int r = c / (BK / 8), kc = c % (BK / 8);
          const int64_t gk = k0 + kc * 8;
          rb[nb][i] = (c < B_CH && r < n_valid && gk < k_end)
                          ? ldg16(Bb + (int64_t)(n0 + r) * lb + gk) : zero4();
        }
      } else {
#pragma unroll
        for (int i = 0; i < B_IT; ++i) {
          const int b = tid + i * NT;
          const int rc = b % (BN / 8), kb = b / (BN / 8);
          const bool ok = b < B_CH / 8 && rc * 8 < n_valid;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int64_t gk = k0 + kb * 8 + j;
            rb[nb][i * 8 + j] = (ok && gk < k_end) ? ldg16(Bb + gk * lb + n0 + rc * 8) : zero4();
          }
        }
      }
    }
  };

  auto store_tiles = [&](int buf) {
    uint16_t* As = smem + buf * STAGE;
    if (A_KMAJ) {
#pragma unroll
      for (int i = 0; i < A_IT; ++i) {
        const int c = tid + i * NT;
        if (c < A_CH) {
          const int r = c / (BK / 8), kc = c % (BK / 8);
          *reinterpret_cast<uint4*>(As + r * LDK + kc * 8) = ra[i];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < A_IT; ++i) {
        const int b = tid + i * NT;
        if (b < A_CH / 8) {
          const int rc = b % (BM / 8), kb = b / (BM / 8);
          uint4 v[8], o[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = ra[i * 8 + j];
          transpose8x8(v, o);
#pragma unroll
          for (int r = 0; r < 8; ++r) *reinterpret_cast<uint4*>(As + (rc * 8 + r) * LDK + kb * 8) = o[r];
        }
      }
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      uint16_t* Bs = As + A_ELEMS + nb * B_ELEMS;
      if (B_KMAJ) {
#pragma unroll
        for (int i = 0; i < B_IT; ++i) {
          const int c = tid + i * NT;
          if (c < B_CH) {
            const int r = c / (BK / 8), kc = c % (BK / 8);
            *reinterpret_cast<uint4*>(Bs + r * LDK + kc * 8) = rb[nb][i];
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < B_IT; ++i) {
          const int b = tid + i * NT;
          if (b < B_CH / 8) {
            const int rc = b % (BN / 8), kb = b / (BN / 8);
            uint4 v[8], o[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = rb[nb][i * 8 + j];
            transpose8x8(v, o);
#pragma unroll
            for (int r = 0; r < 8; ++r) *reinterpret_cast<uint4*>(Bs + (rc * 8 + r) * LDK + kb * 8) = o[r];
          }
        }
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

  const int l16 = lane & 15, lg = lane >> 4;
  if (nk > 0) {
    load_tiles(0);
    store_tiles(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) load_tiles(kt + 1);
      const uint16_t* As = smem + buf * STAGE;
#pragma unroll
      for (int ks = 0; ks < BK / 32; ++ks) {
        bf16x8_t af[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i)
          af[i] = *reinterpret_cast<const bf16x8_t*>(As + (wm * WM + i * 16 + l16) * LDK + ks * 32 + lg * 8);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint16_t* Bs = As + A_ELEMS + nb * B_ELEMS;
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const bf16x8_t bf =
                *reinterpret_cast<const bf16x8_t*>(Bs + (wn * WN + j * 16 + l16) * LDK + ks * 32 + lg * 8);
#pragma unroll
            for (int i = 0; i < TM; ++i)
              acc[nb][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf, af[i], acc[nb][i][j], 0, 0, 0);
          }
        }
      }
      if (kt + 1 < nk) store_tiles(buf ^ 1);
      __syncthreads();
    }
  }

  // ---------------- epilogue ---------------------------------------------------
  // lane holds rows m = wm*WM + i*16 + l16, cols n = wn*WN + j*16 + 4*lg + {0..3}
  const int64_t cbase = WGRAD ? (int64_t)e * p.sc : 0;
  const int64_t row0 = m_start;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = wm * WM + i * 16 + l16;
    if (m >= m_valid) continue;
    const int64_t row = row0 + m;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = wn * WN + j * 16 + 4 * lg;
      if (n >= n_valid) continue;
      const int64_t off = cbase + row * p.ldc + n0 + n;
      const f32x4_t a = acc[0][i][j];
      if (EPI == EPI_STORE) {
        *reinterpret_cast<uint2*>(p.c0 + off) = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
      } else if (EPI == EPI_SWIGLU) {
        const f32x4_t b = acc[NB - 1][i][j];
        uint32_t gw0 = pack_bf16x2(a[0], a[1]), gw1 = pack_bf16x2(a[2], a[3]);
        uint32_t uw0 = pack_bf16x2(b[0], b[1]), uw1 = pack_bf16x2(b[2], b[3]);
        *reinterpret_cast<uint2*>(p.c0 + off) = make_uint2(gw0, gw1);
        *reinterpret_cast<uint2*>(p.c1 + off) = make_uint2(uw0, uw1);
        float g0 = bf16lo(gw0), g1 = bf16hi(gw0), g2 = bf16lo(gw1), g3 = bf16hi(gw1);
        float h0 = g0 * sigmoidf_(g0) * bf16lo(uw0);
        float h1 = g1 * sigmoidf_(g1) * bf16hi(uw0);
        float h2 = g2 * sigmoidf_(g2) * bf16lo(uw1);
        float h3 = g3 * sigmoidf_(g3) * bf16hi(uw1);
        *reinterpret_cast<uint2*>(p.c2 + off) = make_uint2(pack_bf16x2(h0, h1), pack_bf16x2(h2, h3));
      } else {  // EPI_SWIGLU_BWD: a = dH; saved g, u at the same position
        const uint2 gw = *reinterpret_cast<const uint2*>(p.g + off);
        const uint2 uw = *reinterpret_cast<const uint2*>(p.u + off);
        float gg[4] = {bf16lo(gw.x), bf16hi(gw.x), bf16lo(gw.y), bf16hi(gw.y)};
        float uu[4] = {bf16lo(uw.x), bf16hi(uw.x), bf16lo(uw.y), bf16hi(uw.y)};
        float dg[4], du[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float s = sigmoidf_(gg[q]);
          dg[q] = a[q] * uu[q] * s * (1.0f + gg[q] * (1.0f - s));
          du[q] = a[q] * gg[q] * s;
        }
        *reinterpret_cast<uint2*>(p.c0 + off) = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
        *reinterpret_cast<uint2*>(p.c1 + off) = make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
      }
    }
  }
}

// ---- m-block table of the ROWS kind: one workgroup --------------------------------
__global__ __launch_bounds__(1024) void build_mtiles_kernel(const int32_t* __restrict__ offsets, int E,
                                                            int BM, int32_t* __restrict__ out) {
  __shared__ int s_wsum[16];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int nb = 0, start = 0;
  if ((int)threadIdx.x < E) {
    start = offsets[threadIdx.x];
    nb = (offsets[threadIdx.x + 1] - start + BM - 1) / BM;
  }
  int inc = nb;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int n = __shfl_up(inc, o, 64);
    if (lane >= o) inc += n;
  }
  if (lane == 63) s_wsum[wv] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < 16; ++w) { int t = s_wsum[w]; s_wsum[w] = run; run += t; }
    out[0] = run;
    out[1] = 0;
  }
  __syncthreads();
  const int first = inc - nb + s_wsum[wv];
  for (int i = 0; i < nb; ++i) {
    out[2 + 2 * (first + i)] = threadIdx.x;
    out[3 + 2 * (first + i)] = start + i * BM;
  }
}

// ---------------- host side ----------------------------------------------------------
hipError_t launch_build_mtiles(const int32_t* offsets, int64_t E, int BM, int32_t* table, hipStream_t s) {
  build_mtiles_kernel<<<1, 1024, 0, s>>>(offsets, (int)E, BM, table);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool A_KMAJ, bool B_KMAJ, bool DUAL,
          bool KCAT, int EPI, bool WGRAD>
static hipError_t run(const GemmParams& p, unsigned grid, hipStream_t s) {
  if (grid == 0) return hipSuccess;
  gemm_bf16_kernel<BM, BN, BK, WAVES_M, WAVES_N, A_KMAJ, B_KMAJ, DUAL, KCAT, EPI, WGRAD>
      <<<grid, WAVES_M * WAVES_N * 64, 0, s>>>(p);
  return hipGetLastError();
}

int64_t mtile_table_ints(int64_t rows_cap, int64_t E, int BM) { return 2 + 2 * (rows_cap / BM + E + 1); }

// Shape rule for the M tile: small per-expert batches (< 256 rows on average)
// take 64-row tiles, larger ones 128.
static int pick_bm(int64_t rows_cap, int64_t E) { return (rows_cap / (E > 0 ? E : 1)) < 256 ? 64 : 128; }

hipError_t launch_gemm_fwd_bf16(const GemmFwd& f, int32_t* table, hipStream_t s) {
  const int BM = pick_bm(f.rows_cap, f.E);
  build_mtiles_kernel<<<1, 1024, 0, s>>>(f.offsets, (int)f.E, BM, table);
  GemmParams p{};
  p.offsets = f.offsets;
  p.mtiles = table;
  p.E = (int)f.E;
  p.N = (int)f.n_dim;
  p.K = (int)f.k_dim;
  p.a0 = (const uint16_t*)f.a;
  p.lda0 = f.k_dim;
  p.b0 = (const uint16_t*)f.b0;
  p.ldb0 = f.k_dim;
  p.sb0 = f.n_dim * f.k_dim;
  p.b1 = (const uint16_t*)f.b1;
  p.ldb1 = f.k_dim;
  p.sb1 = f.n_dim * f.k_dim;
  p.c0 = (uint16_t*)f.c0;
  p.c1 = (uint16_t*)f.c1;
  p.c2 = (uint16_t*)f.act;
  p.ldc = f.n_dim;
  const int64_t max_mb = f.rows_cap / BM + f.E + 1;
  if (f.swiglu) {
    constexpr int BN = 128;
    p.n_tiles = (int)((f.n_dim + BN - 1) / BN);
    const unsigned grid = (unsigned)(max_mb * p.n_tiles);
    if (BM == 64) return run<64, BN, 64, 2, 2, true, true, true, false, EPI_SWIGLU, false>(p, grid, s);
    return run<128, BN, 64, 2, 2, true, true, true, false, EPI_SWIGLU, false>(p, grid, s);
  }
  constexpr int BN = 128;
  p.n_tiles = (int)((f.n_dim + BN - 1) / BN);
  const unsigned grid = (unsigned)(max_mb * p.n_tiles);
  if (BM == 64) return run<64, BN, 64, 2, 2, true, true, false, false, EPI_STORE, false>(p, grid, s);
  return run<128, BN, 64, 2, 2, true, true, false, false, EPI_STORE, false>(p, grid, s);
}

hipError_t launch_gemm_dgrad_bf16(const GemmBwd& b, int32_t* table, hipStream_t s) {
  // da[rows][k_dim] = dc0[rows][n_dim] . b0[e] (n_dim x k_dim, k_dim contiguous)
  const int BM = pick_bm(b.rows_cap, b.E);
  build_mtiles_kernel<<<1, 1024, 0, s>>>(b.offsets, (int)b.E, BM, table);
  GemmParams p{};
  p.offsets = b.offsets;
  p.mtiles = table;
  p.E = (int)b.E;
  p.N = (int)b.k_dim;
  p.K = (int)b.n_dim;
  p.a0 = (const uint16_t*)b.dc0;
  p.lda0 = b.n_dim;
  p.b0 = (const uint16_t*)b.b0;
  p.ldb0 = b.k_dim;
  p.sb0 = b.n_dim * b.k_dim;
  p.a1 = (const uint16_t*)b.dc1;
  p.lda1 = b.n_dim;
  p.b1 = (const uint16_t*)b.b1;
  p.ldb1 = b.k_dim;
  p.sb1 = b.n_dim * b.k_dim;
  p.ldc = b.k_dim;
  constexpr int BN = 128;
  p.n_tiles = (int)((b.k_dim + BN - 1) / BN);
  const int64_t max_mb = b.rows_cap / BM + b.E + 1;
  const unsigned grid = (unsigned)(max_mb * p.n_tiles);
  if (b.swiglu_bwd) {
    p.c0 = (uint16_t*)b.dg;
    p.c1 = (uint16_t*)b.du;
    p.g = (const uint16_t*)b.g;
    p.u = (const uint16_t*)b.u;
    if (BM == 64) return run<64, BN, 64, 2, 2, true, false, false, false, EPI_SWIGLU_BWD, false>(p, grid, s);
    return run<128, BN, 64, 2, 2, true, false, false, false, EPI_SWIGLU_BWD, false>(p, grid, s);
  }
  p.c0 = (uint16_t*)b.da;
  if (b.dc1) {
    if (BM == 64) return run<64, BN, 64, 2, 2, true, false, false, true, EPI_STORE, false>(p, grid, s);
    return run<128, BN, 64, 2, 2, true, false, false, true, EPI_STORE, false>(p, grid, s);
  }
  if (BM == 64) return run<64, BN, 64, 2, 2, true, false, false, false, EPI_STORE, false>(p, grid, s);
  return run<128, BN, 64, 2, 2, true, false, false, false, EPI_STORE, false>(p, grid, s);
}

hipError_t launch_gemm_wgrad_bf16(const GemmBwd& b, const void* dc, void* db, hipStream_t s) {
  // db[e][n][k] = sum_{i in e} dc[i][n] a[i][k]:  output rows n (M_fixed = n_dim),
  // cols k (N = k_dim); operand A' = dc (row-contiguous in n), B' = a (in k)
  GemmParams p{};
  p.offsets = b.offsets;
  p.E = (int)b.E;
  p.M_fixed = (int)b.n_dim;
  p.N = (int)b.k_dim;
  p.a0 = (const uint16_t*)dc;
  p.lda0 = b.n_dim;
  p.b0 = (const uint16_t*)b.a;
  p.ldb0 = b.k_dim;
  p.sb0 = 0;
  p.c0 = (uint16_t*)db;
  p.ldc = b.k_dim;
  p.sc = b.n_dim * b.k_dim;
  constexpr int BM = 128, BN = 128;
  p.m_tiles_fixed = (int)((b.n_dim + BM - 1) / BM);
  p.n_tiles = (int)((b.k_dim + BN - 1) / BN);
  const unsigned grid = (unsigned)(b.E * p.m_tiles_fixed * p.n_tiles);
  return run<BM, BN, 64, 2, 2, false, false, false, false, EPI_STORE, true>(p, grid, s);
}

}  // namespace moe
