// Router logits L = X W_r^T + b on bf16 MFMA with fp32 accumulation (KOSMOS
// section 3.3.1 step 1: router logits in FP32 tiles; its router tile is narrow
// because the product has only as many columns as experts).
//
// One workgroup (4 waves) owns 16 token rows and all E columns.  The E/16
// column tiles are split over the waves; when there are fewer than four
// column tiles the waves split the contraction instead and their partial sums
// are added in LDS in a fixed order.  Operands come straight from global
// memory in 16-byte fragments: each token row is read from HBM once, W_r is
// small and stays in L2.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kRouterMaxTiles = 16;   // column tiles per wave (E <= 1024)

__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
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

hipError_t launch_router_logits(const void* x, const void* w_r, const float* bias, int64_t N,
                                int64_t D, int64_t E, float* logits, hipStream_t s) {
  if (N == 0) return hipSuccess;
  router_logits_kernel<<<(unsigned)((N + 15) / 16), 256, 0, s>>>(
      (const uint16_t*)x, (const uint16_t*)w_r, bias, (int)N, (int)D, (int)E, logits);
  return hipGetLastError();
}

}  // namespace moe
