// MXFP8 conversions of the backward pass (gfx950).
//
// A matrix used in both orientations is quantized twice, each copy along its
// own contraction dimension and each from the bf16 source, never one copy
// from the other (KOSMOS section 2.2).  The forward's weights are quantized
// row-wise (along D for gate/up, along H for down); the data gradients need
// the transposed copies quantized along the other dimension (OLMo-core
// Appendix A, A.13: the right-hand operand prequantized for dgrad), which
// quantize_cols_kernel produces.  The weight gradients take bf16 operands:
// the saved MXFP8 activations are dequantized (A.13's wgrad policy), which
// dequant_rows_kernel does exactly (an E4M3 value times a power of two has at
// most four significant bits, so it is a bf16 value).
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

// Column-wise quantization with transpose:
//   src bf16 [B][R][C]  ->  q[b][c][col0 + r] (row stride ld bytes),
//   blocks of 32 consecutive r of one column c, scale [b][c][(col0 + r) / 32]
//   (row stride ld / 32).
// A 256-thread block moves a 128 (r) x 64 (c) tile through LDS: the loads are
// 16-byte row pieces of src; thread (blk, c) then quantizes column c's 32
// elements r0 + 32 blk .. + 31 and stores 32 code bytes and one scale.
constexpr int kQR = 128, kQC = 64, kQPad = 8;

__global__ __launch_bounds__(256) void quantize_cols_kernel(const uint16_t* __restrict__ src, int64_t R,
                                                            int64_t C, int64_t ld, int64_t col0,
                                                            uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kQR][kQC + kQPad];
  const int64_t b = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.y * kQR, c0 = (int64_t)blockIdx.x * kQC;
  const uint16_t* s = src + b * R * C;
  const int t = threadIdx.x;
  // load: thread t takes piece t % 8 (8 columns) of rows t / 8 + 32 i
#pragma unroll
  for (int i = 0; i < kQR / 32; ++i) {
    const int rr = t / 8 + 32 * i, cc = (t % 8) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r0 + rr < R && c0 + cc < C) v = ldg16(s + (r0 + rr) * C + c0 + cc);
    *reinterpret_cast<uint4*>(&tile[rr][cc]) = v;
  }
  __syncthreads();
  const int c = t % kQC, blk = t / kQC;
  const int64_t r = r0 + 32 * blk;
  if (c0 + c >= C || r >= R) return;
  float f[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    f[i] = bf16_to_f32(tile[32 * blk + i][c]);
    amax = fmaxf(amax, fabsf(f[i]));
  }
  const int code = e8m0_code(amax);
  const int e = code - 127;
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = e4m3x4(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3], e);
  const int64_t qrow = (b * C + c0 + c) * ld;
  uint8_t* dst = q + qrow + col0 + r;
  stg16(dst, make_uint4(w[0], w[1], w[2], w[3]));
  stg16(dst + 16, make_uint4(w[4], w[5], w[6], w[7]));
  sc[(b * C + c0 + c) * (ld / 32) + (col0 + r) / 32] = (uint8_t)code;
}

// Column-wise copies of a row-segmented matrix for the native MXFP8 weight
// gradient, one contiguous block per expert.  Expert e's rows
// [offsets[e], offsets[e+1]) (a multiple of 32) become a [C][len128]
// E4M3 block, len128 = the segment rounded up to 128 columns, quantized
// along its rows in blocks of 32, columns past the segment zero; the blocks
// follow each other: expert e's starts at byte C * toff[e] (toff = the
// exclusive scan of len128) and its scales ([C][len128 / 32]) at byte
// C * toff[e] / 32.  A weight-gradient tile then reads 128-column steps of one
// expert's rows as contiguous runs instead of short pieces of long rows.
//
// seg128_scan_kernel: toff[0..Ex] in one workgroup (Ex <= 1024).
__global__ __launch_bounds__(1024) void seg128_scan_kernel(const int32_t* __restrict__ offsets, int Ex,
                                                           int32_t* __restrict__ toff) {
  __shared__ int s_w[16];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int len = t < Ex ? offsets[t + 1] - offsets[t] : 0;
  const int own = (len + 127) / 128 * 128;
  int inc = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(inc, o, 64);
    if (lane >= o) inc += v;
  }
  if (lane == 63) s_w[wv] = inc;
  __syncthreads();
  if (t == 0) {
    int r = 0;
    for (int w = 0; w < 16; ++w) { const int v = s_w[w]; s_w[w] = r; r += v; }
  }
  __syncthreads();
  inc += s_w[wv];
  if (t < Ex) toff[t] = inc - own;
  if (t == Ex - 1) toff[Ex] = inc;
}

// Block y of the grid covers destination columns [128 y, 128 y + 128) of the
// concatenated blocks (one 128-column chunk of one expert): source rows
// offsets[e] + 128 y - toff[e] + (0..127), zero past the segment.  gather:
// source row r is token row_route[r] / K of x (zero without a route), and
// the shared expert's segment (shared0 .. shared0 + N, when given) holds x.
// Blocks past toff[Ex] exit.
__global__ __launch_bounds__(256) void quantize_cols_seg_kernel(const uint16_t* __restrict__ src, int64_t C,
                                                                const int32_t* __restrict__ offsets, int Ex,
                                                                const int32_t* __restrict__ toff,
                                                                const int32_t* __restrict__ row_route, int K,
                                                                const int32_t* __restrict__ shared0, int64_t N,
                                                                uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kQR][kQC + kQPad];
  const int64_t p = (int64_t)blockIdx.y * kQR;   // destination column of the chunk
  if (p >= toff[Ex]) return;
  // the expert whose block holds column p (toff is non-decreasing)
  int lo = 0, hi = Ex - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (toff[mid] <= p) lo = mid;
    else hi = mid - 1;
  }
  const int e = lo;
  const int64_t local = p - toff[e];
  const int64_t seg0 = offsets[e], seg1 = offsets[e + 1];
  const int64_t len128 = toff[e + 1] - toff[e];
  const int64_t c0 = (int64_t)blockIdx.x * kQC;
  const int64_t s0 = shared0 ? (int64_t)*shared0 : -1;
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kQR / 32; ++i) {
    const int rr = t / 8 + 32 * i, cc = (t % 8) * 8;
    const int64_t r = seg0 + local + rr;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < seg1 && c0 + cc < C) {
      int64_t srow = r;
      if (row_route) {
        const int rt = row_route[r];
        srow = rt >= 0 ? rt / K : ((s0 >= 0 && r >= s0 && r < s0 + N) ? r - s0 : -1);
      }
      if (srow >= 0) v = ldg16(src + srow * C + c0 + cc);
    }
    *reinterpret_cast<uint4*>(&tile[rr][cc]) = v;
  }
  __syncthreads();
  const int c = t % kQC, blk = t / kQC;
  if (c0 + c >= C) return;
  float f[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    f[i] = bf16_to_f32(tile[32 * blk + i][c]);
    amax = fmaxf(amax, fabsf(f[i]));
  }
  const int code = e8m0_code(amax);
  const int ex = code - 127;
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = e4m3x4(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3], ex);
  const int64_t col = local + 32 * blk;   // within the expert's block
  uint8_t* dst = q + C * toff[e] + (c0 + c) * len128 + col;
  stg16(dst, make_uint4(w[0], w[1], w[2], w[3]));
  stg16(dst + 16, make_uint4(w[4], w[5], w[6], w[7]));
  sc[(C * toff[e] + (c0 + c) * len128 + col) / 32] = (uint8_t)code;
}

// E4M3FN code -> its value as fp32 (exact; codes 0x7F / 0xFF, NaN in E4M3FN,
// are never produced by the quantizer).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t ef = (c >> 3) & 0xFu, m = c & 7u;
  const float v = ef ? __uint_as_float(((ef + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return __uint_as_float(__float_as_uint(v) | ((c & 0x80u) << 24));
}

// bf16 [rows][cols] = E4M3 [rows][cols] x 2^(scale - 127); each lane converts
// 16 codes (half a block) per pass, one wave per row.  Rows at or past
// *rows_end (when given) are skipped.
__global__ __launch_bounds__(256) void dequant_rows_kernel(const uint8_t* __restrict__ q,
                                                           const uint8_t* __restrict__ sc, int64_t rows,
                                                           int cols, const int32_t* __restrict__ rows_end,
                                                           uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows || (rows_end && r >= *rows_end)) return;
  const int nvec = cols >> 4;
  for (int v = lane; v < nvec; v += kWave) {
    const uint4 c = ldg16(q + r * cols + v * 16);
    const float s = exp2i((int)sc[r * (cols >> 5) + (v >> 1)] - 127);
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = pack_bf16x2(e4m3_value(cw[i] & 0xFF) * s, e4m3_value((cw[i] >> 8) & 0xFF) * s);
      o[2 * i + 1] = pack_bf16x2(e4m3_value((cw[i] >> 16) & 0xFF) * s, e4m3_value(cw[i] >> 24) * s);
    }
    uint16_t* dst = out + r * cols + v * 16;
    stg16(dst, make_uint4(o[0], o[1], o[2], o[3]));
    stg16(dst + 8, make_uint4(o[4], o[5], o[6], o[7]));
  }
}

}  // namespace

hipError_t launch_quantize_cols(const void* src, int64_t batch, int64_t rows, int64_t cols, int64_t ld,
                                int64_t col0, uint8_t* q, uint8_t* sc, hipStream_t s) {
  if (batch == 0 || rows == 0 || cols == 0) return hipSuccess;
  const dim3 grid((unsigned)((cols + kQC - 1) / kQC), (unsigned)((rows + kQR - 1) / kQR), (unsigned)batch);
  quantize_cols_kernel<<<grid, 256, 0, s>>>((const uint16_t*)src, rows, cols, ld, col0, q, sc);
  return hipGetLastError();
}

hipError_t launch_seg128_scan(const int32_t* offsets, int64_t Ex, int32_t* toff, hipStream_t s) {
  seg128_scan_kernel<<<1, 1024, 0, s>>>(offsets, (int)Ex, toff);
  return hipGetLastError();
}

hipError_t launch_quantize_cols_seg(const void* src, int64_t cols, const int32_t* offsets, int64_t Ex,
                                    const int32_t* toff, int64_t max_cols, const int32_t* row_route, int64_t K,
                                    const int32_t* shared0, int64_t N, uint8_t* q, uint8_t* sc, hipStream_t s) {
  if (cols == 0 || max_cols == 0) return hipSuccess;
  const dim3 grid((unsigned)((cols + kQC - 1) / kQC), (unsigned)((max_cols + kQR - 1) / kQR), 1);
  quantize_cols_seg_kernel<<<grid, 256, 0, s>>>((const uint16_t*)src, cols, offsets, (int)Ex, toff, row_route,
                                                (int)K, shared0, N, q, sc);
  return hipGetLastError();
}

hipError_t launch_dequant_rows(const uint8_t* q, const uint8_t* sc, int64_t rows, int64_t cols,
                               const int32_t* rows_end, void* out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  dequant_rows_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(q, sc, rows, (int)cols, rows_end,
                                                                  (uint16_t*)out);
  return hipGetLastError();
}

}  // namespace moe
