// Row permutes of the MoE layer over local HBM: dispatch into expert-
// contiguous rows, the weighted fold (combine), the combine backward with the
// route-weight gradient, and the MXFP8 row quantizer (OLMo-core Appendix A,
// A.1-A.4; KOSMOS section 3.3.1 steps 3 and 5, section 3.3.2 step 1).
//
// All of them move rows with 16-byte vectors, one wave per token row or per
// row segment (the combine, the MXFP8 dispatch), several vectors in flight
// per lane.  Dispatch reads each token row once and
// writes it K times (scatter form), so x crosses HBM once.  Combine gathers the
// K rows of a token and folds them in fp32 in ascending k with fmaf.
#include "common.h"
#include "launch.h"
#include "permute_dev.h"

namespace moe {

constexpr int kVPL = 8;   // 16-byte vectors per lane per pass

using perm::scale_bf16x8;

// Destination row of route k of token t (wave-uniform t and k, so a scalar
// load): routes 0..K-1 from dst_rows, route K the shared expert's row srow.
// Read where it is used rather than kept in a per-lane array, which the
// compiler would place in scratch memory.
__device__ __forceinline__ int route_row(const int32_t* __restrict__ dst_rows, int t, int K, int k,
                                         int srow) {
  return k < K ? dst_rows[(int64_t)t * K + k] : srow;
}

// dispatch (bf16): one wave per token; WEIGHTED multiplies by the route weight
template <bool WEIGHTED>
__global__ __launch_bounds__(256) void dispatch_bf16_kernel(const uint16_t* __restrict__ x,
                                                            const int32_t* __restrict__ dst_rows,
                                                            const float* __restrict__ weight,
                                                            int N, int D, int K,
                                                            uint16_t* __restrict__ xd,
                                                            const int32_t* __restrict__ shared_row0) {
  const int lane = threadIdx.x & 63;
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (t >= N) return;
  // route K (when there is a shared expert): its row of this token, weight 1
  const int KK = K + (shared_row0 ? 1 : 0);
  const int srow = shared_row0 ? *shared_row0 + t : -1;
  const int nvec = D >> 3;
  const uint16_t* src = x + (int64_t)t * D;
  // the token's destination rows (and weights), lane k holding route k's:
  // one vector load, read back with readlane in the store loop
  const int dkl = lane < K ? dst_rows[(int64_t)t * K + lane] : -1;
  const float wkl = (WEIGHTED && lane < K) ? weight[(int64_t)t * K + lane] : 1.0f;
  for (int v0 = 0; v0 < nvec; v0 += kWave * kVPL) {
    uint4 r[kVPL];
#pragma unroll
    for (int j = 0; j < kVPL; ++j) {
      const int v = v0 + lane + j * kWave;
      if (v < nvec) r[j] = ldg16(src + v * 8);
    }
    for (int k = 0; k < KK; ++k) {
      const int dk = k < K ? __builtin_amdgcn_readlane(dkl, k) : srow;
      if (dk < 0) continue;
      const float wk = (WEIGHTED && k < K) ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                                  __builtin_bit_cast(int, wkl), k))
                                           : 1.0f;
      uint16_t* out = xd + (int64_t)dk * D;
#pragma unroll
      for (int j = 0; j < kVPL; ++j) {
        const int v = v0 + lane + j * kWave;
        if (v < nvec) stg16(out + v * 8, (WEIGHTED && k < K) ? scale_bf16x8(r[j], wk) : r[j]);
      }
    }
  }
}

// MXFP8 quantization of one 16-byte vector (8 bf16 values); lanes 4j..4j+3 of
// a wave hold one 32-element block.  Returns the 8 E4M3 bytes and the scale.
__device__ __forceinline__ uint2 quant_vec(uint4 v, int& code_out) {
  float f[8] = {bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y),
                bf16lo(v.z), bf16hi(v.z), bf16lo(v.w), bf16hi(v.w)};
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const int code = e8m0_code(amax);
  const int e = code - 127;
  code_out = code;
  return make_uint2(e4m3x4(f[0], f[1], f[2], f[3], e), e4m3x4(f[4], f[5], f[6], f[7], e));
}

// dispatch (MXFP8): quantize each token row once along D, write q and scales
// to its K rows.  D is a multiple of 32, so 4 consecutive lanes own a block
// and every wave-wide pass covers whole blocks.
__global__ __launch_bounds__(256) void dispatch_mxfp8_kernel(const uint16_t* __restrict__ x,
                                                             const int32_t* __restrict__ dst_rows,
                                                             int N, int D, int K,
                                                             uint8_t* __restrict__ q,
                                                             uint8_t* __restrict__ sc,
                                                             const int32_t* __restrict__ shared_row0,
    const int32_t* __restrict__ pad_counts, const int32_t* __restrict__ pad_offsets) {
  // trailing workgroups: one per expert, zeroing its padding rows
  const int tok_blocks = (N + 3) / 4;
  if (pad_counts && (int)blockIdx.x >= tok_blocks) {
    perm::zero_pad_rows_mx((int)blockIdx.x - tok_blocks, pad_counts, pad_offsets, D, q, sc, 4);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (t >= N) return;
  const int KK = K + (shared_row0 ? 1 : 0);
  const int srow = shared_row0 ? *shared_row0 + t : -1;   // the shared expert's row of this token
  const int nvec = D >> 3;
  const uint16_t* src = x + (int64_t)t * D;
  for (int v0 = 0; v0 < nvec; v0 += kWave * kVPL) {
    uint2 qv[kVPL];
    int code[kVPL];
#pragma unroll
    for (int j = 0; j < kVPL; ++j) {
      const int v = v0 + lane + j * kWave;
      uint4 r = make_uint4(0, 0, 0, 0);
      if (v < nvec) r = ldg16(src + v * 8);
      qv[j] = quant_vec(r, code[j]);     // all lanes take part in the shuffles
    }
    for (int k = 0; k < KK; ++k) {
      const int dk = route_row(dst_rows, t, K, k, srow);
      if (dk < 0) continue;
#pragma unroll
      for (int j = 0; j < kVPL; ++j) {
        const int v = v0 + lane + j * kWave;
        if (v < nvec) {
          *reinterpret_cast<uint2*>(q + (int64_t)dk * D + v * 8) = qv[j];
          if ((v & 3) == 0) sc[(int64_t)dk * (D >> 5) + (v >> 2)] = (uint8_t)code[j];
        }
      }
    }
  }
}

// Same result for D % 128 == 0, a wave per row segment of a token
// (perm::dispatch_mx_token: a lane quantizes 16 adjacent elements, a 32-block
// is a lane pair).
using perm::quant4;

__global__ __launch_bounds__(256) void dispatch_mxfp8_packed_kernel(const uint16_t* __restrict__ x,
                                                                    const int32_t* __restrict__ dst_rows,
                                                                    int N, int D, int K,
                                                                    uint8_t* __restrict__ q,
                                                                    uint8_t* __restrict__ sc,
                                                             const int32_t* __restrict__ shared_row0,
    const int32_t* __restrict__ pad_counts, const int32_t* __restrict__ pad_offsets) {
  // trailing workgroups: one per expert, zeroing its padding rows
  const int nseg = perm::mx_dispatch_segs(D);
  const int tok_blocks = (int)(((int64_t)N * nseg + 3) / 4);
  if (pad_counts && (int)blockIdx.x >= tok_blocks) {
    perm::zero_pad_rows_mx((int)blockIdx.x - tok_blocks, pad_counts, pad_offsets, D, q, sc, 4);
    return;
  }
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int t = w / nseg;
  if (t >= N) return;
  const int srow = shared_row0 ? *shared_row0 + t : -1;   // the shared expert's row of this token
  perm::dispatch_mx_token(t, w - t * nseg, x, dst_rows, D, K, srow, q, sc);
}

// zero n16 16-byte vectors from p, then the bytes up to `bytes`
__global__ __launch_bounds__(256) void zero_bytes_kernel(uint8_t* __restrict__ p, int64_t n16, int64_t bytes) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint4* q = reinterpret_cast<uint4*>(p);
  for (int64_t j = i; j < n16; j += stride) q[j] = make_uint4(0, 0, 0, 0);
  for (int64_t j = n16 * 16 + i; j < bytes; j += stride) p[j] = 0;
}

// zero the padding rows [offsets[e] + counts[e], offsets[e+1]) of each expert:
// one workgroup of 16 waves per expert, padding row i on wave i % 16, 16-byte
// stores for the data rows (row_bytes is a multiple of 16) and bytes for the
// scale rows
constexpr int kPadThreads = 1024;
__global__ __launch_bounds__(kPadThreads) void zero_padding_kernel(const int32_t* __restrict__ counts,
                                                                   const int32_t* __restrict__ offsets,
                                                                   int64_t row_bytes, uint8_t* __restrict__ a,
                                                                   int64_t row_bytes2,
                                                                   uint8_t* __restrict__ b,
                                                                   int64_t row_bytes3,
                                                                   uint8_t* __restrict__ c) {
  const int e = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r0 = offsets[e] + counts[e];
  const int64_t r1 = offsets[e + 1];
  for (int64_t r = r0 + wave; r < r1; r += kPadThreads / 64) {
    uint4* pa = reinterpret_cast<uint4*>(a + r * row_bytes);
    for (int64_t i = lane; i < row_bytes / 16; i += 64) pa[i] = make_uint4(0, 0, 0, 0);
    if (b && (row_bytes2 & 15) == 0) {
      uint4* pb = reinterpret_cast<uint4*>(b + r * row_bytes2);
      for (int64_t i = lane; i < row_bytes2 / 16; i += 64) pb[i] = make_uint4(0, 0, 0, 0);
    } else if (b) {
      uint8_t* pb = b + r * row_bytes2;
      for (int64_t i = lane; i < row_bytes2; i += 64) pb[i] = 0;
    }
    if (c) {
      uint8_t* pc = c + r * row_bytes3;
      for (int64_t i = lane; i < row_bytes3; i += 64) pc[i] = 0;
    }
  }
}

// combine: out[t] = bf16(sum_k w[t,k] * y[dst[t,k]]), a wave per segment of
// a token row (nseg segments a row)
template <bool WEIGHTED>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ dst_rows,
                                                      const float* __restrict__ weight, int N,
                                                      int D, int K, uint16_t* __restrict__ out,
                                                      const uint16_t* __restrict__ addend,
                                                      const int32_t* __restrict__ shared_row0, int nseg) {
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int t = w / nseg;
  if (t >= N) return;
  perm::combine_seg<WEIGHTED>(t, w - t * nseg, nseg, y, dst_rows, weight, D, K, out, addend, shared_row0);
}

// combine backward, a wave per token (QUANT: dY_d also quantized row-wise)
template <bool QUANT>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const uint16_t* __restrict__ dout,
                                                          const int32_t* __restrict__ dst_rows,
                                                          const float* __restrict__ weight,
                                                          const uint16_t* __restrict__ y, int N,
                                                          int D, int K, uint16_t* __restrict__ dyd,
                                                          float* __restrict__ dprob,
                                                          const int32_t* __restrict__ shared_row0,
                                                          uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (t >= N) return;
  perm::combine_bwd_token<QUANT>(t, dout, dst_rows, weight, y, D, K, dyd, dprob, shared_row0, q, sc);
}

// row-wise MXFP8 quantization of bf16 [rows][cols]; one wave per row.  Rows
// at or past *rows_end (when given) are skipped.
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint16_t* __restrict__ src,
                                                            int64_t rows, int cols,
                                                            uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ sc,
                                                            const int32_t* __restrict__ rows_end) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows || (rows_end && r >= *rows_end)) return;
  const int nvec = cols >> 3;
  const uint16_t* s = src + r * cols;
  for (int v0 = 0; v0 < nvec; v0 += kWave) {
    const int v = v0 + lane;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (v < nvec) x = ldg16(s + v * 8);
    int code;
    uint2 qq = quant_vec(x, code);
    if (v < nvec) {
      *reinterpret_cast<uint2*>(q + r * cols + v * 8) = qq;
      if ((v & 3) == 0) sc[r * (cols >> 5) + (v >> 2)] = (uint8_t)code;
    }
  }
}

// Same result for cols % 128 == 0 (and 4-byte aligned scale rows): each lane
// quantizes 16 adjacent elements, so a 32-block is a lane pair, with four
// such pieces per lane in flight; 16-byte code stores, and lanes 8i store the
// codes of four consecutive blocks as one 4-byte word.
__global__ __launch_bounds__(256) void quantize_rows_packed_kernel(const uint16_t* __restrict__ src,
                                                                   int64_t rows, int cols,
                                                                   uint8_t* __restrict__ q,
                                                                   uint8_t* __restrict__ sc,
                                                                   const int32_t* __restrict__ rows_end) {
  constexpr int PP = 4;   // 16-element pieces per lane per pass
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows || (rows_end && r >= *rows_end)) return;
  const int npair = cols >> 4, nblk = cols >> 5;
  const uint16_t* s = src + r * cols;
  uint8_t* qrow = q + r * cols;
  uint8_t* crow = sc + r * nblk;
  for (int p0 = 0; p0 < npair; p0 += kWave * PP) {
    uint4 x0[PP], x1[PP];
#pragma unroll
    for (int j = 0; j < PP; ++j) {
      const int pc = p0 + lane + j * kWave;
      x0[j] = make_uint4(0, 0, 0, 0);
      x1[j] = make_uint4(0, 0, 0, 0);
      if (pc < npair) {
        x0[j] = ldg16(s + pc * 16);
        x1[j] = ldg16(s + pc * 16 + 8);
      }
    }
#pragma unroll
    for (int j = 0; j < PP; ++j) {
      const int pc = p0 + lane + j * kWave;
      const uint4 r0 = x0[j], r1 = x1[j];
      float f[16] = {bf16lo(r0.x), bf16hi(r0.x), bf16lo(r0.y), bf16hi(r0.y), bf16lo(r0.z), bf16hi(r0.z),
                     bf16lo(r0.w), bf16hi(r0.w), bf16lo(r1.x), bf16hi(r1.x), bf16lo(r1.y), bf16hi(r1.y),
                     bf16lo(r1.z), bf16hi(r1.z), bf16lo(r1.w), bf16hi(r1.w)};
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));   // every lane takes part
      const int code = e8m0_code(amax);
      const int e = code - 127;
      const uint4 qv = make_uint4(quant4(f, e), quant4(f + 4, e), quant4(f + 8, e), quant4(f + 12, e));
      const uint32_t c1 = (uint32_t)__shfl_down(code, 2, 64), c2 = (uint32_t)__shfl_down(code, 4, 64),
                     c3 = (uint32_t)__shfl_down(code, 6, 64);
      if (pc < npair) {
        *reinterpret_cast<uint4*>(qrow + pc * 16) = qv;
        if ((lane & 7) == 0)
          *reinterpret_cast<uint32_t*>(crow + (pc >> 1)) = (uint32_t)code | (c1 << 8) | (c2 << 16) | (c3 << 24);
      }
    }
  }
}

// h = bf16(silu(g) * u), optionally quantized row-wise; one wave per row
__global__ __launch_bounds__(256) void swiglu_kernel(const uint16_t* __restrict__ g,
                                                     const uint16_t* __restrict__ u, int64_t rows,
                                                     int n, uint16_t* __restrict__ h,
                                                     uint8_t* __restrict__ hq,
                                                     uint8_t* __restrict__ hs) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int nvec = n >> 3;
  for (int v0 = 0; v0 < nvec; v0 += kWave) {
    const int v = v0 + lane;
    uint4 out = make_uint4(0, 0, 0, 0);
    if (v < nvec) {
      uint4 a = ldg16(g + r * n + v * 8), b = ldg16(u + r * n + v * 8);
      uint32_t ga[4] = {a.x, a.y, a.z, a.w}, ub[4] = {b.x, b.y, b.z, b.w}, o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float g0 = bf16lo(ga[i]), g1 = bf16hi(ga[i]);
        float h0 = g0 * sigmoidf_(g0) * bf16lo(ub[i]);
        float h1 = g1 * sigmoidf_(g1) * bf16hi(ub[i]);
        o[i] = pack_bf16x2(h0, h1);
      }
      out = make_uint4(o[0], o[1], o[2], o[3]);
      if (h) stg16(h + r * n + v * 8, out);
    }
    if (hq) {
      int code;
      uint2 qq = quant_vec(out, code);
      if (v < nvec) {
        *reinterpret_cast<uint2*>(hq + r * n + v * 8) = qq;
        if ((v & 3) == 0) hs[r * (n >> 5) + (v >> 2)] = (uint8_t)code;
      }
    }
  }
}

// ---- host launchers -----------------------------------------------------------
static inline unsigned waves_grid(int64_t rows) { return (unsigned)((rows + 3) / 4); }

hipError_t launch_dispatch_bf16(const void* x, const int32_t* dst_rows, const float* weight,
                                int64_t N, int64_t D, int64_t K, void* xd, hipStream_t s,
                                const int32_t* shared_row0) {
  if (N == 0) return hipSuccess;
  if (weight)
    dispatch_bf16_kernel<true><<<waves_grid(N), 256, 0, s>>>((const uint16_t*)x, dst_rows, weight,
                                                            (int)N, (int)D, (int)K, (uint16_t*)xd, shared_row0);
  else
    dispatch_bf16_kernel<false><<<waves_grid(N), 256, 0, s>>>((const uint16_t*)x, dst_rows, nullptr,
                                                             (int)N, (int)D, (int)K, (uint16_t*)xd, shared_row0);
  return hipGetLastError();
}

hipError_t launch_dispatch_mxfp8(const void* x, const int32_t* dst_rows, int64_t N, int64_t D,
                                 int64_t K, uint8_t* q, uint8_t* sc, hipStream_t s, const int32_t* shared_row0,
                                 const int32_t* pad_counts, const int32_t* pad_offsets, int64_t pad_E) {
  if (N == 0) return hipSuccess;
  const bool packed = D % 128 == 0 && ((uintptr_t)sc & 3) == 0;
  const unsigned grid = waves_grid(packed ? N * perm::mx_dispatch_segs((int)D) : N) +
                        (pad_counts ? (unsigned)pad_E : 0u);
  if (packed)
    dispatch_mxfp8_packed_kernel<<<grid, 256, 0, s>>>((const uint16_t*)x, dst_rows, (int)N, (int)D, (int)K, q,
                                                      sc, shared_row0, pad_counts, pad_offsets);
  else
    dispatch_mxfp8_kernel<<<grid, 256, 0, s>>>((const uint16_t*)x, dst_rows, (int)N, (int)D, (int)K, q, sc,
                                               shared_row0, pad_counts, pad_offsets);
  return hipGetLastError();
}

hipError_t launch_zero_bytes(void* p, int64_t bytes, hipStream_t s) {
  if (bytes <= 0) return hipSuccess;
  const int64_t n16 = bytes / 16;
  const int64_t blocks = (n16 + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 1 ? 1 : (blocks > 4096 ? 4096 : blocks));
  zero_bytes_kernel<<<grid, 256, 0, s>>>((uint8_t*)p, n16, bytes);
  return hipGetLastError();
}

hipError_t launch_zero_padding(const int32_t* counts, const int32_t* offsets, int64_t E,
                               int64_t row_bytes, void* a, int64_t row_bytes2, void* b,
                               hipStream_t s, int64_t row_bytes3, void* c) {
  if (E == 0) return hipSuccess;
  zero_padding_kernel<<<(unsigned)E, kPadThreads, 0, s>>>(counts, offsets, row_bytes, (uint8_t*)a,
                                                   row_bytes2, (uint8_t*)b, row_bytes3, (uint8_t*)c);
  return hipGetLastError();
}

hipError_t launch_combine(const void* y, const int32_t* dst_rows, const float* weight, int64_t N,
                          int64_t D, int64_t K, void* out, hipStream_t s, const void* addend,
                          const int32_t* shared_row0) {
  if (N == 0) return hipSuccess;
  const int nseg = perm::combine_segs((int)(D >> 3));
  const unsigned grid = waves_grid(N * nseg);
  if (weight)
    combine_kernel<true><<<grid, 256, 0, s>>>((const uint16_t*)y, dst_rows, weight, (int)N, (int)D, (int)K,
                                             (uint16_t*)out, (const uint16_t*)addend, shared_row0, nseg);
  else
    combine_kernel<false><<<grid, 256, 0, s>>>((const uint16_t*)y, dst_rows, nullptr, (int)N, (int)D, (int)K,
                                              (uint16_t*)out, (const uint16_t*)addend, shared_row0, nseg);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const void* dout, const int32_t* dst_rows, const float* weight,
                              const void* y, int64_t N, int64_t D, int64_t K, void* dyd,
                              float* dprob, hipStream_t s, const int32_t* shared_row0, uint8_t* q, uint8_t* sc) {
  if (N == 0) return hipSuccess;
  if (q) {
    if (!combine_bwd_quant_ok(D, q, sc)) return hipErrorInvalidValue;
    combine_bwd_kernel<true><<<waves_grid(N), 256, 0, s>>>((const uint16_t*)dout, dst_rows, weight,
                                                           (const uint16_t*)y, (int)N, (int)D, (int)K,
                                                           (uint16_t*)dyd, dprob, shared_row0, q, sc);
  } else {
    combine_bwd_kernel<false><<<waves_grid(N), 256, 0, s>>>((const uint16_t*)dout, dst_rows, weight,
                                                            (const uint16_t*)y, (int)N, (int)D, (int)K,
                                                            (uint16_t*)dyd, dprob, shared_row0, nullptr, nullptr);
  }
  return hipGetLastError();
}

bool combine_bwd_quant_ok(int64_t D, const void* q, const void* sc) {
  return D % 128 == 0 && ((uintptr_t)q & 15) == 0 && ((uintptr_t)sc & 3) == 0;
}

hipError_t launch_quantize_rows(const void* src, int64_t rows, int64_t cols, uint8_t* q,
                                uint8_t* sc, hipStream_t s, const int32_t* rows_end) {
  if (rows == 0) return hipSuccess;
  if (cols % 128 == 0 && ((uintptr_t)q & 15) == 0 && ((uintptr_t)sc & 3) == 0)
    quantize_rows_packed_kernel<<<waves_grid(rows), 256, 0, s>>>((const uint16_t*)src, rows, (int)cols, q, sc,
                                                                 rows_end);
  else
    quantize_rows_kernel<<<waves_grid(rows), 256, 0, s>>>((const uint16_t*)src, rows, (int)cols, q, sc, rows_end);
  return hipGetLastError();
}

hipError_t launch_swiglu(const void* g, const void* u, int64_t rows, int64_t n, void* h,
                         uint8_t* hq, uint8_t* hs, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  swiglu_kernel<<<waves_grid(rows), 256, 0, s>>>((const uint16_t*)g, (const uint16_t*)u, rows, (int)n,
                                                 (uint16_t*)h, hq, hs);
  return hipGetLastError();
}

}  // namespace moe
