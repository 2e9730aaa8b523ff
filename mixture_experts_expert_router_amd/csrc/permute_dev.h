// Device bodies of the token-row permutes that the persistent layer kernels
// run inside their workgroups as well: the MXFP8 dispatch of a row segment,
// the fold (combine) of a row segment, the combine backward of a token, and
// their vector helpers.  permute.hip launches them a wave per segment or
// token.
#pragma once

#include "common.h"

namespace moe {
namespace perm {

__device__ __forceinline__ uint4 scale_bf16x8(uint4 v, float w) {
  uint4 o;
  o.x = pack_bf16x2(w * bf16lo(v.x), w * bf16hi(v.x));
  o.y = pack_bf16x2(w * bf16lo(v.y), w * bf16hi(v.y));
  o.z = pack_bf16x2(w * bf16lo(v.z), w * bf16hi(v.z));
  o.w = pack_bf16x2(w * bf16lo(v.w), w * bf16hi(v.w));
  return o;
}

__device__ __forceinline__ uint32_t quant4(const float* f, int e) {
  return e4m3x4(f[0], f[1], f[2], f[3], e);
}

// MXFP8 dispatch of segment seg of token t's row by one wave (D % 128 == 0):
// the segment quantized once and its codes and scales written to the token's
// rows (route k to dst_rows[t, k], the shared expert's row srow last when
// srow >= 0).  A lane takes 16 adjacent elements, so a 32-block is a lane
// pair; a route gets one 16-byte code store a lane, and lanes 8i pack the
// codes of four consecutive blocks into one 4-byte store.  A segment is one
// pass of kMxSegPieces 16-element pieces (4 a lane), so a wave's loads never
// queue behind its own stores of an earlier pass (vector memory operations
// complete in order).
constexpr int kMxSegPieces = kWave * 4;
__device__ __host__ __forceinline__ int mx_dispatch_segs(int D) {
  return ((D >> 4) + kMxSegPieces - 1) / kMxSegPieces;
}

__device__ __forceinline__ void dispatch_mx_token(int t, int seg, const uint16_t* __restrict__ x,
                                                  const int32_t* __restrict__ dst_rows, int D, int K, int srow,
                                                  uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
  constexpr int PP = kMxSegPieces / kWave;   // lane pairs of vectors per pass
  const int lane = threadIdx.x & 63;
  const int KK = K + (srow >= 0 ? 1 : 0);
  const int npair = D >> 4;              // 16-element pieces per row
  const int nblk = D >> 5;
  const uint16_t* src = x + (int64_t)t * D;
  // the token's destination rows, lane k holding route k's: one vector load,
  // read back with readlane, so the store loop waits on no load per route
  const int dkl = lane < K ? dst_rows[(int64_t)t * K + lane] : -1;
  {
    const int p0 = seg * kMxSegPieces;
    uint4 qv[PP];
    uint32_t packed[PP];
#pragma unroll
    for (int j = 0; j < PP; ++j) {
      const int pc = p0 + lane + j * kWave;   // this lane's 16-element piece
      uint4 r0 = make_uint4(0, 0, 0, 0), r1 = make_uint4(0, 0, 0, 0);
      if (pc < npair) {
        r0 = ldg16(src + pc * 16);
        r1 = ldg16(src + pc * 16 + 8);
      }
      float f[16] = {bf16lo(r0.x), bf16hi(r0.x), bf16lo(r0.y), bf16hi(r0.y), bf16lo(r0.z), bf16hi(r0.z),
                     bf16lo(r0.w), bf16hi(r0.w), bf16lo(r1.x), bf16hi(r1.x), bf16lo(r1.y), bf16hi(r1.y),
                     bf16lo(r1.z), bf16hi(r1.z), bf16lo(r1.w), bf16hi(r1.w)};
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      const int code = e8m0_code(amax);
      const int e = code - 127;
      qv[j] = make_uint4(quant4(f, e), quant4(f + 4, e), quant4(f + 8, e), quant4(f + 12, e));
      // block codes of lanes 8i, 8i+2, 8i+4, 8i+6 into lane 8i
      const uint32_t c1 = (uint32_t)__shfl_down(code, 2, 64), c2 = (uint32_t)__shfl_down(code, 4, 64),
                     c3 = (uint32_t)__shfl_down(code, 6, 64);
      packed[j] = (uint32_t)code | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
    for (int k = 0; k < KK; ++k) {
      const int dk = k < K ? __builtin_amdgcn_readlane(dkl, k) : srow;
      if (dk < 0) continue;
      uint8_t* qrow = q + (int64_t)dk * D;
      uint8_t* crow = sc + (int64_t)dk * nblk;
#pragma unroll
      for (int j = 0; j < PP; ++j) {
        const int pc = p0 + lane + j * kWave;
        if (pc < npair) {
          *reinterpret_cast<uint4*>(qrow + pc * 16) = qv[j];
          if ((lane & 7) == 0) *reinterpret_cast<uint32_t*>(crow + (pc >> 1)) = packed[j];
        }
      }
    }
  }
}

// Zero the padding rows [offsets[e] + counts[e], offsets[e+1]) of expert e in
// the MXFP8 dispatch output: codes (D bytes a row, 16-byte stores) and scales
// (D/32 bytes a row), the workgroup's nwaves waves taking the rows in turn.
__device__ __forceinline__ void zero_pad_rows_mx(int e, const int32_t* __restrict__ counts,
                                                 const int32_t* __restrict__ offsets, int D,
                                                 uint8_t* __restrict__ q, uint8_t* __restrict__ sc, int nwaves) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r0 = offsets[e] + counts[e], r1 = offsets[e + 1];
  const int nb = D >> 5;
  for (int64_t r = r0 + wave; r < r1; r += nwaves) {
    uint4* pq = reinterpret_cast<uint4*>(q + r * D);
    for (int i = lane; i < (D >> 4); i += 64) pq[i] = make_uint4(0, 0, 0, 0);
    uint8_t* ps = sc + r * nb;
    for (int i = lane; i < nb; i += 64) ps[i] = 0;
  }
}

// The fold (combine) of token rows: out[t] = bf16(sum over k of w[t,k]
// y[dst[t,k]] (+ addend[t])), fp32 fmaf in ascending k, the shared expert's
// row (weight 1) last.  A row of nvec 16-byte vectors is cut into
// combine_segs(nvec) segments of at most kSegV vectors per lane; one wave
// folds one segment, reading each route's part of the row as one long run
// (measured: 7 KB runs of two routes at a time keep HBM busier than 2 KB runs
// of eight routes) with the next route's run in flight while one is added.
// The gathered rows and the output are touched once: non-temporal accesses.
constexpr int kSegV = 7;
__device__ __host__ __forceinline__ int combine_segs(int nvec) {
  return (nvec + kSegV * kWave - 1) / (kSegV * kWave);
}

template <bool WEIGHTED>
__device__ __forceinline__ void combine_seg(int t, int seg, int nseg, const uint16_t* __restrict__ y,
                                            const int32_t* __restrict__ dst_rows,
                                            const float* __restrict__ weight, int D, int K,
                                            uint16_t* __restrict__ out, const uint16_t* __restrict__ addend,
                                            const int32_t* __restrict__ shared_row0) {
  constexpr int KC = 2;
  const int lane = threadIdx.x & 63;
  const int nvec = D >> 3;
  const int vl = (nvec + nseg * kWave - 1) / (nseg * kWave);   // vectors per lane, at most kSegV
  const int vb = seg * vl * kWave + lane;                      // this lane's first vector
  // route K (when there is a shared expert): its row of this token, weight 1
  const int KK = K + (shared_row0 ? 1 : 0);
  const int srow = shared_row0 ? *shared_row0 + t : -1;
  float acc[kSegV][8];
#pragma unroll
  for (int j = 0; j < kSegV; ++j) {
    const int v = vb + j * kWave;
    const uint4 q = (addend && j < vl && v < nvec) ? ldg16(addend + (int64_t)t * D + v * 8) : make_uint4(0, 0, 0, 0);
    acc[j][0] = bf16lo(q.x);
    acc[j][1] = bf16hi(q.x);
    acc[j][2] = bf16lo(q.y);
    acc[j][3] = bf16hi(q.y);
    acc[j][4] = bf16lo(q.z);
    acc[j][5] = bf16hi(q.z);
    acc[j][6] = bf16lo(q.w);
    acc[j][7] = bf16hi(q.w);
  }
  for (int k0 = 0; k0 < KK; k0 += KC) {
    uint4 r[KC][kSegV];
    int dk[KC];
    float wk[KC];
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      const int k = k0 + kk;
      dk[kk] = k < K ? dst_rows[(int64_t)t * K + k] : (k == K ? srow : -1);
      wk[kk] = (WEIGHTED && k < K) ? weight[(int64_t)t * K + k] : 1.0f;
      const uint16_t* src = y + (int64_t)(dk[kk] < 0 ? 0 : dk[kk]) * D;
#pragma unroll
      for (int j = 0; j < kSegV; ++j) {
        const int v = vb + j * kWave;
        r[kk][j] = (dk[kk] >= 0 && j < vl && v < nvec) ? ldg16_nt(src + v * 8) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      if (dk[kk] < 0) continue;
      const float w = wk[kk];
#pragma unroll
      for (int j = 0; j < kSegV; ++j) {
        const uint4 q = r[kk][j];
        acc[j][0] = fmaf(w, bf16lo(q.x), acc[j][0]);
        acc[j][1] = fmaf(w, bf16hi(q.x), acc[j][1]);
        acc[j][2] = fmaf(w, bf16lo(q.y), acc[j][2]);
        acc[j][3] = fmaf(w, bf16hi(q.y), acc[j][3]);
        acc[j][4] = fmaf(w, bf16lo(q.z), acc[j][4]);
        acc[j][5] = fmaf(w, bf16hi(q.z), acc[j][5]);
        acc[j][6] = fmaf(w, bf16lo(q.w), acc[j][6]);
        acc[j][7] = fmaf(w, bf16hi(q.w), acc[j][7]);
      }
    }
  }
  uint16_t* o = out + (int64_t)t * D;
#pragma unroll
  for (int j = 0; j < kSegV; ++j) {
    const int v = vb + j * kWave;
    if (j < vl && v < nvec)
      stg16_nt(o + v * 8, make_uint4(pack_bf16x2(acc[j][0], acc[j][1]), pack_bf16x2(acc[j][2], acc[j][3]),
                                     pack_bf16x2(acc[j][4], acc[j][5]), pack_bf16x2(acc[j][6], acc[j][7])));
  }
}

// The fold of token t (wave-uniform) by one wave, segment after segment.
template <bool WEIGHTED>
__device__ __forceinline__ void combine_token(int t, const uint16_t* __restrict__ y,
                                              const int32_t* __restrict__ dst_rows,
                                              const float* __restrict__ weight, int D, int K,
                                              uint16_t* __restrict__ out, const uint16_t* __restrict__ addend,
                                              const int32_t* __restrict__ shared_row0) {
  const int nseg = combine_segs(D >> 3);
  for (int s = 0; s < nseg; ++s)
    combine_seg<WEIGHTED>(t, s, nseg, y, dst_rows, weight, D, K, out, addend, shared_row0);
}

// combine backward: dyd[dst] = bf16(w * dout[t]); dprob[t,k] = <dout[t], y[dst]>
// The combine backward of token t (wave-uniform) by one wave: dY_d rows of
// its valid routes and dprob.  QUANT (D % 128 == 0): each dY_d row is also quantized row-wise to MXFP8
// where it lands (KOSMOS section 3.3.2 step 1), the same codes a separate
// quantize_rows pass over dyd gives: a lane holds 8 elements, so a 32-block
// is a lane quad; 8-byte code stores, and lanes 16i store the scales of four
// consecutive blocks as one word.
template <bool QUANT>
__device__ __forceinline__ void combine_bwd_token(int t, const uint16_t* __restrict__ dout,
                                                  const int32_t* __restrict__ dst_rows,
                                                  const float* __restrict__ weight,
                                                  const uint16_t* __restrict__ y, int D, int K,
                                                  uint16_t* __restrict__ dyd, float* __restrict__ dprob,
                                                  const int32_t* __restrict__ shared_row0,
                                                  uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
  // routes in chunks of KCH: every Y row of the chunk is loaded before any
  // product uses it, so the gathers overlap instead of waiting one by one;
  // each lane still sums its vectors in increasing order
  constexpr int VPL = 2, KCH = 8;
  const int lane = threadIdx.x & 63;
  const int nvec = D >> 3;
  const uint16_t* src = dout + (int64_t)t * D;
  // route K (when there is a shared expert): dY of its row is dOut, weight 1,
  // and it has no route weight to differentiate
  const int KK = K + (shared_row0 ? 1 : 0);
  const int srow = shared_row0 ? *shared_row0 + t : -1;
  for (int kb = 0; kb < KK; kb += KCH) {
    int dk[KCH];
    float wk[KCH], dot[KCH];
#pragma unroll
    for (int kk = 0; kk < KCH; ++kk) {
      const int k = kb + kk;
      dk[kk] = k < K ? dst_rows[(int64_t)t * K + k] : (k == K ? srow : -1);
      wk[kk] = k < K ? weight[(int64_t)t * K + k] : 1.0f;
      dot[kk] = 0.0f;
    }
    for (int v0 = 0; v0 < nvec; v0 += kWave * VPL) {
      uint4 r[VPL];
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int v = v0 + lane + j * kWave;
        r[j] = v < nvec ? ldg16(src + v * 8) : make_uint4(0, 0, 0, 0);
      }
      uint4 yy[KCH][VPL];
      if (dprob) {
#pragma unroll
        for (int kk = 0; kk < KCH; ++kk)
#pragma unroll
          for (int j = 0; j < VPL; ++j) {
            const int v = v0 + lane + j * kWave;
            yy[kk][j] = (dk[kk] >= 0 && kb + kk < K && v < nvec) ? ldg16_nt(y + (int64_t)dk[kk] * D + v * 8)
                                                                  : make_uint4(0, 0, 0, 0);
          }
      }
#pragma unroll
      for (int kk = 0; kk < KCH; ++kk) {
        if (dk[kk] < 0) continue;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
          const int v = v0 + lane + j * kWave;
          const uint4 o = scale_bf16x8(r[j], wk[kk]);
          if constexpr (QUANT) {
            // every lane takes part in the shuffles; a quad is all in or all
            // out (nvec % 16 == 0), and lanes past the row hold zeros
            const float f[8] = {bf16lo(o.x), bf16hi(o.x), bf16lo(o.y), bf16hi(o.y),
                                bf16lo(o.z), bf16hi(o.z), bf16lo(o.w), bf16hi(o.w)};
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
            amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
            amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
            const int code = e8m0_code(amax);
            const int e = code - 127;
            const uint2 qv = make_uint2(quant4(f, e), quant4(f + 4, e));
            const uint32_t c1 = (uint32_t)__shfl_down(code, 4, 64), c2 = (uint32_t)__shfl_down(code, 8, 64),
                           c3 = (uint32_t)__shfl_down(code, 12, 64);
            if (v < nvec) {
              *reinterpret_cast<uint2*>(q + (int64_t)dk[kk] * D + v * 8) = qv;
              if ((lane & 15) == 0)
                *reinterpret_cast<uint32_t*>(sc + (int64_t)dk[kk] * (D >> 5) + (v >> 2)) =
                    (uint32_t)code | (c1 << 8) | (c2 << 16) | (c3 << 24);
            }
          }
          if (v >= nvec) continue;
          stg16(dyd + (int64_t)dk[kk] * D + v * 8, o);
          if (dprob) {
            const uint4 q = yy[kk][j];
            float s2 = dot[kk];
            s2 = fmaf(bf16lo(r[j].x), bf16lo(q.x), s2);
            s2 = fmaf(bf16hi(r[j].x), bf16hi(q.x), s2);
            s2 = fmaf(bf16lo(r[j].y), bf16lo(q.y), s2);
            s2 = fmaf(bf16hi(r[j].y), bf16hi(q.y), s2);
            s2 = fmaf(bf16lo(r[j].z), bf16lo(q.z), s2);
            s2 = fmaf(bf16hi(r[j].z), bf16hi(q.z), s2);
            s2 = fmaf(bf16lo(r[j].w), bf16lo(q.w), s2);
            s2 = fmaf(bf16hi(r[j].w), bf16hi(q.w), s2);
            dot[kk] = s2;
          }
        }
      }
    }
    if (dprob) {
#pragma unroll
      for (int kk = 0; kk < KCH; ++kk) {
        const float sum = wave_sum(dot[kk]);
        if (lane == 0 && kb + kk < K) dprob[(int64_t)t * K + kb + kk] = dk[kk] >= 0 ? sum : 0.0f;
      }
    }
  }
}

}  // namespace perm
}  // namespace moe
