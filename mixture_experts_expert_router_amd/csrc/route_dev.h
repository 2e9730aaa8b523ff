// Device bodies of the route step (KOSMOS section 3.3.1 steps 1-2, "Route"
// and "Plan"): softmax and top-K with the in-chunk ranks and the per-chunk
// histogram, the histogram scan, the scatter.  route.hip launches them as
// three kernels; the single-launch layer runs them inside its persistent
// workgroups.  Each body takes its workgroup size as a template parameter
// and its LDS as arguments, and computes the same values at any size.
#pragma once

#include "common.h"

namespace moe {
namespace route {

constexpr int kChunk = 16;   // tokens per route chunk (one histogram row)
constexpr int kMaxE = 1024;

// bytes of the histogram ([chunks][E] ints, at least one chunk) at the start
// of the route workspace; the in-chunk ranks follow
inline size_t hist_bytes(int64_t N, int64_t E) {
  const int64_t nchunks = N > 0 ? (N + kChunk - 1) / kChunk : 1;
  return ((size_t)nchunks * E * 4 + 255) & ~(size_t)255;
}

// (value desc, index asc): true if (va, ia) ranks before (vb, ib)
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Top-K of the kChunk tokens of `chunk` by a workgroup of THREADS threads,
// a token per wave at a time, in order; writes topk_idx / topk_prob, the
// in-chunk rank of every valid route and the chunk's histogram row.
// Group-limited selection (n_group > 1): the experts form n_group contiguous
// groups; a group scores the sum of its two largest routing probabilities,
// the topk_group best groups (ties to the lower group) are kept, and top-K
// runs over their experts.  psum (optional): this chunk's per-expert sums of
// the routing probabilities, the aux-loss input.  Both use a dynamic LDS row
// of E floats per wave.
// NPL: logits per lane (E <= 64 NPL), so loads, exps and the arg-max rounds
// touch only the experts that exist
// LDS: s_sel [kChunk * 32] and s_hist [E] ints; s_row [kChunk][E] floats when
// grouped or psum.  psum needs THREADS == kChunk * 64 (a wave per token).
template <int NPL, int THREADS>
__device__ __forceinline__ void topk_chunk(int chunk, const float* __restrict__ logits,
                                           const uint8_t* __restrict__ drop, int N, int E, int K, int renorm,
                                           int32_t* __restrict__ topk_idx, float* __restrict__ topk_prob,
                                           int32_t* __restrict__ hist, int32_t* __restrict__ rank, int n_group,
                                           int topk_group, float* __restrict__ psum, int32_t* __restrict__ status,
                                           int* s_sel, int* s_hist, float* s_row) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = chunk * kChunk;
  const bool grouped = n_group > 1;
  float pacc[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) pacc[j] = 0.0f;

  for (int e = threadIdx.x; e < E; e += THREADS) s_hist[e] = 0;

  for (int tl = wave; tl < kChunk; tl += THREADS / 64) {
    const int t = t0 + tl;
    if (t >= N) {
      if (lane < K) s_sel[tl * K + lane] = -1;
      continue;
    }
    float v[NPL];
    const float* row = logits + (int64_t)t * E;
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      int e = lane + j * kWave;
      v[j] = (e < E) ? row[e] : -INFINITY;
      mx = fmaxf(mx, v[j]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    float se = 0.0f;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      int e = lane + j * kWave;
      if (e < E) se += expf(v[j] - mx);
    }
    se = wave_sum(se);
    uint32_t taken = 0;
    if (grouped || psum) {
      float* prow = s_row + wave * E;
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        const int e = lane + j * kWave;
        if (e < E) {
          const float pj = expf(v[j] - mx) / se;
          pacc[j] += pj;
          prow[e] = pj;
        }
      }
      if (grouped) {
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        const int gs = E / n_group;
        float sc = -INFINITY;                  // lane g < n_group: group g's score
        if (lane < n_group) {
          float b1 = -INFINITY, b2 = -INFINITY;
          for (int i = 0; i < gs; ++i) {
            const float q = prow[lane * gs + i];
            if (q > b1) { b2 = b1; b1 = q; }
            else if (q > b2) b2 = q;
          }
          sc = gs > 1 ? b1 + b2 : b1;
        }
        uint64_t keep = 0;
        for (int r = 0; r < topk_group; ++r) {
          float bv = (lane < n_group && !((keep >> lane) & 1ull)) ? sc : -INFINITY;
          int bi = lane < n_group && !((keep >> lane) & 1ull) ? lane : 0x7FFFFFFF;
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(bv, o, 64);
            const int oi = __shfl_xor(bi, o, 64);
            if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
          }
          keep |= 1ull << bi;
        }
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
          const int e = lane + j * kWave;
          if (e < E && !((keep >> (e / gs)) & 1ull)) taken |= 1u << j;
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      }
    }
    // top-K: K rounds of a wave arg-max (value desc, index asc)
    float psel = 0.0f;       // this lane's slot-k probability, lane k holds slot k
    int isel = 0;
    for (int k = 0; k < K; ++k) {
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        int e = lane + j * kWave;
        if (e < E && !((taken >> j) & 1u) && better(v[j], e, bv, bi)) { bv = v[j]; bi = e; }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        float ov = __shfl_xor(bv, o, 64);
        int oi = __shfl_xor(bi, o, 64);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      // no candidate left only when the remaining logits are NaN: the slot
      // becomes an invalid route (expert -1, probability 0, no row)
      const bool found = bi != 0x7FFFFFFF;
      if (found && (bi & 63) == lane) taken |= 1u << (bi >> 6);
      if (lane == k) {
        isel = found ? bi : -1;
        psel = found ? expf(bv - mx) / se : 0.0f;
        if (!found && status) atomicOr(status, 2);
      }
    }
    if (renorm) {
      float s = (lane < K) ? psel : 0.0f;
      s = wave_sum(s);
      psel = psel / s;
    }
    if (lane < K) {
      const int64_t r = (int64_t)t * K + lane;
      topk_idx[r] = isel;
      topk_prob[r] = psel;
      const bool valid = (drop == nullptr || drop[r] == 0) && isel >= 0;
      s_sel[tl * K + lane] = valid ? isel : -1;
    }
  }
  __syncthreads();

  // stable rank of each route within the chunk: routes of earlier tokens with
  // the same expert (a token's K experts are distinct)
  for (int rl = threadIdx.x; rl < kChunk * K; rl += THREADS) {
    const int tl = rl / K;
    const int e = s_sel[rl];
    if (e < 0) continue;
    int c = 0;
    for (int j = 0; j < tl * K; ++j) c += (s_sel[j] == e);
    const int t = t0 + tl;
    rank[(int64_t)t * K + (rl - tl * K)] = c;
    atomicAdd(&s_hist[e], 1);           // LDS only; integer sums commute
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += THREADS) hist[(int64_t)chunk * E + e] = s_hist[e];
  if (psum) {
    // the chunk's probability sums, added over its waves in order
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int e = lane + j * kWave;
      if (e < E) s_row[wave * E + e] = pacc[j];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += THREADS) {
      float a = 0.0f;
      for (int w = 0; w < kChunk; ++w) a += s_row[w * E + e];
      psum[(int64_t)chunk * E + e] = a;
    }
  }
}

// Histogram scan by one workgroup of THREADS threads (E <= THREADS).  Thread
// (e, g) owns expert e and the chunk range of group g; partial sums are
// scanned over groups, then over experts.
// n_shared = 1: counts[E] = N and offsets[E+1] = offsets[E] + N rounded up to
// align, the shared expert's segment of every token.
// LDS: s_part [THREADS], s_tot [E], s_off [E + 1], s_wsum [THREADS / 64] ints.
template <int THREADS>
__device__ __forceinline__ void scan_hist(int32_t* __restrict__ hist, int nchunks, int E, int align,
                                          int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int N,
                                          int n_shared, int* s_part, int* s_tot, int* s_off, int* s_wsum) {
  int Ep = 1;
  while (Ep < E) Ep <<= 1;
  const int G = THREADS / Ep;                       // chunk groups
  const int cpg = (nchunks + G - 1) / G;         // chunks per group
  const int e = threadIdx.x % Ep;
  const int g = threadIdx.x / Ep;
  // The first kScanRegs counts of a thread's chunk range are loaded at once
  // and kept in registers for the second pass; the rest (large N only) are
  // read in batches of 16 in both passes.
  constexpr int kScanRegs = 64;
  const int cb = g * cpg, c1 = e < E ? min(nchunks, cb + cpg) : cb;
  int hr[kScanRegs];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kScanRegs; ++i) hr[i] = cb + i < c1 ? hist[(int64_t)(cb + i) * E + e] : 0;
#pragma unroll
  for (int i = 0; i < kScanRegs; ++i) sum += hr[i];
  for (int c0 = cb + kScanRegs; c0 < c1; c0 += 16) {
    int h[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) h[i] = c0 + i < c1 ? hist[(int64_t)(c0 + i) * E + e] : 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += h[i];
  }
  s_part[threadIdx.x] = sum;
  __syncthreads();
  if (g == 0 && e < E) {
    int run = 0;
    for (int gg = 0; gg < G; ++gg) {
      int p = s_part[gg * Ep + e];
      s_part[gg * Ep + e] = run;                 // exclusive prefix over groups
      run += p;
    }
    s_tot[e] = run;
    counts[e] = run;
  }
  __syncthreads();
  {
    // exclusive scan of the aligned segment sizes over experts: wave scans,
    // then a scan of the 16 wave totals
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int own = (threadIdx.x < E) ? ((s_tot[threadIdx.x] + align - 1) / align) * align : 0;
    int inc = own;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int n = __shfl_up(inc, o, 64);
      if (lane >= o) inc += n;
    }
    if (lane == 63) s_wsum[wv] = inc;
    __syncthreads();
    if (threadIdx.x == 0) {
      int run = 0;
      for (int w = 0; w < THREADS / 64; ++w) { int t = s_wsum[w]; s_wsum[w] = run; run += t; }
    }
    __syncthreads();
    inc += s_wsum[wv];
    if (threadIdx.x < E) s_off[threadIdx.x] = inc - own;
    if (threadIdx.x == E - 1) s_off[E] = inc;
    if (E == 0 && threadIdx.x == 0) s_off[0] = 0;
  }
  __syncthreads();
  for (int ee = threadIdx.x; ee <= E; ee += THREADS) offsets[ee] = s_off[ee];
  if (n_shared && threadIdx.x == 0) {
    counts[E] = N;
    offsets[E + 1] = s_off[E] + ((N + align - 1) / align) * align;
  }
  if (e < E) {
    int run = s_off[e] + s_part[g * Ep + e];
#pragma unroll
    for (int i = 0; i < kScanRegs; ++i) {
      if (cb + i < c1) hist[(int64_t)(cb + i) * E + e] = run;   // first row of (chunk, e)
      run += hr[i];
    }
    for (int c0 = cb + kScanRegs; c0 < c1; c0 += 16) {
      int h[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) h[i] = c0 + i < c1 ? hist[(int64_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (c0 + i < c1) hist[(int64_t)(c0 + i) * E + e] = run;
        run += h[i];
      }
    }
  }
}

// Route r's row: base(chunk, e) + its in-chunk rank; -1 for an invalid route.
__device__ __forceinline__ void scatter_route(int64_t r, const int32_t* __restrict__ topk_idx,
                                              const uint8_t* __restrict__ drop, const int32_t* __restrict__ base,
                                              const int32_t* __restrict__ rank, int K, int E,
                                              int32_t* __restrict__ dst_rows, int32_t* __restrict__ row_route) {
  const int e = topk_idx[r];
  const bool valid = (drop == nullptr || drop[r] == 0) && e >= 0 && e < E;
  if (!valid) {
    dst_rows[r] = -1;
    return;
  }
  const int64_t chunk = (r / K) / kChunk;
  const int dst = base[chunk * E + e] + rank[r];
  dst_rows[r] = dst;
  row_route[dst] = (int32_t)r;
}

// The single-launch layer's form of the scan, spread over the workgroups:
// expert e's column of the histogram is scanned by one workgroup of THREADS
// threads, each chunk's count replaced by the rows of e in the chunks before
// it (its first row relative to the expert's segment), the total written to
// counts[e].  The same prefix sums as scan_hist, in the same order.  LDS:
// s_w [THREADS / 64] ints.
template <int THREADS>
__device__ __forceinline__ void scan_expert(int32_t* __restrict__ hist, int nchunks, int E, int e,
                                            int32_t* __restrict__ counts, int* s_w) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int cpt = (nchunks + THREADS - 1) / THREADS;
  const int c0 = min(nchunks, t * cpt), c1 = min(nchunks, c0 + cpt);
  int sum = 0;
  for (int c = c0; c < c1; ++c) sum += hist[(int64_t)c * E + e];
  int inc = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(inc, o, 64);
    if (lane >= o) inc += n;
  }
  if (lane == 63) s_w[wv] = inc;
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int w = 0; w < THREADS / 64; ++w) { const int a = s_w[w]; s_w[w] = run; run += a; }
  }
  __syncthreads();
  int run = inc - sum + s_w[wv];
  for (int c = c0; c < c1; ++c) {
    const int h = hist[(int64_t)c * E + e];
    hist[(int64_t)c * E + e] = run;
    run += h;
  }
  if (t == THREADS - 1) counts[e] = run;
  __syncthreads();   // s_w is free for the next expert
}

// Segment offsets from the counts (E <= THREADS): s_off[e] = the aligned
// sizes of the experts before e, s_off[E] = the total, as scan_hist sets
// them.  LDS: s_off [E + 1], s_w [THREADS / 64] ints.
template <int THREADS>
__device__ __forceinline__ void offsets_of(const int32_t* __restrict__ counts, int E, int align, int* s_off,
                                           int* s_w) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int own = t < E ? ((counts[t] + align - 1) / align) * align : 0;
  int inc = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(inc, o, 64);
    if (lane >= o) inc += n;
  }
  if (lane == 63) s_w[wv] = inc;
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int w = 0; w < THREADS / 64; ++w) { const int a = s_w[w]; s_w[w] = run; run += a; }
  }
  __syncthreads();
  inc += s_w[wv];
  if (t < E) s_off[t] = inc - own;
  if (t == E - 1) s_off[E] = inc;
  if (E == 0 && t == 0) s_off[0] = 0;
  __syncthreads();
}

// scatter_route with chunk bases relative to the segments (scan_expert) and
// the segment offsets seg (offsets_of).
__device__ __forceinline__ void scatter_route_seg(int64_t r, const int32_t* __restrict__ topk_idx,
                                                  const uint8_t* __restrict__ drop,
                                                  const int32_t* __restrict__ base, const int* seg,
                                                  const int32_t* __restrict__ rank, int K, int E,
                                                  int32_t* __restrict__ dst_rows, int32_t* __restrict__ row_route) {
  const int e = topk_idx[r];
  const bool valid = (drop == nullptr || drop[r] == 0) && e >= 0 && e < E;
  if (!valid) {
    dst_rows[r] = -1;
    return;
  }
  const int64_t chunk = (r / K) / kChunk;
  const int dst = seg[e] + base[chunk * E + e] + rank[r];
  dst_rows[r] = dst;
  row_route[dst] = (int32_t)r;
}

}  // namespace route
}  // namespace moe
