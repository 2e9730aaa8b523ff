// Route: softmax + top-K per token, then the route map by a stable counting
// sort (KOSMOS section 3.3.1 steps 1-2, "Route" and "Plan"; OLMo-core
// Appendix A, A.2-A.3: dst_rows[N,K], route id t*K+k, -1 = invalid).
//
// Three launches, none with a contended global atomic (the multi-XCD atomic
// trap described in the Meta MI350X paper, section IV-B1):
//   1. route_topk: one wave per token computes softmax and top-K; each
//      workgroup (one wave per token of its chunk) owns a chunk of kChunk
//      tokens and, in LDS, the stable rank of every route inside its chunk
//      plus the chunk's per-expert histogram.
//   2. route_scan: one workgroup turns the [chunks][E] histogram into counts,
//      aligned offsets and the first row of every (chunk, expert) pair.
//   3. route_scatter: every valid route's row = base(chunk, e) + rank.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kChunk = 16;         // tokens per workgroup in route_topk (one per wave)
constexpr int kTopkThreads = kChunk * 64;
constexpr int kMaxE = 1024;
constexpr int kMaxPerLane = kMaxE / kWave;

// (value desc, index asc): true if (va, ia) ranks before (vb, ib)
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(kTopkThreads) void route_topk_kernel(
    const float* __restrict__ logits, const uint8_t* __restrict__ drop, int N, int E, int K,
    int renorm, int32_t* __restrict__ topk_idx, float* __restrict__ topk_prob,
    int32_t* __restrict__ row_route, int64_t rows_cap, int32_t* __restrict__ hist,
    int32_t* __restrict__ rank) {
  __shared__ int s_sel[kChunk * 32];      // K <= 32 checked on the host
  __shared__ int s_hist[kMaxE];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kChunk;

  // row_route = -1 everywhere first (the scatter overwrites the used rows)
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows_cap;
       i += (int64_t)gridDim.x * blockDim.x)
    row_route[i] = -1;
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_hist[e] = 0;

  for (int tl = wave; tl < kChunk; tl += kTopkThreads / 64) {
    const int t = t0 + tl;
    if (t >= N) {
      if (lane < K) s_sel[tl * K + lane] = -1;
      continue;
    }
    float v[kMaxPerLane];
    const float* row = logits + (int64_t)t * E;
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      int e = lane + j * kWave;
      v[j] = (e < E) ? row[e] : -INFINITY;
      mx = fmaxf(mx, v[j]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    float se = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      int e = lane + j * kWave;
      if (e < E) se += expf(v[j] - mx);
    }
    se = wave_sum(se);
    // top-K: K rounds of a wave arg-max (value desc, index asc)
    uint32_t taken = 0;
    float psel = 0.0f;       // this lane's slot-k probability, lane k holds slot k
    int isel = 0;
    for (int k = 0; k < K; ++k) {
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int j = 0; j < kMaxPerLane; ++j) {
        int e = lane + j * kWave;
        if (e < E && !((taken >> j) & 1u) && better(v[j], e, bv, bi)) { bv = v[j]; bi = e; }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        float ov = __shfl_xor(bv, o, 64);
        int oi = __shfl_xor(bi, o, 64);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
      if (lane == k) { isel = bi; psel = expf(bv - mx) / se; }
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
      const bool valid = drop == nullptr || drop[r] == 0;
      s_sel[tl * K + lane] = valid ? isel : -1;
    }
  }
  __syncthreads();

  // stable rank of each route within the chunk: routes of earlier tokens with
  // the same expert (a token's K experts are distinct)
  for (int rl = threadIdx.x; rl < kChunk * K; rl += blockDim.x) {
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
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(int64_t)blockIdx.x * E + e] = s_hist[e];
}

// One workgroup of 1024 threads.  Thread (e, g) owns expert e and the chunk
// range of group g; partial sums are scanned over groups, then over experts.
__global__ __launch_bounds__(1024) void route_scan_kernel(int32_t* __restrict__ hist, int nchunks,
                                                          int E, int align,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets) {
  __shared__ int s_part[1024];
  __shared__ int s_tot[kMaxE];
  __shared__ int s_off[kMaxE + 1];
  int Ep = 1;
  while (Ep < E) Ep <<= 1;
  const int G = 1024 / Ep;                       // chunk groups
  const int cpg = (nchunks + G - 1) / G;         // chunks per group
  const int e = threadIdx.x % Ep;
  const int g = threadIdx.x / Ep;
  int sum = 0;
  if (e < E) {
    // loads in batches of 16, so they are in flight together
    const int c1 = min(nchunks, (g + 1) * cpg);
    for (int c0 = g * cpg; c0 < c1; c0 += 16) {
      int h[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) h[i] = c0 + i < c1 ? hist[(int64_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) sum += h[i];
    }
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
    __shared__ int s_wsum[16];
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
      for (int w = 0; w < 16; ++w) { int t = s_wsum[w]; s_wsum[w] = run; run += t; }
    }
    __syncthreads();
    inc += s_wsum[wv];
    if (threadIdx.x < E) s_off[threadIdx.x] = inc - own;
    if (threadIdx.x == E - 1) s_off[E] = inc;
    if (E == 0 && threadIdx.x == 0) s_off[0] = 0;
  }
  __syncthreads();
  for (int ee = threadIdx.x; ee <= E; ee += blockDim.x) offsets[ee] = s_off[ee];
  if (e < E) {
    int run = s_off[e] + s_part[g * Ep + e];
    const int c1 = min(nchunks, (g + 1) * cpg);
    for (int c0 = g * cpg; c0 < c1; c0 += 16) {
      int h[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) h[i] = c0 + i < c1 ? hist[(int64_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (c0 + i < c1) hist[(int64_t)(c0 + i) * E + e] = run;   // first row of (chunk, e)
        run += h[i];
      }
    }
  }
}

__global__ __launch_bounds__(256) void route_scatter_kernel(
    const int32_t* __restrict__ topk_idx, const uint8_t* __restrict__ drop,
    const int32_t* __restrict__ base, const int32_t* __restrict__ rank, int64_t NK, int K, int E,
    int32_t* __restrict__ dst_rows, int32_t* __restrict__ row_route) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= NK) return;
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

size_t route_workspace_bytes(int64_t N, int64_t E, int64_t K) {
  const int64_t nchunks = N > 0 ? (N + kChunk - 1) / kChunk : 1;
  size_t b = (size_t)nchunks * E * 4;   // hist / bases
  b = (b + 255) & ~(size_t)255;
  b += (size_t)N * K * 4;               // in-chunk ranks
  return (b + 255) & ~(size_t)255;
}

hipError_t launch_route(const float* logits, const uint8_t* drop, int64_t N, int64_t E, int64_t K,
                        int renorm, int align, int64_t rows_cap, int32_t* topk_idx, float* topk_prob,
                        int32_t* counts, int32_t* offsets, int32_t* dst_rows, int32_t* row_route,
                        void* ws, hipStream_t s) {
  const int64_t nchunks = (N + kChunk - 1) / kChunk;
  const int64_t nalloc = nchunks > 0 ? nchunks : 1;
  int32_t* hist = (int32_t*)ws;
  size_t hb = ((size_t)nalloc * E * 4 + 255) & ~(size_t)255;
  int32_t* rank = (int32_t*)((char*)ws + hb);
  if (nchunks > 0) {
    route_topk_kernel<<<dim3((unsigned)nchunks), dim3(kTopkThreads), 0, s>>>(
        logits, drop, (int)N, (int)E, (int)K, renorm, topk_idx, topk_prob, row_route, rows_cap,
        hist, rank);
  } else {
    // no tokens: still mark every row unused
    route_topk_kernel<<<dim3(1), dim3(kTopkThreads), 0, s>>>(logits, drop, 0, (int)E, (int)K, renorm,
                                                    topk_idx, topk_prob, row_route, rows_cap,
                                                    hist, rank);
  }
  route_scan_kernel<<<dim3(1), dim3(1024), 0, s>>>(hist, (int)nchunks, (int)E, align, counts,
                                                   offsets);
  const int64_t NK = N * K;
  if (NK > 0) {
    route_scatter_kernel<<<dim3((unsigned)((NK + 255) / 256)), dim3(256), 0, s>>>(
        topk_idx, drop, hist, rank, NK, (int)K, (int)E, dst_rows, row_route);
  }
  return hipGetLastError();
}

}  // namespace moe
