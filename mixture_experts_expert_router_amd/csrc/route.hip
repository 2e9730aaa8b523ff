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

// (value desc, index asc): true if (va, ia) ranks before (vb, ib)
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Group-limited selection (n_group > 1): the experts form n_group contiguous
// groups; a group scores the sum of its two largest routing probabilities,
// the topk_group best groups (ties to the lower group) are kept, and top-K
// runs over their experts.  psum (optional): this chunk's per-expert sums of
// the routing probabilities, the aux-loss input.  Both use a dynamic LDS row
// of E floats per wave.
// NPL: logits per lane (E <= 64 NPL), so loads, exps and the arg-max rounds
// touch only the experts that exist
template <int NPL>
__global__ __launch_bounds__(kTopkThreads) void route_topk_kernel(
    const float* __restrict__ logits, const uint8_t* __restrict__ drop, int N, int E, int K,
    int renorm, int32_t* __restrict__ topk_idx, float* __restrict__ topk_prob,
    int32_t* __restrict__ row_route, int64_t rows_cap, int32_t* __restrict__ hist,
    int32_t* __restrict__ rank, int n_group, int topk_group, float* __restrict__ psum,
    int32_t* __restrict__ status) {
  __shared__ int s_sel[kChunk * 32];      // K <= 32 checked on the host
  __shared__ int s_hist[kMaxE];
  extern __shared__ float s_row[];        // [kChunk][E] when grouped or psum
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kChunk;
  const bool grouped = n_group > 1;
  float pacc[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) pacc[j] = 0.0f;

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
  if (psum) {
    // the chunk's probability sums, added over its waves in order
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int e = lane + j * kWave;
      if (e < E) s_row[wave * E + e] = pacc[j];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      float a = 0.0f;
      for (int w = 0; w < kChunk; ++w) a += s_row[w * E + e];
      psum[(int64_t)blockIdx.x * E + e] = a;
    }
  }
}

// Aux loss (KOSMOS section 3.3.1 step 1: the routing step's aux-loss inputs,
// reduced once per layer): P_e = the routing probabilities of expert e summed
// over tokens (one wave per expert, chunks strided over lanes, fixed order),
// then aux = alpha E sum_e (counts_e / (N K)) (P_e / N) in one wave.
__global__ __launch_bounds__(64) void aux_psum_kernel(const float* __restrict__ psum, int64_t nchunks, int E,
                                                      float* __restrict__ prob_sum) {
  const int e = blockIdx.x;
  float a = 0.0f;
  for (int64_t c = threadIdx.x; c < nchunks; c += 64) a += psum[c * E + e];
  a = wave_sum(a);
  if (threadIdx.x == 0) prob_sum[e] = a;
}

__global__ __launch_bounds__(64) void aux_loss_kernel(const float* __restrict__ prob_sum,
                                                      const int32_t* __restrict__ counts, int64_t N, int E,
                                                      int K, float alpha, float* __restrict__ aux) {
  float a = 0.0f;
  for (int e = threadIdx.x; e < E; e += 64) a += (float)counts[e] * prob_sum[e];
  a = wave_sum(a);
  if (threadIdx.x == 0) aux[0] = alpha * (float)E * a / ((float)N * (float)K * (float)N);
}

// One workgroup of 1024 threads.  Thread (e, g) owns expert e and the chunk
// range of group g; partial sums are scanned over groups, then over experts.
// n_shared = 1: counts[E] = N and offsets[E+1] = offsets[E] + N rounded up to
// align, the shared expert's segment of every token.
__global__ __launch_bounds__(1024) void route_scan_kernel(int32_t* __restrict__ hist, int nchunks,
                                                          int E, int align,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets, int N, int n_shared) {
  __shared__ int s_part[1024];
  __shared__ int s_tot[kMaxE];
  __shared__ int s_off[kMaxE + 1];
  int Ep = 1;
  while (Ep < E) Ep <<= 1;
  const int G = 1024 / Ep;                       // chunk groups
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

namespace {
size_t route_psum_offset(int64_t N, int64_t E, int64_t K) {
  const int64_t nchunks = N > 0 ? (N + kChunk - 1) / kChunk : 1;
  size_t b = (size_t)nchunks * E * 4;   // hist / bases
  b = (b + 255) & ~(size_t)255;
  b += (size_t)N * K * 4;               // in-chunk ranks
  return (b + 255) & ~(size_t)255;
}
}  // namespace

size_t route_workspace_bytes(int64_t N, int64_t E, int64_t K) {
  const int64_t nchunks = N > 0 ? (N + kChunk - 1) / kChunk : 1;
  // then per-chunk probability sums [chunks][E] and P [E] for the aux loss
  return route_psum_offset(N, E, K) + (((size_t)nchunks * E * 4 + 255) & ~(size_t)255) +
         (((size_t)E * 4 + 255) & ~(size_t)255);
}

hipError_t launch_aux_loss(void* ws, int64_t N, int64_t E, int64_t K, const int32_t* counts, float alpha,
                           float* aux, hipStream_t s) {
  if (N == 0) return hipSuccess;
  const int64_t nchunks = (N + kChunk - 1) / kChunk;
  float* psum = (float*)((char*)ws + route_psum_offset(N, E, K));
  float* prob_sum = psum + (((size_t)nchunks * E * 4 + 255) & ~(size_t)255) / 4;
  aux_psum_kernel<<<(unsigned)E, 64, 0, s>>>(psum, nchunks, (int)E, prob_sum);
  aux_loss_kernel<<<1, 64, 0, s>>>(prob_sum, counts, N, (int)E, (int)K, alpha, aux);
  return hipGetLastError();
}

hipError_t launch_route(const float* logits, const uint8_t* drop, int64_t N, int64_t E, int64_t K,
                        int renorm, int align, int64_t rows_cap, int32_t* topk_idx, float* topk_prob,
                        int32_t* counts, int32_t* offsets, int32_t* dst_rows, int32_t* row_route,
                        void* ws, hipStream_t s, int n_group, int topk_group, bool aux_inputs, int n_shared,
                        int32_t* status) {
  const int64_t nchunks = (N + kChunk - 1) / kChunk;
  const int64_t nalloc = nchunks > 0 ? nchunks : 1;
  int32_t* hist = (int32_t*)ws;
  size_t hb = ((size_t)nalloc * E * 4 + 255) & ~(size_t)255;
  int32_t* rank = (int32_t*)((char*)ws + hb);
  float* psum = aux_inputs ? (float*)((char*)ws + route_psum_offset(N, E, K)) : nullptr;
  const int ng = n_group > 1 ? n_group : 0;
  const size_t lds = (ng || psum) ? (size_t)kChunk * E * 4 : 0;
  int npl = 1;
  while (npl * kWave < E) npl <<= 1;   // E <= kMaxE is checked by the caller
  // no tokens: one workgroup still marks every row unused
  const unsigned grid = nchunks > 0 ? (unsigned)nchunks : 1u;
  const int Nk = nchunks > 0 ? (int)N : 0;
  const size_t lds_k = nchunks > 0 ? lds : 0;
  auto go = [&](auto kern) {
    kern<<<dim3(grid), dim3(kTopkThreads), lds_k, s>>>(logits, drop, Nk, (int)E, (int)K, renorm, topk_idx,
                                                       topk_prob, row_route, rows_cap, hist, rank,
                                                       nchunks > 0 ? ng : 0, nchunks > 0 ? topk_group : 0,
                                                       nchunks > 0 ? psum : nullptr, status);
  };
  switch (npl) {
    case 1: go(route_topk_kernel<1>); break;
    case 2: go(route_topk_kernel<2>); break;
    case 4: go(route_topk_kernel<4>); break;
    case 8: go(route_topk_kernel<8>); break;
    default: go(route_topk_kernel<16>); break;
  }
  route_scan_kernel<<<dim3(1), dim3(1024), 0, s>>>(hist, (int)nchunks, (int)E, align, counts,
                                                   offsets, (int)N, n_shared);
  const int64_t NK = N * K;
  if (NK > 0) {
    route_scatter_kernel<<<dim3((unsigned)((NK + 255) / 256)), dim3(256), 0, s>>>(
        topk_idx, drop, hist, rank, NK, (int)K, (int)E, dst_rows, row_route);
  }
  return hipGetLastError();
}

__global__ void status_clear_kernel(int32_t* status) { *status = 0; }

hipError_t launch_status_clear(int32_t* status, hipStream_t s) {
  status_clear_kernel<<<1, 1, 0, s>>>(status);
  return hipGetLastError();
}

}  // namespace moe
