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
#include "route_dev.h"

namespace moe {

using route::kChunk;                      // tokens per workgroup in route_topk (one per wave)
constexpr int kTopkThreads = kChunk * 64;
using route::kMaxE;

// A workgroup per chunk, a wave per token.
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
  // row_route = -1 everywhere first (the scatter overwrites the used rows)
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows_cap;
       i += (int64_t)gridDim.x * blockDim.x)
    row_route[i] = -1;
  route::topk_chunk<NPL, kTopkThreads>(blockIdx.x, logits, drop, N, E, K, renorm, topk_idx, topk_prob, hist, rank,
                                       n_group, topk_group, psum, status, s_sel, s_hist, s_row);
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

__global__ __launch_bounds__(1024) void route_scan_kernel(int32_t* __restrict__ hist, int nchunks,
                                                          int E, int align,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets, int N, int n_shared) {
  __shared__ int s_part[1024];
  __shared__ int s_tot[kMaxE];
  __shared__ int s_off[kMaxE + 1];
  __shared__ int s_wsum[16];
  route::scan_hist<1024>(hist, nchunks, E, align, counts, offsets, N, n_shared, s_part, s_tot, s_off, s_wsum);
}

__global__ __launch_bounds__(256) void route_scatter_kernel(
    const int32_t* __restrict__ topk_idx, const uint8_t* __restrict__ drop,
    const int32_t* __restrict__ base, const int32_t* __restrict__ rank, int64_t NK, int K, int E,
    int32_t* __restrict__ dst_rows, int32_t* __restrict__ row_route) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= NK) return;
  route::scatter_route(r, topk_idx, drop, base, rank, K, E, dst_rows, row_route);
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
  int32_t* hist = (int32_t*)ws;
  int32_t* rank = (int32_t*)((char*)ws + route::hist_bytes(N, E));
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
