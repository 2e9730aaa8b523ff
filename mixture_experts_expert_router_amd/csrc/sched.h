// Row scheduler shared by the persistent grouped GEMMs whose rows are expert
// segments (the forward GEMMs and the backward dgrad): a one-workgroup
// planner, per-XCD queues and the item decode (KOSMOS section 3.1:
// persistent workgroups claiming tiles from device queues).
//
// An item is (expert, row block, n-tile).  Experts with at least kBigRows
// rows take 256-row blocks, the others 128-row blocks.  The planner lists the
// experts with rows, interleaving the two classes in proportion to their
// work, and writes the item prefix sums; nothing visits the host.  The item
// sequence is cut into chunks of kChunk items; chunk c belongs to the queue
// of XCD c % kXcds, so the CUs of one XCD (each XCD has its own L2) work on
// neighbouring items at the same time.  Inside an expert, items run in
// super-blocks of kSbM row blocks x kSbN n-tiles, row block fastest.  A
// workgroup drains its own XCD's queue, then takes items from the others.
#pragma once

#include "common.h"
#include "launch.h"

namespace moe {
namespace sched {
namespace {

constexpr int kBigRows = 256;       // experts with at least this many rows use 256-row blocks
constexpr int kBigBM = 256, kSmallBM = 128;
constexpr int kTinyRows = 64;       // small experts this short may use 64-row tiles
constexpr int kTiny32Rows = 32;     // and this short 32-row tiles
constexpr int kXcds = 8;            // XCDs of the chip; queue q holds chunks q, q + 8, ...
constexpr int kChunk = 32;          // items per chunk (the CUs of one XCD)
constexpr int kSbM = 4, kSbN = 8;   // super-block: row blocks x n-tiles

constexpr int kHeadStride = 32;     // ints between queue heads: one 128-byte line each
static_assert(kXcds * kHeadStride == kGemmHeadInts, "head block of the workspace");

// plan layout (int32): [0] total items, [1] number of listed experts L,
// [2 .. 2+L) expert ids in processing order, [2+E .. 2+E+L] item prefix sums
// (entry L = total).  The queue heads are kXcds counters kHeadStride apart.

// A claimed queue item, decoded: rows [m_start, min(m_start + BM, m1)) of
// expert e, output columns [n0, n0 + NCOL), tile class by the expert's rows
// (a large expert's last row block takes the 128-row class when it holds at
// most 128 rows, the 64-row one at most 64, the 32-row one at most 32).
struct Item {
  int e, m_start, m1, n0;
  bool big, valid;
  bool tiny;   // the expert has at most kTinyRows rows (one row block either way)
  bool tiny32; // at most kTiny32Rows rows
};

__device__ __host__ __forceinline__ bool is_big(int rows) { return rows >= kBigRows; }

// item w of an expert with nmb row blocks and n_tiles n-tiles: n-groups of
// kSbN tiles, in each m-groups of kSbM row blocks, row block fastest (the
// last group of each kind may be short); a bijection onto the (mb, n_t) grid
__device__ __forceinline__ void superblock_decode(int w, int nmb, int n_tiles, int& mb, int& n_t) {
  const int gn = w / (kSbN * nmb);
  const int w1 = w - gn * kSbN * nmb;
  const int nb = min(kSbN, n_tiles - gn * kSbN);
  const int gm = w1 / (kSbM * nb);
  const int w2 = w1 - gm * kSbM * nb;
  const int mbk = min(kSbM, nmb - gm * kSbM);
  mb = gm * kSbM + w2 % mbk;
  n_t = gn * kSbN + w2 / mbk;
}

// XCD this workgroup runs on (hardware register XCC_ID).  Only locality
// depends on it: any value in range gives the same results.
__device__ __forceinline__ int xcd_id() {
  return (int)(__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & (kXcds - 1));
}

// global position of the k-th item of queue q
__device__ __forceinline__ int queue_item(int q, int k) { return (kXcds * (k / kChunk) + q) * kChunk + k % kChunk; }

// Claim the next item and decode it (every thread gets the same result).
// Queue q's items have increasing positions and end at the first one past
// the total, so a failed claim means the queue is exhausted.  li is the
// workgroup's position in the expert list, walked forward for its own queue's
// increasing items and searched for items taken from other queues.
// Claim the next position of the item sequence [0, total) for the workgroup
// (thread 0 takes it, every lane returns it); -1 when all queues are empty.
__device__ __forceinline__ int claim_global(int32_t* head, int total, int* s_item, int xcd) {
  if (threadIdx.x == 0) {
    int g = -1;
    for (int t = 0; t < kXcds; ++t) {
      const int q = (xcd + t) & (kXcds - 1);
      const int gi = queue_item(q, atomicAdd(head + q * kHeadStride, 1));
      if (gi < total) {
        g = gi;
        break;
      }
    }
    *s_item = g;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*s_item);   // same for every lane
}

__device__ __forceinline__ Item claim_rows(const int32_t* plan, const int32_t* offsets, int32_t* head, int E,
                                          int n_tiles, int ncol, int* s_item, int& li, int xcd) {
  const int item = claim_global(head, plan[0], s_item, xcd);
  Item it{};
  if (item < 0) return it;
  const int L = plan[1];
  const int32_t* order = plan + 2;
  const int32_t* pref = plan + 2 + E;
  if (pref[li] > item) {   // an earlier item (taken from another queue): binary search
    int lo = 0, hi = L - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pref[mid] <= item) lo = mid;
      else hi = mid - 1;
    }
    li = lo;
  }
  while (li + 1 < L && pref[li + 1] <= item) ++li;
  it.e = order[li];
  const int m0 = offsets[it.e];
  it.m1 = offsets[it.e + 1];
  it.big = is_big(it.m1 - m0);
  it.tiny = it.m1 - m0 <= kTinyRows;
  it.tiny32 = it.m1 - m0 <= kTiny32Rows;
  const int bm = it.big ? kBigBM : kSmallBM;
  const int nmb = (it.m1 - m0 + bm - 1) / bm;
  int mb, n_t;
  superblock_decode(item - pref[li], nmb, n_tiles, mb, n_t);
  it.m_start = m0 + mb * bm;
  it.n0 = n_t * ncol;
  it.valid = true;
  // the last row block of a large expert, when at most kSmallBM rows are
  // left, runs as a 128-row tile, or a 64- or 32-row one where those classes
  // exist and that few rows are left (every tile class accumulates the same
  // contraction steps in the same order, so the result is the same)
  if (it.big && it.m1 - it.m_start <= kSmallBM) {
    it.big = false;
    it.tiny = it.m1 - it.m_start <= kTinyRows;
    it.tiny32 = it.m1 - it.m_start <= kTiny32Rows;
  }
  return it;
}

// Planner: one workgroup of 1024 threads (E <= 1024).  Each expert with rows
// gets ceil(rows / BM) * n_tiles items, BM by its tile class.  The experts of
// each class keep ascending id; the two classes are merged by the midpoint of
// each expert's items within its class, so both progress at the same rate.
// The planner's body for a workgroup of THREADS threads (E <= THREADS).
// LDS: s_w0, s_w1, s_pref [THREADS / 64] and s_tot [2] ints, s_key [THREADS]
// floats, s_items, s_ids [THREADS] ints.
template <int THREADS>
__device__ __forceinline__ void plan_rows_body(const int32_t* __restrict__ offsets, int E, int n_tiles,
                                               int32_t* __restrict__ plan, int32_t* __restrict__ head, int* s_w0,
                                               int* s_w1, int* s_tot, float* s_key, int* s_items, int* s_ids,
                                               int* s_pref) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  int items = 0, big = 0;
  if (t < E) {
    const int m = offsets[t + 1] - offsets[t];
    big = is_big(m);
    const int bm = big ? kBigBM : kSmallBM;
    items = m > 0 ? ((m + bm - 1) / bm) * n_tiles : 0;
  }
  int i0 = big ? 0 : items, i1 = big ? items : 0;   // per-class inclusive scans
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int a = __shfl_up(i0, o, 64), b = __shfl_up(i1, o, 64);
    if (lane >= o) { i0 += a; i1 += b; }
  }
  if (lane == 63) { s_w0[wv] = i0; s_w1[wv] = i1; }
  __syncthreads();
  if (t == 0) {
    int r0 = 0, r1 = 0;
    for (int w = 0; w < THREADS / 64; ++w) {
      const int a = s_w0[w], b = s_w1[w];
      s_w0[w] = r0; s_w1[w] = r1;
      r0 += a; r1 += b;
    }
    s_tot[0] = r0; s_tot[1] = r1;
  }
  __syncthreads();
  const int pre = big ? (i1 - items + s_w1[wv]) : (i0 - items + s_w0[wv]);
  const int tot = s_tot[big];
  s_key[t] = (items > 0) ? ((float)pre + 0.5f * (float)items) / (float)tot : 2.0f;
  __syncthreads();
  if (items > 0) {
    const float k = s_key[t];
    int rank = 0;
    for (int f = 0; f < E; ++f) {
      const float kf = s_key[f];
      rank += (kf < k) || (kf == k && f < t);
    }
    s_items[rank] = items;
    s_ids[rank] = t;
  }
  const int L = __syncthreads_count(items > 0);
  // exclusive scan of the items in rank order
  const int v = t < L ? s_items[t] : 0;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int a = __shfl_up(inc, o, 64);
    if (lane >= o) inc += a;
  }
  if (lane == 63) s_pref[wv] = inc;
  __syncthreads();
  if (t == 0) {
    int r = 0;
    for (int w = 0; w < THREADS / 64; ++w) { const int a = s_pref[w]; s_pref[w] = r; r += a; }
    plan[0] = r;
    plan[1] = L;
    plan[2 + E + L] = r;
  }
  if (t < kXcds) head[t * kHeadStride] = 0;
  __syncthreads();
  if (t < L) {
    plan[2 + t] = s_ids[t];
    plan[2 + E + t] = inc - v + s_pref[wv];
  }
}

__global__ __launch_bounds__(1024) void plan_rows_kernel(const int32_t* __restrict__ offsets, int E, int n_tiles,
                                                        int32_t* __restrict__ plan, int32_t* __restrict__ head) {
  __shared__ int s_w0[16], s_w1[16], s_tot[2];
  __shared__ float s_key[1024];
  __shared__ int s_items[1024], s_ids[1024], s_pref[16];
  plan_rows_body<1024>(offsets, E, n_tiles, plan, head, s_w0, s_w1, s_tot, s_key, s_items, s_ids, s_pref);
}

}  // namespace
}  // namespace sched
}  // namespace moe
