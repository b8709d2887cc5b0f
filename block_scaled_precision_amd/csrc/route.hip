// Routing: softmax/top-k per token and the permutation of assignments by expert.
//
// top-k (mxfp6-sm120 page, table of paths: the routed path starts with
// routing; fusedtok page: selection ties resolve to the earliest index):
// one wave per token.  Each lane keeps E/64 logits; k rounds of a wave-wide
// arg-max over 64-bit keys (order-preserving fp32 bits, then inverted id) pick
// the experts in slot order, so equal logits go to the lower id.  The weights
// are a softmax over the chosen logits in fp32 (the full softmax renormalised
// over the chosen experts).
//
// Permutation (mxfp6-sm120 page, "Execution model": indirect routing) is a
// deterministic counting sort with no global atomics on positions:
//   1. per block of 64 tokens, an LDS bit mask per expert marks which lanes
//      (tokens) chose it; popcount gives the block histogram, and the popcount
//      below a lane gives the rank of its assignment inside the block;
//   2. one block scans the histograms over blocks (each block's base within
//      its expert) and over experts (expert offsets), and emits the GEMM tile
//      list;
//   3. every assignment is written to expert offset + base + rank.
// The order inside an expert segment is therefore ascending token.  Batches of
// at most 64 tokens (one token block) run the three steps in one workgroup.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "topk_device.h"

namespace moe_mx {

// 4 waves per block, one token per wave.  Lane j keeps the id and logit of
// slot j (k <= E <= 1024, so slots past 63 are kept by lane j % 64 in round
// j / 64); lane j writes slot j's id and, once the sum is complete, weight.
template <int NS>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ wts) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;
  TopkToken<NS> tk(logits + (int64_t)t * E, E, lane);
  for (int j0 = 0; j0 < k; j0 += 64) {
    int my_e;
    float my_v;
    const int jn = min(k - j0, 64);
    tk.select(E, j0, jn, lane, my_e, my_v);
    if (lane < jn) ids[(int64_t)t * k + j0 + lane] = my_e;
    if (k <= 64) {
      // one batch: the sum is complete, the slot's logit is still in a register
      if (lane < jn) wts[(int64_t)t * k + lane] = expf(my_v - tk.top) * (1.0f / tk.sum);
      return;
    }
    // the weights need the full sum: park the logits, normalised below
    if (lane < jn) wts[(int64_t)t * k + j0 + lane] = my_v;
  }
  const float inv = 1.0f / tk.sum;
  for (int j = lane; j < k; j += 64) wts[(int64_t)t * k + j] = expf(wts[(int64_t)t * k + j] - tk.top) * inv;
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                       hipStream_t stream) {
  if (T == 0) return hipSuccess;
  // as many key slots per lane as E needs (the selection rounds walk them all)
  const int g = (T + 3) / 4, ns = (E + 63) / 64;
  if (ns <= 1) k_topk<1><<<g, 256, 0, stream>>>(logits, T, E, k, ids, w);
  else if (ns <= 2) k_topk<2><<<g, 256, 0, stream>>>(logits, T, E, k, ids, w);
  else if (ns <= 4) k_topk<4><<<g, 256, 0, stream>>>(logits, T, E, k, ids, w);
  else if (ns <= 6) k_topk<6><<<g, 256, 0, stream>>>(logits, T, E, k, ids, w);
  else if (ns <= 8) k_topk<8><<<g, 256, 0, stream>>>(logits, T, E, k, ids, w);
  else k_topk<16><<<g, 256, 0, stream>>>(logits, T, E, k, ids, w);
  return hipGetLastError();
}

// Block = one wave of 64 tokens.  mask[e] bit l = token (64*blk + l) chose local expert e.
__global__ __launch_bounds__(64) void k_rank(const int32_t* __restrict__ ids, int T, int k, int off,
                                             int L, int32_t* __restrict__ hist,
                                             int32_t* __restrict__ rank) {
  __shared__ unsigned long long mask[kMaxExperts];
  const int lane = threadIdx.x;
  for (int e = lane; e < L; e += 64) mask[e] = 0ull;
  __syncthreads();
  const int t = blockIdx.x * 64 + lane;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = ids[(int64_t)t * k + j] - off;
      if (e >= 0 && e < L) atomicOr(&mask[e], 1ull << lane);
    }
  }
  __syncthreads();
  for (int e = lane; e < L; e += 64) hist[(int64_t)blockIdx.x * L + e] = __popcll(mask[e]);
  if (t < T) {
    const unsigned long long below = lane ? (~0ull >> (64 - lane)) : 0ull;
    for (int j = 0; j < k; ++j) {
      const int e = ids[(int64_t)t * k + j] - off;
      rank[(int64_t)t * k + j] = (e >= 0 && e < L) ? __popcll(mask[e] & below) : -1;
    }
  }
}

// One block of 1024 threads; thread e owns local expert e.
__global__ __launch_bounds__(1024) void k_scan(int32_t* __restrict__ hist, int nblk, int L,
                                               int32_t* __restrict__ offsets, Tile* __restrict__ tiles,
                                               int32_t* __restrict__ num_tiles, int bm) {
  __shared__ int32_t s_a[kMaxExperts];
  __shared__ int32_t s_b[kMaxExperts];
  const int e = threadIdx.x;
  // exclusive prefix of expert e's counts over the token blocks, 32 blocks
  // per batch: all loads of a batch go out before its stores, so the walk
  // costs one memory latency per 32 blocks instead of one per block
  constexpr int kBatch = 32;
  int32_t count = 0;
  if (e < L) {
    for (int b0 = 0; b0 < nblk; b0 += kBatch) {
      int32_t h[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) h[i] = b0 + i < nblk ? hist[(int64_t)(b0 + i) * L + e] : 0;
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (b0 + i < nblk) hist[(int64_t)(b0 + i) * L + e] = count;
        count += h[i];
      }
    }
  }
  const int32_t ntile = (e < L && bm > 0) ? (count + bm - 1) / bm : 0;
  // inclusive Hillis-Steele scans of count and ntile over the block
  s_a[e] = e < L ? count : 0;
  s_b[e] = ntile;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int32_t a = e >= d ? s_a[e - d] : 0;
    const int32_t b = e >= d ? s_b[e - d] : 0;
    __syncthreads();
    s_a[e] += a;
    s_b[e] += b;
    __syncthreads();
  }
  const int32_t start = s_a[e] - (e < L ? count : 0);
  const int32_t tstart = s_b[e] - ntile;
  if (e < L) {
    // hist keeps the prefix within the expert; the scatter adds offsets[e]
    offsets[e] = start;
    if (e == L - 1) offsets[L] = s_a[e];
    for (int i = 0; i < ntile; ++i) {
      const int32_t r0 = i * bm;
      Tile tl;
      tl.expert = e;
      tl.p0 = start + r0;
      tl.rows = min(bm, count - r0);
      tl.pad = 0;
      tiles[tstart + i] = tl;
    }
  }
  if (e == 0 && bm > 0) *num_tiles = s_b[1023];
}

// sorted_assign[pos] = a and, if requested, sorted_w[pos] = w[a] (the routing
// weight of the assignment, so that consumers of permuted rows read it directly)
__global__ __launch_bounds__(256) void k_scatter(const int32_t* __restrict__ ids, const float* __restrict__ w,
                                                 int T, int k, int off, int L, const int32_t* __restrict__ base,
                                                 const int32_t* __restrict__ offsets, const int32_t* __restrict__ rank,
                                                 int32_t* __restrict__ sorted_assign, float* __restrict__ sorted_w) {
  const int64_t a = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (a >= (int64_t)T * k) return;
  const int e = ids[a] - off;
  if (e < 0 || e >= L) return;
  const int64_t blk = (a / k) / 64;
  const int32_t pos = offsets[e] + base[blk * L + e] + rank[a];
  sorted_assign[pos] = (int32_t)a;
  if (sorted_w) sorted_w[pos] = w[a];
}

// Small batches (T <= 64 tokens, T*k <= kSmallRouteAssign): the three steps
// of the permutation in one workgroup of 16 waves, with the same results: the
// tokens are one token block, so an expert's mask of tokens gives its count
// and, below a token, that token's rank.  With NS > 0 (at most 16 tokens,
// k <= 64) the workgroup also routes: wave t takes the top-k of token t
// straight into LDS (one launch instead of two), writing the ids and weights
// out as k_topk would.
template <int NS>
__global__ __launch_bounds__(1024) void k_permute_small(const float* __restrict__ logits, int E,
                                                        int32_t* __restrict__ ids_out, float* __restrict__ w_out,
                                                        const int32_t* __restrict__ ids, const float* __restrict__ w,
                                                        int T, int k, int off, int L, int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ sorted_assign,
                                                        float* __restrict__ sorted_w, Tile* __restrict__ tiles,
                                                        int32_t* __restrict__ num_tiles, int bm) {
  __shared__ unsigned long long mask[kMaxExperts];
  __shared__ int32_t s_ids[kSmallRouteAssign];
  __shared__ float s_w[NS > 0 ? kSmallFusedRouteAssign : 1];
  __shared__ int32_t s_a[kMaxExperts];
  __shared__ int32_t s_b[kMaxExperts];
  __shared__ int32_t s_start[kMaxExperts];
  const int e = threadIdx.x;  // one thread per local expert in the scan
  const int A = T * k;
  mask[e] = 0ull;
  if constexpr (NS > 0) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    if (wv < T) {
      TopkToken<NS> tk(logits + (int64_t)wv * E, E, lane);
      int my_e;
      float my_v;
      tk.select(E, 0, k, lane, my_e, my_v);
      if (lane < k) {
        const float wt = expf(my_v - tk.top) * (1.0f / tk.sum);
        s_ids[wv * k + lane] = my_e;
        s_w[wv * k + lane] = wt;
        ids_out[wv * k + lane] = my_e;
        w_out[wv * k + lane] = wt;
      }
    }
  } else {
    for (int a = e; a < A; a += 1024) s_ids[a] = ids[a];
  }
  __syncthreads();
  for (int a = e; a < A; a += 1024) {
    const int el = s_ids[a] - off;
    if (el >= 0 && el < L) atomicOr(&mask[el], 1ull << (a / k));
  }
  __syncthreads();
  // counts, inclusive scans of counts and tile counts over the experts,
  // offsets and tiles (as k_scan with one token block): each wave scans its
  // 64 experts across lanes, wave 0 scans the 16 wave totals
  const int32_t count = e < L ? __popcll(mask[e]) : 0;
  const int32_t ntile = (e < L && bm > 0) ? (count + bm - 1) / bm : 0;
  const int lane_e = e & 63, wv_e = e >> 6;
  int32_t inc_a = count, inc_b = ntile;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t a = __shfl_up(inc_a, d), b = __shfl_up(inc_b, d);
    if (lane_e >= d) {
      inc_a += a;
      inc_b += b;
    }
  }
  if (lane_e == 63) {
    s_a[wv_e] = inc_a;
    s_b[wv_e] = inc_b;
  }
  __syncthreads();
  if (wv_e == 0) {
    int32_t ta = lane_e < 16 ? s_a[lane_e] : 0, tb = lane_e < 16 ? s_b[lane_e] : 0;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int32_t a = __shfl_up(ta, d), b = __shfl_up(tb, d);
      if (lane_e >= d) {
        ta += a;
        tb += b;
      }
    }
    if (lane_e < 16) {
      s_a[16 + lane_e] = ta;  // inclusive totals through wave lane_e
      s_b[16 + lane_e] = tb;
    }
  }
  __syncthreads();
  if (wv_e > 0) {
    inc_a += s_a[16 + wv_e - 1];
    inc_b += s_b[16 + wv_e - 1];
  }
  const int32_t start = inc_a - count;
  s_start[e] = start;
  if (e < L) {
    offsets[e] = start;
    if (e == L - 1) offsets[L] = inc_a;
    const int32_t tstart = inc_b - ntile;
    for (int i = 0; i < ntile; ++i) {
      const int32_t r0 = i * bm;
      Tile tl;
      tl.expert = e;
      tl.p0 = start + r0;
      tl.rows = min(bm, count - r0);
      tl.pad = 0;
      tiles[tstart + i] = tl;
    }
  }
  if (e == 0 && bm > 0) *num_tiles = s_b[16 + 15];
  __syncthreads();
  for (int a = e; a < A; a += 1024) {
    const int el = s_ids[a] - off;
    if (el < 0 || el >= L) continue;
    const int t = a / k;
    const unsigned long long below = t ? (~0ull >> (64 - t)) : 0ull;
    const int32_t pos = s_start[el] + __popcll(mask[el] & below);
    sorted_assign[pos] = a;
    if (sorted_w) sorted_w[pos] = NS > 0 ? s_w[a] : w[a];
  }
}

hipError_t launch_route_permute_small(const float* logits, int T, int E, int k, int32_t* ids, float* w, int off,
                                      int L, int32_t* offsets, int32_t* sorted_assign, float* sorted_w, Tile* tiles,
                                      int32_t* num_tiles, int bm, hipStream_t stream) {
  const int ns = (E + 63) / 64;
  const int b = tiles ? bm : 0;
#define MOE_ROUTE_SMALL(N)                                                                                      \
  k_permute_small<N><<<1, 1024, 0, stream>>>(logits, E, ids, w, nullptr, nullptr, T, k, off, L, offsets,     \
                                             sorted_assign, sorted_w, tiles, num_tiles, b)
  if (ns <= 1) MOE_ROUTE_SMALL(1);
  else if (ns <= 2) MOE_ROUTE_SMALL(2);
  else if (ns <= 4) MOE_ROUTE_SMALL(4);
  else if (ns <= 6) MOE_ROUTE_SMALL(6);
  else if (ns <= 8) MOE_ROUTE_SMALL(8);
  else MOE_ROUTE_SMALL(16);
#undef MOE_ROUTE_SMALL
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* ids, const float* w, int T, int k, int off, int L, int32_t* hist,
                          int32_t* rank, int32_t* offsets, int32_t* sorted_assign, float* sorted_w, Tile* tiles,
                          int32_t* num_tiles, int bm, hipStream_t stream) {
  if (T <= 64 && (int64_t)T * k <= kSmallRouteAssign) {
    k_permute_small<0><<<1, 1024, 0, stream>>>(nullptr, 0, nullptr, nullptr, ids, w, T, k, off, L, offsets,
                                               sorted_assign, sorted_w, tiles, num_tiles, tiles ? bm : 0);
    return hipGetLastError();
  }
  const int nblk = (T + 63) / 64;
  if (nblk > 0) k_rank<<<nblk, 64, 0, stream>>>(ids, T, k, off, L, hist, rank);
  k_scan<<<1, 1024, 0, stream>>>(hist, nblk, L, offsets, tiles, num_tiles, tiles ? bm : 0);
  const int64_t A = (int64_t)T * k;
  if (A > 0) k_scatter<<<(A + 255) / 256, 256, 0, stream>>>(ids, w, T, k, off, L, hist, offsets, rank,
                                                            sorted_assign, sorted_w);
  return hipGetLastError();
}

}  // namespace moe_mx
