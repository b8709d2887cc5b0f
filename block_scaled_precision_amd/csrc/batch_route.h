// Routing of a batch of a few tokens by one workgroup, into LDS: the top-k of
// each token (one wave per token, topk_device.h), the token mask of every
// local expert, and the active local experts in ascending order with the first
// permuted row of each (mxfp6-sm120 page, "Execution model": the small-batch
// path routes without allocations; TokenSpeed SiTU page, "Supported
// contract": softmax over the selected logits, experts renumbered into the
// local range [off, off + L)).  The permuted order is the permutation
// kernels' order: by local expert, then by assignment id, so an expert's rows
// are its tokens in ascending order.  Every workgroup that runs this computes
// the same routing, bit for bit.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "topk_device.h"

namespace moe_mx {

constexpr int kBatchRouteMaxThreads = 1024;

// LDS routing state for at most MAXA assignments of at most 32 tokens (the
// token masks are 32-bit words).
template <int MAXA>
struct BatchRoute {
  int32_t ids[MAXA];
  float wts[MAXA];
  uint32_t mask[kMaxExperts];         // bit t: token t is routed to the local expert
  int32_t act_e[kMaxExperts];         // active local experts, ascending
  int32_t act_off[kMaxExperts + 1];   // first permuted row of each; act_off[nact] = total
  int32_t part[kBatchRouteMaxThreads / 64];  // scan totals of the waves
  int32_t nact;
};

// Block-wide exclusive scan of (active, count) over the L local experts; fills
// act_e / act_off / nact and, if `start` is given, the first permuted row of
// every local expert (start[L] = the total).  Each thread owns ceil(L / NT)
// consecutive experts; the threads' sums are scanned within each wave by
// shuffles and across the waves through their totals.  Ends with a barrier.
template <int NT, int MAXA>
__device__ void scan_experts(BatchRoute<MAXA>& r, int L, int32_t* start) {
  static_assert(NT % 64 == 0 && NT <= kBatchRouteMaxThreads && MAXA < 65536, "scan partials");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per = (L + NT - 1) / NT;
  const int e0 = tid * per;
  int na = 0, nc = 0;
  for (int e = e0; e < min(e0 + per, L); ++e) {
    const int c = __popc(r.mask[e]);
    na += c > 0;
    nc += c;
  }
  // (active experts << 16) | assignments: at most 1024 and MAXA, no carry
  int v = (na << 16) | nc;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d);
    if (lane >= d) v += u;
  }
  if (lane == 63) r.part[wv] = v;
  __syncthreads();
  for (int w = 0; w < wv; ++w) v += r.part[w];
  int pa = (v >> 16) - na, pc = (v & 0xffff) - nc;
  for (int e = e0; e < min(e0 + per, L); ++e) {
    const int c = __popc(r.mask[e]);
    if (start) start[e] = pc;
    if (c > 0) {
      r.act_e[pa] = e;
      r.act_off[pa] = pc;
      ++pa;
      pc += c;
    }
  }
  if (tid == NT - 1) {
    r.nact = v >> 16;
    r.act_off[r.nact] = v & 0xffff;
    if (start) start[L] = v & 0xffff;
  }
  __syncthreads();
}

// Top-k of each of the T tokens from router logits [T, E], one wave per
// token: ids [T, k] and softmax weights over the chosen logits (LDS arrays).
// No barrier.
template <int NS, int NT>
__device__ void topk_batch(const float* logits, int T, int E, int k, int32_t* ids, float* wts) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int t = wv; t < T; t += NT / 64) {
    TopkToken<NS> tk(logits + (int64_t)t * E, E, lane);
    int my_e;
    float my_v;
    tk.select(E, 0, k, lane, my_e, my_v);
    if (lane < k) {
      ids[t * k + lane] = my_e;
      wts[t * k + lane] = expf(my_v - tk.top) * (1.0f / tk.sum);
    }
  }
}

// Routing of the batch (T tokens, T * k <= MAXA, T <= 32) from router logits
// [T, E], or from a precomputed top-k ids_in / w_in [T, k] when logits is
// null; `start` as in scan_experts.  Ends with a barrier.
template <int NS, int NT, int MAXA>
__device__ void route_batch(const float* logits, const int32_t* ids_in, const float* w_in, int T, int E, int k,
                            int off, int L, BatchRoute<MAXA>& r, int32_t* start) {
  const int A = T * k;
  if (!logits) {
    for (int i = threadIdx.x; i < A; i += NT) {
      r.ids[i] = ids_in[i];
      r.wts[i] = w_in[i];
    }
  } else {
    topk_batch<NS, NT>(logits, T, E, k, r.ids, r.wts);
  }
  for (int e = threadIdx.x; e < L; e += NT) r.mask[e] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < A; i += NT) {
    const int e = r.ids[i] - off;
    if (e >= 0 && e < L) atomicOr(&r.mask[e], 1u << (i / k));
  }
  __syncthreads();
  scan_experts<NT>(r, L, start);
}

}  // namespace moe_mx
