// Host-side declarations shared by the translation units of libmoe_mx.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_mx.h"

namespace moe_mx {

// One M-tile of the grouped GEMMs: local expert, first permuted row, row count.
struct Tile {
  int32_t expert;
  int32_t p0;
  int32_t rows;
  int32_t pad;
};

constexpr int kTokensPerRouteBlock = 64;  // tokens per block in the permutation kernels
constexpr int kMaxExperts = 1024;         // limit of the wave-level top-k / scan design

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Checks that the current device is gfx950 (cached per device).
moe_status_t check_arch();

// Launch helpers (all asynchronous on `stream`; return hipGetLastError()).
hipError_t launch_quantize(const void* src, moe_src_t src_dtype, int64_t rows, int64_t cols,
                           int64_t src_ld, mx_elem_t fmt, uint8_t* codes, uint8_t* scales,
                           hipStream_t stream);

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                       hipStream_t stream);

// Permutation of the T*k assignments over local experts [off, off+L):
// per-block histograms `hist` [nblk, L] (turned into write bases in place),
// ranks [T*k], counts-derived offsets [L+1], sorted_assign, if sorted_w is
// non-null the routing weights w in the same order, and, if tiles is non-null,
// the GEMM tile list for M-tiles of `bm` rows with its count.
hipError_t launch_permute(const int32_t* ids, const float* w, int T, int k, int off, int L, int32_t* hist,
                          int32_t* rank, int32_t* offsets, int32_t* sorted_assign, float* sorted_w, Tile* tiles,
                          int32_t* num_tiles, int bm, hipStream_t stream);

// Batches of at most 64 tokens with T*k at most this many assignments take a
// one-workgroup permutation (same results; hist and rank are not used).
constexpr int kSmallRouteAssign = 4096;

// Batches of at most kSmallFusedRouteTokens tokens (k <= 64) route and permute
// in that one workgroup: top-k of router logits [T, E] into ids / w [T, k],
// then the permutation as launch_permute does it.
constexpr int kSmallFusedRouteTokens = 16;
constexpr int kSmallFusedRouteAssign = kSmallFusedRouteTokens * 64;
hipError_t launch_route_permute_small(const float* logits, int T, int E, int k, int32_t* ids, float* w, int off,
                                      int L, int32_t* offsets, int32_t* sorted_assign, float* sorted_w, Tile* tiles,
                                      int32_t* num_tiles, int bm, hipStream_t stream);

}  // namespace moe_mx
