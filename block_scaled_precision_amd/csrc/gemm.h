// Arguments of the grouped FC1 / FC2 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace moe_mx {

struct FcArgs {
  // M-tiles: routed mode reads `tiles[0 .. *num_tiles)`, grid sized for max_tiles;
  // dense mode (dense_rows > 0) covers rows [0, dense_rows) of a single expert.
  const Tile* tiles;
  const int32_t* num_tiles;
  int max_tiles;
  int dense_rows;
  // routed rows: permuted position p -> assignment a = t*k + j
  const int32_t* sorted_assign;
  int k;
  uint32_t kdiv;       // k > 1: ceil(2^32 / k), so that the token of assignment a is
                       // umulhi(a, kdiv), exact while a*k < 2^32
  const float* topk_w;  // FC2 routed: weight of assignment a
  const float* sorted_w;  // routed: weight of permuted row p (= topk_w[sorted_assign[p]])
  float dense_weight;   // FC2 dense: weight of every row
  // A operand: FC1 -> x rows (bf16 [T, K] or E4M3 codes [T, K] + scales [T, K/32]),
  //            FC2 -> h rows in permuted order (bf16 [P, K] or codes + scales)
  const void* a;
  const uint8_t* a_scale;
  // B operand: weights [experts, N_w, K*bits/8] + scales [experts, N_w, K/32]
  const uint8_t* w;
  const uint8_t* w_scale;
  int64_t w_estride;   // bytes per expert
  int64_t ws_estride;  // scale bytes per expert
  int act_fn;          // FC1: gated activation (moe_act_fn_t; 0 = SiLU)
  int K;               // contraction length (H for FC1, I for FC2)
  int N;               // FC1: I (h columns); FC2: H
  int nchunks;         // column chunks of N per M-tile
  // outputs
  void* out;           // FC1: h (bf16 [P, I] or E4M3 codes [P, I])
  uint8_t* out_scale;  // FC1 MX: h scales [P, I/32]
  uint16_t* obuf;      // FC2: bf16 rows [A, N] (routed: row = assignment a, holding
                       // w(a) * o; dense: row = token, holding dense_weight * o),
                       // the product taken in fp32 and rounded once (RNE)
  // dense FC2 on the small-M kernel only: K split into ksplit equal ranges
  // (ksplit > 1), each item writing its unscaled fp32 sum to part
  // [ksplit, dense_rows, N] instead of obuf; 0 or 1 = no split
  int ksplit;
  float* part;
  // few-token FC1 on the small-M kernel (launch_fc_small_routed): every
  // workgroup routes the batch itself from the router logits [T, E] (local
  // experts [off, off + L)) instead of reading tiles, num_tiles and
  // sorted_assign, and workgroup 0 writes the routing out as the routing and
  // permutation kernels would: ids_out / w_out [T, k], offsets_out [L + 1],
  // sorted_out / sorted_w_out (the permuted assignments and their weights),
  // tiles_out and ntiles_out (one tile per active local expert)
  const float* logits;
  int T, E, off, L;
  int32_t* ids_out;
  float* w_out;
  int32_t* offsets_out;
  int32_t* sorted_out;
  float* sorted_w_out;
  Tile* tiles_out;
  int32_t* ntiles_out;
};

// Columns of N covered by one wave of the stream kernels.
constexpr int kStreamColsFc1 = 32;
constexpr int kStreamColsFc2 = 64;
constexpr int kStreamRows = 16;

hipError_t launch_fc_stream(const FcArgs& p, bool fc1, bool mx_act, int wfmt, hipStream_t st);

// Tiled variant (MXFP8 activations): M-tiles of up to `rows` rows (kTiledRows,
// or kTiledRowsLow when experts see fewer rows: less LDS for activations,
// room for wider N-blocks), N-blocks of tiled_weight_rows(rows) weight rows,
// i.e. half as many h columns (FC1: nchunks = I / (that / 2)) or that many
// output columns (FC2: nchunks = H / that); `grid` persistent workgroups
// (rounded down to a multiple of 8, at least 8).  Requires K to be a multiple
// of kTiledKMultiple (scales travel in groups of 4 128-K stages).
constexpr int kTiledRows = 192;
constexpr int kTiledRowsLow = 128;
constexpr int kTiledKMultiple = 512;
// weight rows per N-block of the tiled kernel for M-tiles of `rows` rows
constexpr int tiled_weight_rows(int rows) { return rows == kTiledRowsLow ? 256 : 128; }
// N-blocks of the small-M kernel: 64 h columns (FC1) or 128 output columns (FC2)
constexpr int kSmallColsFc1 = 64;
constexpr int kSmallColsFc2 = 128;
hipError_t launch_fc_tiled(const FcArgs& p, bool fc1, int wfmt, int rows, int grid, hipStream_t st);

// Wide variant (MXFP8 activations x E2M1 weights): M-tiles of up to kTiledRows
// rows, N-blocks of kWideCols weight rows, i.e. 128 h columns (FC1: nchunks =
// I / 128) or 256 output columns (FC2: nchunks = H / 256); `grid` persistent
// workgroups (rounded down to a multiple of 8, at least 8).  Requires
// K % 128 == 0 and K >= 256.
constexpr int kWideCols = 256;
hipError_t launch_fc_wide(const FcArgs& p, bool fc1, int grid, hipStream_t st);

// Small-M variant for bf16 activations and E2M1 weights: M-tiles of up to
// kStreamRows rows (the same tile list as the stream kernels), N-blocks of 64
// h columns (FC1) or 128 output columns (FC2); `grid` persistent workgroups.
// Requires K % kSmallK == 0.
constexpr int kSmallK = 256;
hipError_t launch_fc_small(const FcArgs& p, bool fc1, int grid, hipStream_t st);
// FC1 of the small-M kernel with the routing of a batch of at most
// kSmallRoutedTokens tokens and kSmallRoutedAssign assignments in its prologue
// (p.logits and the routing outputs set; E <= kMaxExperts); the tile height is
// kStreamRows, one tile per active local expert.
constexpr int kSmallRoutedTokens = 16;
constexpr int kSmallRoutedAssign = 128;
hipError_t launch_fc_small_routed(const FcArgs& p, int grid, hipStream_t st);
// y = bf16_RNE(alpha * sum over s of part[s]) for the ksplit partial sums of a
// split dense GEMM, summed in ascending s; n4 = rows * N / 4 (N % 4 == 0)
hipError_t launch_splitk_reduce(const float* part, int ksplit, int64_t n4, float alpha, uint16_t* y,
                                hipStream_t st);

// Mid-M variant for bf16 activations and E2M1 weights when experts see many
// rows: M-tiles of up to `rows` rows (kMidRows or kMidRowsHigh), N-blocks of
// kWideCols weight rows, i.e. 128 h columns (FC1: nchunks = I / 128) or 256
// output columns (FC2: nchunks = H / 256); `grid` persistent workgroups
// (rounded down to a multiple of 8, at least 8).  Requires K % kMidK == 0
// and, for the FC1 gather, A*k < 2^32.
constexpr int kMidRows = 64;
constexpr int kMidRowsHigh = 128;
constexpr int kMidK = 512;
hipError_t launch_fc_mid(const FcArgs& p, bool fc1, int rows, int grid, hipStream_t st);

}  // namespace moe_mx
