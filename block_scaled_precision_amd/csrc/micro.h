// Arguments of the small-batch path (micro.hip): bf16 activations, E2M1
// weights, at most kMicroMaxTokens tokens and kMicroMaxAssign assignments.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe_mx {

constexpr int kMicroMaxTokens = 8;
constexpr int kMicroMaxAssign = 64;
constexpr int kMicroMaxL = kMicroMaxAssign;  // active experts are at most the assignments
// H must be a multiple of this (k_micro_fc1 walks K in 512-value steps)
constexpr int kMicroHMultiple = 512;

// The routing of a batch as k_micro_fc1 publishes it for k_micro_fc2 (in the
// workspace): the active local experts in ascending order, each with its
// token mask, the first row of its tokens in h (rows of one expert are its
// tokens in ascending order) and the routing weight of each token (0 for
// tokens it does not see).
struct MicroList {
  int32_t nact;
  int32_t expert[kMicroMaxL];
  uint32_t mask[kMicroMaxL];
  int32_t off[kMicroMaxL];
  float w[kMicroMaxL * kMicroMaxTokens];
};

struct MicroArgs {
  // routing source: router logits [T, E], or a precomputed top-k [T, k]
  const float* logits;
  const int32_t* ids_in;
  const float* w_in;
  int T, E, k, off, L;  // local experts [off, off + L)
  int32_t* ids_out;     // [T, k] routing as used (optional)
  float* w_out;
  const void* x;        // [T, H] bf16
  int H, I, Is;         // hidden, expert and shared-expert intermediate sizes
  int act_fn;           // gated activation (moe_act_fn_t)
  const uint8_t* w1;    // [L, 2I, H/2] E2M1 + [L, 2I, H/32] scales
  const uint8_t* s1;
  int64_t w1_estride, s1_estride;
  const uint8_t* ws1;   // shared expert [2Is, H/2] + scales (Is > 0)
  const uint8_t* ss1;
  uint16_t* h;          // [T*k, I] bf16: FC2 input of the routed rows
  uint16_t* hs;         // [T, Is] bf16: FC2 input of the shared expert
  MicroList* list;
  const uint8_t* w2;    // [L, H, I/2] + [L, H, I/32]
  const uint8_t* s2;
  int64_t w2_estride, s2_estride;
  const uint8_t* ws2;   // [H, Is/2] + [H, Is/32]
  const uint8_t* ss2;
  float shared_weight;
  uint16_t* y;          // [T, H] bf16 out
};

// Dynamic LDS of k_micro_fc1 (the batch's x rows) for T tokens of H values.
size_t micro_fc1_lds(int T, int H);
// Static LDS of k_micro_fc1 besides that (routing state), an upper bound.
constexpr size_t kMicroFc1StaticLds = 24 * 1024;

// Both kernels on `st`; fc2_mark (optional) is recorded between them.
hipError_t launch_micro(const MicroArgs& p, int cus, hipStream_t st, hipEvent_t fc2_mark);

}  // namespace moe_mx
