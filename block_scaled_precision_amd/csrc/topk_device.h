// Wave-level top-k selection of one token's router logits (shared by the
// routing kernel and the small-batch path): order-preserving 64-bit keys
// (fp32 bits, then the inverted expert id, so equal logits go to the lower
// id) and a wave-wide arg-max per slot; the running softmax denominator over
// the chosen logits is kept in every lane (fusedtok page: selection ties
// resolve to the earliest index).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace moe_mx {

__device__ __forceinline__ uint32_t ordered_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// max of v with the value DPP control `ctrl` brings from another lane of its row
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xf, 0xf, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, true);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > v ? o : v;
}

// Maximum over the wave (all 64 lanes active), returned wave-uniform: within
// each row of 16 lanes by DPP (pairs, quads, then rotations by 4 and 8), then
// across the four rows by reading one lane of each.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_u64<0xb1>(v);   // quad_perm 1,0,3,2
  v = dpp_max_u64<0x4e>(v);   // quad_perm 2,3,0,1
  v = dpp_max_u64<0x124>(v);  // row_ror 4
  v = dpp_max_u64<0x128>(v);  // row_ror 8
  uint64_t m = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * r);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * r);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    m = o > m ? o : m;
  }
  return m;
}

// Top-k of one token by one wave; E <= 1024 -> at most 16 logits per lane.
// Every lane sees the winner of each round, so all lanes carry the same
// running softmax denominator.
template <int NS>  // key slots per lane: experts lane, lane + 64, ..., NS*64 >= E
struct TopkToken {
  uint32_t key[NS];
  uint32_t taken = 0;
  float top = 0.f, sum = 0.f;

  __device__ __forceinline__ TopkToken(const float* row, int E, int lane) {
    // every slot loads (past E from the last logit, then dropped), so that the
    // loads are issued together and waited for once
    float v[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) v[i] = row[min(lane + 64 * i, E - 1)];
#pragma unroll
    for (int i = 0; i < NS; ++i) key[i] = lane + 64 * i < E ? ordered_bits(v[i]) : 0u;
  }
  // slots j0 .. j0+jn-1 (jn <= 64): lane jj gets slot j0+jj's expert and logit
  __device__ __forceinline__ void select(int E, int j0, int jn, int lane, int& my_e, float& my_v) {
    my_e = 0;
    my_v = 0.f;
    for (int jj = 0; jj < jn; ++jj) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int e = lane + 64 * i;
        if (e < E && !(taken >> i & 1u)) {
          const uint64_t kk = ((uint64_t)key[i] << 32) | (uint32_t)(kMaxExperts - 1 - e);
          best = kk > best ? kk : best;
        }
      }
      best = wave_max_u64(best);
      const int e = kMaxExperts - 1 - (int)(best & 0xffffffffu);
      const float v = from_ordered((uint32_t)(best >> 32));
      if (j0 + jj == 0) top = v;
      sum += expf(v - top);
      if ((e & 63) == lane) taken |= 1u << (e >> 6);
      if (lane == jj) {
        my_e = e;
        my_v = v;
      }
    }
  }
};

}  // namespace moe_mx
