// Memory-counter bookkeeping of the copy waves of the 32x32 tiled GEMM
// (gemm_tiled.hip), in closed form, host- and device-callable so that a host
// program can check it against a replay of the issue sequence.
//
// A copy wave has an NS-stage ring, C copies per stage and GC per scale group
// (a group is 4 stages).  Issue order: the prologue copies scale groups 0 and
// 1, then stages 0 .. NS-2; after barrier x the wave copies group x/4 + 1 when
// x % 4 == 0 and x >= 4 (into the buffer of group x/4 - 1, whose last stage
// was read before barrier x), then stage x + NS - 1.  Before barrier b it
// needs stage b and, when b opens a group, that group.  Stages and groups past
// the end of the stream are not issued and not counted.  Row-table copies are
// left out: they only add copies in flight after a given one, so leaving them
// out makes a wait stricter.  The copy waves do nothing else, so the counts
// are computed at run time.
#pragma once
#include <hip/hip_runtime.h>

namespace moe_mx {

template <int NS, int C, int GC>
struct TiledCopyCount {
  int total, ngroups;  // steps of the stream; groups (total / 4)

  __host__ __device__ static int lo(int a, int b) { return a < b ? a : b; }
  __host__ __device__ static int hi(int a, int b) { return a > b ? a : b; }
  // groups issued through the slot after barrier x (x = -1: the prologue)
  __host__ __device__ int groups_through(int x) const { return lo(ngroups, x >= 4 ? 2 + x / 4 : 2); }
  // copies issued through the slot after barrier x
  __host__ __device__ int issued_through(int x) const { return C * lo(total, NS + x) + GC * groups_through(x); }
  // copies issued up to and including stage s (issued in slot s - NS + 1,
  // after that slot's group)
  __host__ __device__ int through_stage(int s) const { return C * (s + 1) + GC * groups_through(s - NS + 1); }
  // copies issued up to and including group G (issued in slot 4G - 4, before
  // that slot's stage; groups 0 and 1 open the prologue)
  __host__ __device__ int through_group(int G) const {
    if (G < 2) return GC * (G + 1);
    return C * lo(total, NS + 4 * G - 5) + GC * (G + 1);
  }
  // copies that may stay in flight before barrier b
  __host__ __device__ int allowed(int b) const {
    int need = through_stage(b);
    if ((b & 3) == 0) need = hi(need, through_group(b >> 2));
    return issued_through(b - 1) - need;
  }
};

}  // namespace moe_mx
