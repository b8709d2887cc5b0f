// Host check of the closed-form copy counts of the tiled GEMM (tiled_count.h)
// and of the wide GEMM (wide_count.h): for every ring shape the kernels
// instantiate, and stream lengths of 1 to 120 scale groups, replay the copy
// waves' issue sequence and compare, before every barrier, the number of
// copies a wait lets stay in flight with the exact count (all copies issued so
// far after the last one the step needs).  The tiled kernel waits for exactly
// that count; the wide kernel waits for a per-phase steady count that must not
// exceed it, except in its last kWideTailWaits waits, which wait for every
// copy.  Prints "ok" and exits 0, or prints the first failure and exits 1.
#include <cstdio>
#include <vector>

#include "tiled_count.h"
#include "wide_count.h"

struct Copy {
  char kind;  // 'S' stage, 'G' scale group
  int index;
};

template <int NS, int C, int GC>
static bool check(int total) {
  const int ngroups = total / 4;
  std::vector<Copy> seq;
  auto group = [&](int g) { for (int i = 0; i < GC; ++i) seq.push_back({'G', g}); };
  auto stage = [&](int s) { for (int i = 0; i < C; ++i) seq.push_back({'S', s}); };
  for (int g = 0; g < 2 && g < ngroups; ++g) group(g);
  int issued = 0;
  for (; issued < NS - 1 && issued < total; ++issued) stage(issued);
  const moe_mx::TiledCopyCount<NS, C, GC> cnt{total, ngroups};
  for (int b = 0; b < total; ++b) {
    // exact: copies after the last copy of stage b and (at a group start) group b/4
    int last = -1;
    for (int i = 0; i < (int)seq.size(); ++i)
      if ((seq[i].kind == 'S' && seq[i].index == b) || ((b & 3) == 0 && seq[i].kind == 'G' && seq[i].index == b / 4))
        last = i;
    if (last < 0) {
      std::printf("NS=%d C=%d GC=%d total=%d: barrier %d needs a copy that was never issued\n", NS, C, GC, total, b);
      return false;
    }
    const int exact = (int)seq.size() - 1 - last;
    if (cnt.allowed(b) != exact) {
      std::printf("NS=%d C=%d GC=%d total=%d barrier %d: closed form %d, replay %d\n", NS, C, GC, total, b,
                  cnt.allowed(b), exact);
      return false;
    }
    if (b >= 4 && (b & 3) == 0 && b / 4 + 1 < ngroups) group(b / 4 + 1);
    if (issued < total) stage(issued++);
  }
  return true;
}

template <int NS, int C, int GC>
static bool sweep() {
  for (int groups = 1; groups <= 120; ++groups)
    if (!check<NS, C, GC>(4 * groups)) return false;
  return true;
}

// Wide GEMM stream: prologue = code stages 0..NS-1 then groups 0 and 1; after
// barrier g, code stage g+NS, then group (g+1)/4 + 1 when g % 4 == 3; stages
// and groups past the stream are not issued.  Before barrier g the step needs
// code stage g+1 and, when step g+1 opens a group, that group.
template <int NS, int C>
static bool check_wide(int total) {
  using W = moe_mx::WideCopyCount<NS, C>;
  std::vector<Copy> seq;
  auto stage = [&](int s) { if (s < total) for (int i = 0; i < C; ++i) seq.push_back({'S', s}); };
  auto group = [&](int G) { if (4 * G < total) seq.push_back({'G', G}); };
  for (int s = 0; s < NS; ++s) stage(s);
  group(0);
  group(1);
  for (int g = 0; g < total; ++g) {
    if (g + moe_mx::kWideTailWaits < total) {
      const int n = g + 1;  // < total here
      int last = -1;
      for (int i = 0; i < (int)seq.size(); ++i)
        if ((seq[i].kind == 'S' && seq[i].index == n) || ((n & 3) == 0 && seq[i].kind == 'G' && seq[i].index == n / 4))
          last = i;
      const int exact = (int)seq.size() - 1 - last;
      if (last < 0 || W::steady(g & 3) > exact) {
        std::printf("wide NS=%d C=%d total=%d barrier %d: steady wait %d, exact %d\n", NS, C, total, g,
                    W::steady(g & 3), last < 0 ? -1 : exact);
        return false;
      }
    }
    stage(g + NS);
    if ((g & 3) == 3) group((g + 1) / 4 + 1);
  }
  return true;
}

template <int NS, int C>
static bool sweep_wide() {
  for (int groups = 1; groups <= 120; ++groups)
    if (!check_wide<NS, C>(4 * groups)) return false;
  return true;
}

int main() {
  // activation waves: 4 stages (3 with E3M2 weights and 128-row tiles) of 8
  // or 12 code copies (128- or 192-row tiles), 1 or 2 group copies; weight
  // waves: 192-row tiles (128-row N-blocks) 6/4 stages (E2M1/E3M2) of 4 or 6
  // copies and 1 group copy, 128-row tiles (256-row N-blocks) 5/4 stages of 8
  // or 12 copies and 2 group copies
  // wide kernel: activation ring 3 stages of 6 copies, weight ring 4 of 4
  const bool ok = sweep<4, 8, 1>() && sweep<3, 8, 1>() && sweep<4, 12, 2>() && sweep<6, 4, 1>() &&
                  sweep<4, 6, 1>() && sweep<5, 8, 2>() && sweep<4, 12, 2>() && sweep_wide<3, 6>() &&
                  sweep_wide<4, 4>();
  std::printf(ok ? "ok\n" : "FAILED\n");
  return ok ? 0 : 1;
}
