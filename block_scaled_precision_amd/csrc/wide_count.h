// Memory-counter bookkeeping of the copy streams of the wide GEMM
// (gemm_wide.hip), in closed form; constexpr, so that the kernel's waits are
// compile-time immediates and a host program can check them against a replay
// of the issue sequence.
//
// A wave issues its prologue (code stages 0..NS-1, C copies each, then scale
// groups 0 and 1, one copy each) and after barrier g the code stage of step
// g+NS and, when g % 4 == 3, scale group (g+1)/4 + 1.  Before barrier g it
// needs the code stage of step g+1 and, when step g+1 opens a scale group,
// that group.  Row-table copies are left out of the count: they only add to
// the copies in flight after a given one, so leaving them out makes a wait
// stricter, never looser.  Stages or groups past the end of the stream are not
// issued but are counted here, which would make a wait looser (copies complete
// in issue order, so a wait that assumes more younger copies than exist can
// pass before the one it guards): the last kWideTailWaits waits of a stream
// wait for every copy instead (a code stage is skipped from barrier
// total - NS on, NS <= 4, a scale group from barrier total - 5 on).
#pragma once

namespace moe_mx {

constexpr int kWideGroup = 4;      // K-steps per scale group
constexpr int kWideTailWaits = 5;  // waits at the end of a stream that wait for every copy

template <int NS, int C>
struct WideCopyCount {
  static constexpr int P = NS * C + 2;
  // copies issued before barrier g
  static constexpr int before(int g) { return P + g * C + g / kWideGroup; }
  // copies issued up to and including code stage s / scale group G
  static constexpr int code_end(int s) { return s < NS ? (s + 1) * C : P + (s - NS + 1) * C + (s - NS) / kWideGroup; }
  static constexpr int group_end(int G) {
    return G < 2 ? NS * C + G + 1 : P + (kWideGroup * G - kWideGroup) * C + (G - 2) + 1;
  }
  // copies that may stay in flight before barrier g: all but those up to the
  // code stage of step g+1 and, when step g+1 opens a scale group, that group
  static constexpr int allowed(int g) {
    const int ce = code_end(g + 1);
    const int ge = group_end((g + 1) / kWideGroup);
    return before(g) - (((g + 1) % kWideGroup) == 0 && ge > ce ? ge : ce);
  }
  // From step kWideGroup on, allowed(g) depends only on g % kWideGroup; over
  // the first steps it is larger.  So the steady-state value of g's phase is
  // never looser than the exact count, and each wait is an immediate.
  static constexpr int steady(int q) { return allowed(4 * kWideGroup + q); }
  static constexpr bool steady_is_safe() {
    for (int g = 0; g < 8 * kWideGroup; ++g)
      if (steady(g % kWideGroup) > allowed(g)) return false;
    return true;
  }
};

}  // namespace moe_mx
