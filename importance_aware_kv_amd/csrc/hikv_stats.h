// hikv_stats.h -- a unit's softmax statistics from its split-K tiles.
#ifndef HIKV_STATS_H
#define HIKV_STATS_H

#include "hikv_common.h"

namespace hikv {

// The softmax statistics of q-head g of unit u's group (log2-domain max and
// sum over every live token), combined from the unit's split-K tile partials
// in tile order in one pass (online rescaling), so that the launches after
// the attention tiles need no combine launch.  A tile whose every token was
// masked (max -inf) adds nothing.
__device__ __forceinline__ void unit_softmax_stats(const StepArgs &a, int u, int g, float &M, float &S) {
  const int U = a.n_units;
  const int t0 = a.ws.plan[u], t1 = (u + 1 < U) ? a.ws.plan[u + 1] : a.ws.plan[U];
  const float *pm = a.ws.part_ml;
  float m = -INFINITY, s = 0.f;
  for (int t = t0; t < t1; ++t) {
    const float mt = pm[((size_t)t * a.G + g) * 2], lt = pm[((size_t)t * a.G + g) * 2 + 1];
    if (mt == -INFINITY) continue;
    if (mt > m) {
      s = (m == -INFINITY) ? 0.f : s * fast_exp2(m - mt);
      m = mt;
    }
    s += lt * fast_exp2(mt - m);
  }
  M = m;
  S = s;
}

}  // namespace hikv

#endif
