// Native self-test of the oracle, built with AddressSanitizer and
// UndefinedBehaviorSanitizer (oracle/build.py --selftest, and a CPU test).
// Random tiny caches; checks memory safety plus invariants that hold for any
// input: each step adds exactly G to a unit's total importance (softmax rows
// sum to one), the cache ends at min(len+1, budget), sinks and the recent
// window survive.
#include "hikv_ref.h"

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

static int fail(const char *what, int a, int b) {
  std::fprintf(stderr, "selftest failure: %s (%d, %d)\n", what, a, b);
  return 1;
}

int main() {
  std::mt19937 rng(12345);
  std::normal_distribution<float> nd(0.f, 1.f);
  for (int trial = 0; trial < 300; ++trial) {
    const int B = 1 + rng() % 2, Hkv = 1 + rng() % 2, G = 1 + rng() % 3, D = 4 + 4 * (rng() % 3);
    const int Hq = Hkv * G, cap = 8 + rng() % 24, dtype = rng() % 2;
    const int S = rng() % 3, W = rng() % 4;
    const int r = (trial % 3 == 0) ? 1 + rng() % D : 0;
    const int kT = 1 + rng() % 10;
    const size_t el = dtype ? 2 : 4, row = (size_t)D * el, U = (size_t)B * Hkv;
    std::vector<char> k(U * cap * row), v(U * cap * row);
    std::vector<int32_t> pos(U * cap, -1), len(U), budget(U);
    std::vector<float> imp(U * cap, 0.f);
    for (size_t i = 0; i < k.size(); i += el) {
      float a = nd(rng), b = nd(rng);
      if (dtype) {
        uint32_t ua, ub;
        std::memcpy(&ua, &a, 4);
        std::memcpy(&ub, &b, 4);
        uint16_t ha = ua >> 16, hb = ub >> 16;
        std::memcpy(&k[i], &ha, 2);
        std::memcpy(&v[i], &hb, 2);
      } else {
        std::memcpy(&k[i], &a, 4);
        std::memcpy(&v[i], &b, 4);
      }
    }
    int newest = 0;
    for (size_t u = 0; u < U; ++u) {
      len[u] = rng() % cap;  // leave room for one append
      for (int n = 0; n < len[u]; ++n) pos[u * cap + n] = n;
      newest = std::max(newest, len[u]);
      budget[u] = S + (rng() % (cap - S));
    }
    std::vector<char> q(B * Hq * row), kn(U * row), vn(U * row);
    for (size_t i = 0; i < q.size(); ++i) q[i] = (char)(rng() & 0x3f);
    for (size_t i = 0; i < kn.size(); ++i) { kn[i] = (char)(rng() & 0x3f); vn[i] = (char)(rng() & 0x3f); }
    std::vector<int32_t> np(B, newest);
    std::vector<float> out((size_t)B * Hq * D);
    std::vector<double> psum(U);
    std::vector<uint8_t> kept(U * cap);
    hikv_ref_shape sh = {B, Hq, Hkv, D, cap, dtype, 0.f};
    hikv_ref_cache c = {k.data(), v.data(), pos.data(), imp.data(), len.data()};
    hikv_ref_policy pol = {budget.data(), 0, S, W, r, kT};
    hikv_ref_debug dbg;
    std::memset(&dbg, 0, sizeof dbg);
    std::vector<int32_t> selc((size_t)B * Hq * (r > 0 ? r : 1)), selt((size_t)B * Hq * kT), seln(B * Hq);
    std::vector<double> ax((size_t)B * Hq * cap);
    std::vector<float> ipe(U * cap);
    dbg.prob_sum = psum.data();
    dbg.kept = kept.data();
    dbg.sel_channels = selc.data();
    dbg.sel_tokens = selt.data();
    dbg.sel_count = seln.data();
    dbg.approx_logits = ax.data();
    dbg.imp_pre_evict = ipe.data();
    std::vector<int32_t> len0 = len;
    int st = hikv_ref_decode_step(&sh, &c, &pol, q.data(), kn.data(), vn.data(), np.data(), out.data(), &dbg);
    if (st != 0) return fail("status", st, trial);
    for (size_t u = 0; u < U; ++u) {
      if (std::fabs(psum[u] - G) > 1e-9 * G) return fail("prob sum", (int)u, trial);
      const int want = std::min(len0[u] + 1, budget[u]);
      if (len[u] != want) return fail("len", len[u], want);
      const int Wp = std::min(W, budget[u] - S);
      std::vector<int> seen(newest + 1, 0);
      for (int n = 0; n < len[u]; ++n) seen[pos[u * cap + n]] = 1;
      for (int p = 0; p <= newest; ++p) {
        const bool live_before = p < len0[u] || p == newest;
        const bool prot = p < S || p > newest - Wp;
        if (live_before && prot && !seen[p]) return fail("protected token evicted", p, trial);
      }
    }
  }
  std::printf("oracle selftest ok\n");
  return 0;
}
