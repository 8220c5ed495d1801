// hikv_ref.cpp -- plain, slow, single-threaded CPU oracle.
//
// TEST INFRASTRUCTURE ONLY (see hikv_ref.h).  Written for a reader checking it
// against the pages by eye: no blocking, no fusion, no reordering.  fp64
// arithmetic throughout; the cache's importance array keeps its fp32 type and
// is rounded once per step after the fp64 sum is formed.
//
// Readings where the pages are silent or disagree (each is stated once here):
//  R1 logits are scaled by 1/sqrt(D) unless the caller gives a scale.  The
//     Stage II approximate logits use the same scale.
//  R2 the new token is appended first and attends to itself.
//  R3 importance is the post-softmax probability a token receives, summed over
//     the q-heads of its KV group and over every step it is live.
//  R4 eviction is per (batch, KV head); ranking key = (importance desc,
//     position asc), so among equal scores the newer token goes first.
//  R5 sinks are absolute positions 0..S-1; the recent window is the W'
//     newest positions including the new token, W' = min(W, budget - S).
//  R7 block-granular eviction: a block is the P consecutive positions
//     [P b, P b + P); its score is the fp64 sum of its live tokens'
//     importance; a block with any protected token is never evicted.
//  R6 Stage II: per q-head, channels E = top-r |q_d| (ties: lower d);
//     approximate logits over E; importance from their softmax over all live
//     tokens; output = exact full-D softmax restricted to the k_T tokens with
//     the largest approximate logit (ties: lower position), times V.

#include "hikv_ref.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

namespace {

struct Dims {
  int B, Hq, Hkv, D, cap, dtype, G;
  double scale;
  size_t el;
};

bool read_dims(const hikv_ref_shape *s, Dims *d) {
  if (!s) return false;
  if (s->batch < 0 || s->n_kv_heads < 1 || s->n_q_heads < 1 || s->head_dim < 1 || s->capacity < 1)
    return false;
  if (s->n_q_heads % s->n_kv_heads != 0) return false;
  if (s->kv_dtype != HIKV_REF_F32 && s->kv_dtype != HIKV_REF_BF16) return false;
  d->B = s->batch;
  d->Hq = s->n_q_heads;
  d->Hkv = s->n_kv_heads;
  d->D = s->head_dim;
  d->cap = s->capacity;
  d->dtype = s->kv_dtype;
  d->G = s->n_q_heads / s->n_kv_heads;
  d->scale = s->scale > 0.0f ? (double)s->scale : 1.0 / std::sqrt((double)s->head_dim);
  d->el = s->kv_dtype == HIKV_REF_F32 ? 4 : 2;
  return true;
}

// Widen one stored element to double (bf16 is the top half of an fp32).
double elem(const void *base, int dtype, size_t i) {
  if (dtype == HIKV_REF_F32) return (double)static_cast<const float *>(base)[i];
  uint32_t bits = (uint32_t) static_cast<const uint16_t *>(base)[i] << 16;
  float f;
  std::memcpy(&f, &bits, 4);
  return (double)f;
}

// One (batch, KV head) unit viewed as plain arrays.
struct Unit {
  char *k, *v;
  int32_t *pos;
  float *imp;
  int32_t *len;
};

Unit unit_view(const Dims &d, const hikv_ref_cache *c, int b, int j) {
  size_t u = (size_t)b * d.Hkv + j;
  size_t row = (size_t)d.D * d.el;
  Unit x;
  x.k = static_cast<char *>(c->k) + u * d.cap * row;
  x.v = static_cast<char *>(c->v) + u * d.cap * row;
  x.pos = c->pos + u * d.cap;
  x.imp = c->imp + u * d.cap;
  x.len = c->len + u;
  return x;
}

double key_elem(const Dims &d, const Unit &x, int n, int c) {
  return elem(x.k, d.dtype, (size_t)n * d.D + c);
}
double val_elem(const Dims &d, const Unit &x, int n, int c) {
  return elem(x.v, d.dtype, (size_t)n * d.D + c);
}

// softmax over the listed logits (max-subtracted for range only).
std::vector<double> softmax(const std::vector<double> &s) {
  std::vector<double> p(s.size());
  if (s.empty()) return p;
  double m = *std::max_element(s.begin(), s.end());
  double z = 0.0;
  for (size_t i = 0; i < s.size(); ++i) {
    p[i] = std::exp(s[i] - m);
    z += p[i];
  }
  for (size_t i = 0; i < s.size(); ++i) p[i] /= z;
  return p;
}

int unit_budget(const Dims &d, const hikv_ref_policy *pol, int b, int j) {
  return pol->budget ? pol->budget[(size_t)b * d.Hkv + j] : pol->budget_all;
}

bool budget_ok(const Dims &d, const hikv_ref_policy *pol, int beta) {
  return beta >= pol->n_sink && beta <= d.cap;
}

// Block-granular selection (R7): which slots survive when whole blocks of P
// positions are evicted, lowest summed importance first (equal sums: higher
// block id first), until at most beta tokens are live.
void select_blocks(const Unit &x, int L, int beta, int P, const std::vector<uint8_t> &prot,
                   std::vector<uint8_t> &keep) {
  struct Blk {
    int64_t id;
    double score;
    int count;
    bool prot;
  };
  std::vector<Blk> blk;
  std::vector<int> of(L);  // slot -> index in blk
  for (int n = 0; n < L; ++n) {
    const int64_t p = x.pos[n];
    const int64_t id = p >= 0 ? p / P : -((-p + P - 1) / P);  // floor(pos / P)
    int k = 0;
    while (k < (int)blk.size() && blk[k].id != id) ++k;
    if (k == (int)blk.size()) blk.push_back({id, 0.0, 0, false});
    blk[k].score += (double)x.imp[n];
    blk[k].count += 1;
    blk[k].prot = blk[k].prot || prot[n];
    of[n] = k;
  }
  std::vector<int> order;
  for (int k = 0; k < (int)blk.size(); ++k)
    if (!blk[k].prot) order.push_back(k);
  std::sort(order.begin(), order.end(), [&](int a, int b) {
    if (blk[a].score != blk[b].score) return blk[a].score < blk[b].score;
    return blk[a].id > blk[b].id;
  });
  std::vector<uint8_t> gone(blk.size(), 0);
  int live = L;
  for (int k : order) {
    if (live <= beta) break;
    gone[k] = 1;
    live -= blk[k].count;
  }
  for (int n = 0; n < L; ++n) keep[n] = !gone[of[n]];
}

// Eviction of one unit down to budget beta (H2O with protected sinks and
// window; whole blocks of positions with pol->block_tokens >= 2).  kept[]
// (pre-eviction slot order) is filled when non-null.  The survivors are
// compacted stably into slots [0, len).
void evict_unit(const Dims &d, const Unit &x, const hikv_ref_policy *pol, int beta,
                int32_t newest, uint8_t *kept_out) {
  const int L = *x.len;
  std::vector<uint8_t> keep(L, 1);
  if (L > beta) {
    const int S = pol->n_sink;
    const int W = std::min(pol->n_recent, beta - S);
    std::vector<uint8_t> prot(L, 0);
    int n_prot = 0;
    std::vector<int> cand;
    for (int n = 0; n < L; ++n) {
      prot[n] = (x.pos[n] < S) || (x.pos[n] > newest - W);
      if (prot[n])
        ++n_prot;
      else
        cand.push_back(n);
    }
    if (pol->block_tokens >= 2) {
      select_blocks(x, L, beta, pol->block_tokens, prot, keep);
    } else {
      // Rank candidates: higher importance first, then lower position.
      std::sort(cand.begin(), cand.end(), [&](int a, int b) {
        if (x.imp[a] != x.imp[b]) return x.imp[a] > x.imp[b];
        return x.pos[a] < x.pos[b];
      });
      int keep_n = std::max(0, beta - n_prot);
      for (int n = 0; n < L; ++n) keep[n] = prot[n];
      for (int i = 0; i < (int)cand.size() && i < keep_n; ++i) keep[cand[i]] = 1;
    }
    // Stable in-place compaction of the survivors.
    const size_t row = (size_t)d.D * d.el;
    int w = 0;
    for (int n = 0; n < L; ++n) {
      if (!keep[n]) continue;
      if (w != n) {
        std::memmove(x.k + (size_t)w * row, x.k + (size_t)n * row, row);
        std::memmove(x.v + (size_t)w * row, x.v + (size_t)n * row, row);
        x.pos[w] = x.pos[n];
        x.imp[w] = x.imp[n];
      }
      ++w;
    }
    *x.len = w;
  }
  if (kept_out)
    for (int n = 0; n < L; ++n) kept_out[n] = keep[n];
}

bool policy_ok(const Dims &d, const hikv_ref_policy *pol) {
  if (!pol || pol->n_sink < 0 || pol->n_recent < 0) return false;
  if (pol->accumulate != HIKV_REF_ACC_ALL && pol->accumulate != HIKV_REF_ACC_RECENT &&
      pol->accumulate != HIKV_REF_ACC_LOGIT)
    return false;
  if (pol->stage2_channels < 0 || pol->stage2_channels > d.D) return false;
  if (pol->stage2_v != HIKV_REF_S2V_TOPK && pol->stage2_v != HIKV_REF_S2V_CHUNK) return false;
  if (pol->stage2_channels > 0 && pol->stage2_v == HIKV_REF_S2V_TOPK && pol->stage2_tokens < 1)
    return false;
  if (pol->block_tokens < 0 || pol->block_tokens > HIKV_REF_MAX_BLOCK) return false;
  return true;
}

}  // namespace

extern "C" int hikv_ref_decode_step(const hikv_ref_shape *shape, const hikv_ref_cache *cache,
                                    const hikv_ref_policy *pol, const void *q,
                                    const void *k_new, const void *v_new,
                                    const int32_t *new_pos, float *out, hikv_ref_debug *dbg) {
  Dims d;
  if (!read_dims(shape, &d) || !cache || !policy_ok(d, pol)) return HIKV_REF_EINVAL;
  if (d.B == 0) return HIKV_REF_OK;
  if (!q || !k_new || !v_new || !new_pos || !out) return HIKV_REF_EINVAL;
  const int r = pol->stage2_channels;
  const int kT = pol->stage2_tokens;
  const size_t row = (size_t)d.D * d.el;
  int status = HIKV_REF_OK;

  for (int b = 0; b < d.B; ++b) {
    for (int j = 0; j < d.Hkv; ++j) {
      Unit x = unit_view(d, cache, b, j);
      const size_t u = (size_t)b * d.Hkv + j;
      const int beta = unit_budget(d, pol, b, j);
      int err = HIKV_REF_OK;
      if (*x.len + 1 > d.cap) err = HIKV_REF_ECAPACITY;
      else if (!budget_ok(d, pol, beta)) err = HIKV_REF_EBUDGET;
      if (err != HIKV_REF_OK) {
        if (status == HIKV_REF_OK) status = err;
        for (int g = 0; g < d.G; ++g)
          for (int c = 0; c < d.D; ++c)
            out[((size_t)b * d.Hq + j * d.G + g) * d.D + c] = 0.0f;
        continue;
      }

      // Append: the new token takes the next free slot with importance 0.
      const int slot = *x.len;
      std::memcpy(x.k + (size_t)slot * row,
                  static_cast<const char *>(k_new) + ((size_t)b * d.Hkv + j) * row, row);
      std::memcpy(x.v + (size_t)slot * row,
                  static_cast<const char *>(v_new) + ((size_t)b * d.Hkv + j) * row, row);
      x.pos[slot] = new_pos[b];
      x.imp[slot] = 0.0f;
      *x.len = slot + 1;
      const int L = *x.len;

      std::vector<double> added(L, 0.0);  // importance this step, per slot
      const bool by_logit = pol->accumulate == HIKV_REF_ACC_LOGIT;
      for (int g = 0; g < d.G; ++g) {
        const int h = j * d.G + g;
        std::vector<double> qh(d.D);
        for (int c = 0; c < d.D; ++c)
          qh[c] = elem(q, d.dtype, ((size_t)b * d.Hq + h) * d.D + c);
        std::vector<double> o(d.D, 0.0);

        if (r == 0) {
          // Stage I: logits over every live token, softmax, P.V.
          std::vector<double> s(L);
          for (int n = 0; n < L; ++n) {
            double acc = 0.0;
            for (int c = 0; c < d.D; ++c) acc += qh[c] * key_elem(d, x, n, c);
            s[n] = d.scale * acc;
          }
          std::vector<double> p = softmax(s);
          for (int n = 0; n < L; ++n) {
            for (int c = 0; c < d.D; ++c) o[c] += p[n] * val_elem(d, x, n, c);
            added[n] += by_logit ? s[n] : p[n];
          }
        } else {
          // Stage II, K side: channels with the largest |q_d|.
          std::vector<int> ch(d.D);
          for (int c = 0; c < d.D; ++c) ch[c] = c;
          std::sort(ch.begin(), ch.end(), [&](int a, int bb) {
            double fa = std::fabs(qh[a]), fb = std::fabs(qh[bb]);
            if (fa != fb) return fa > fb;
            return a < bb;
          });
          std::vector<int> E(ch.begin(), ch.begin() + r);
          // Approximate logits from the chosen channels only.
          std::vector<double> st(L);
          for (int n = 0; n < L; ++n) {
            double acc = 0.0;
            for (int c : E) acc += qh[c] * key_elem(d, x, n, c);
            st[n] = d.scale * acc;
          }
          std::vector<double> pt = softmax(st);
          for (int n = 0; n < L; ++n) added[n] += by_logit ? st[n] : pt[n];
          if (dbg && dbg->sel_channels) {
            std::vector<int> e = E;
            std::sort(e.begin(), e.end());
            for (int i = 0; i < r; ++i) dbg->sel_channels[((size_t)b * d.Hq + h) * r + i] = e[i];
          }
          if (dbg && dbg->approx_logits)
            for (int n = 0; n < L; ++n)
              dbg->approx_logits[((size_t)b * d.Hq + h) * d.cap + n] = st[n];
          if (pol->stage2_v == HIKV_REF_S2V_CHUNK) {
            // V side, HiKV's chunked selection: the live tokens in position
            // order, cut into chunks of D; each chunk keeps its r largest
            // probabilities (ties: lower position) and the output sums those
            // probabilities times their V rows, with no renormalisation.
            std::vector<int> byp(L);
            for (int n = 0; n < L; ++n) byp[n] = n;
            std::sort(byp.begin(), byp.end(), [&](int a, int bb) { return x.pos[a] < x.pos[bb]; });
            int kept_total = 0;
            for (int c0 = 0; c0 < L; c0 += d.D) {
              const int m = std::min(d.D, L - c0);
              std::vector<int> chunk(byp.begin() + c0, byp.begin() + c0 + m);
              std::sort(chunk.begin(), chunk.end(), [&](int a, int bb) {
                if (pt[a] != pt[bb]) return pt[a] > pt[bb];
                return x.pos[a] < x.pos[bb];
              });
              const int keep = std::min(r, m);
              for (int i = 0; i < keep; ++i)
                for (int c = 0; c < d.D; ++c) o[c] += pt[chunk[i]] * val_elem(d, x, chunk[i], c);
              kept_total += keep;
            }
            if (dbg && dbg->sel_count) dbg->sel_count[(size_t)b * d.Hq + h] = kept_total;
            for (int c = 0; c < d.D; ++c) out[((size_t)b * d.Hq + h) * d.D + c] = (float)o[c];
            continue;
          }
          // Tokens kept for the exact pass: largest approximate logit first.
          std::vector<int> order(L);
          for (int n = 0; n < L; ++n) order[n] = n;
          std::sort(order.begin(), order.end(), [&](int a, int bb) {
            if (st[a] != st[bb]) return st[a] > st[bb];
            return x.pos[a] < x.pos[bb];
          });
          const int nt = std::min(kT, L);
          std::vector<int> T(order.begin(), order.begin() + nt);
          // Exact logits over T, softmax over T only, P.V over T.
          std::vector<double> s(nt);
          for (int i = 0; i < nt; ++i) {
            double acc = 0.0;
            for (int c = 0; c < d.D; ++c) acc += qh[c] * key_elem(d, x, T[i], c);
            s[i] = d.scale * acc;
          }
          std::vector<double> p = softmax(s);
          for (int i = 0; i < nt; ++i)
            for (int c = 0; c < d.D; ++c) o[c] += p[i] * val_elem(d, x, T[i], c);

          if (dbg && dbg->sel_tokens) {
            std::vector<int32_t> tp(nt);
            for (int i = 0; i < nt; ++i) tp[i] = x.pos[T[i]];
            std::sort(tp.begin(), tp.end());
            for (int i = 0; i < kT; ++i)
              dbg->sel_tokens[((size_t)b * d.Hq + h) * kT + i] = i < nt ? tp[i] : -1;
          }
          if (dbg && dbg->sel_count) dbg->sel_count[(size_t)b * d.Hq + h] = nt;
        }
        for (int c = 0; c < d.D; ++c) out[((size_t)b * d.Hq + h) * d.D + c] = (float)o[c];
      }

      // Accumulate: every live token gets the probability it received, or,
      // with the HiKV dual bank, only the tokens of the recent window (the
      // window eviction protects); older scores stay frozen.
      const int Wacc = std::min(pol->n_recent, beta - pol->n_sink);
      double total = 0.0;
      for (int n = 0; n < L; ++n) {
        if (pol->accumulate == HIKV_REF_ACC_RECENT && !(x.pos[n] > new_pos[b] - Wacc)) continue;
        x.imp[n] = (float)((double)x.imp[n] + added[n]);
        total += added[n];
      }
      if (dbg && dbg->prob_sum) dbg->prob_sum[u] = total;
      if (dbg && dbg->imp_pre_evict)
        for (int n = 0; n < L; ++n) dbg->imp_pre_evict[u * d.cap + n] = x.imp[n];

      // Evict down to the budget.
      evict_unit(d, x, pol, beta, new_pos[b], dbg && dbg->kept ? dbg->kept + u * d.cap : nullptr);
    }
  }
  return status;
}

extern "C" int hikv_ref_evict(const hikv_ref_shape *shape, const hikv_ref_cache *cache,
                              const hikv_ref_policy *pol, const int32_t *newest_pos,
                              hikv_ref_debug *dbg) {
  Dims d;
  if (!read_dims(shape, &d) || !cache || !policy_ok(d, pol)) return HIKV_REF_EINVAL;
  if (d.B == 0) return HIKV_REF_OK;
  if (!newest_pos) return HIKV_REF_EINVAL;
  int status = HIKV_REF_OK;
  for (int b = 0; b < d.B; ++b)
    for (int j = 0; j < d.Hkv; ++j) {
      Unit x = unit_view(d, cache, b, j);
      const size_t u = (size_t)b * d.Hkv + j;
      const int beta = unit_budget(d, pol, b, j);
      if (!budget_ok(d, pol, beta) || *x.len > d.cap) {
        if (status == HIKV_REF_OK) status = HIKV_REF_EBUDGET;
        continue;
      }
      if (dbg && dbg->imp_pre_evict)
        for (int n = 0; n < *x.len; ++n) dbg->imp_pre_evict[u * d.cap + n] = x.imp[n];
      evict_unit(d, x, pol, beta, newest_pos[b], dbg && dbg->kept ? dbg->kept + u * d.cap : nullptr);
    }
  return status;
}

extern "C" int hikv_ref_prefill_scores(const hikv_ref_shape *shape, const hikv_ref_cache *cache,
                                       const void *q_obs, const int32_t *q_pos, int32_t n_obs,
                                       int32_t window, int32_t pool) {
  Dims d;
  if (!read_dims(shape, &d) || !cache || n_obs < 0 || window < 0 || pool < 0) return HIKV_REF_EINVAL;
  if (d.B == 0 || n_obs == 0) return HIKV_REF_OK;
  if (!q_obs || !q_pos) return HIKV_REF_EINVAL;
  for (int b = 0; b < d.B; ++b)
    for (int j = 0; j < d.Hkv; ++j) {
      Unit x = unit_view(d, cache, b, j);
      const int L = *x.len;
      if (L > d.cap) return HIKV_REF_EINVAL;
      std::vector<double> added(L, 0.0);
      for (int g = 0; g < d.G; ++g) {
        const int h = j * d.G + g;
        for (int i = 0; i < n_obs; ++i) {
          const int32_t qp = q_pos[(size_t)b * n_obs + i];
          // The query's softmax row runs over every token it may see (causal).
          std::vector<int> vis;
          for (int n = 0; n < L; ++n)
            if ((int64_t)qp - x.pos[n] >= 0) vis.push_back(n);
          if (vis.empty()) continue;
          std::vector<double> s(vis.size());
          for (size_t t = 0; t < vis.size(); ++t) {
            double acc = 0.0;
            for (int c = 0; c < d.D; ++c)
              acc += elem(q_obs, d.dtype, (((size_t)b * d.Hq + h) * n_obs + i) * d.D + c) *
                     key_elem(d, x, vis[t], c);
            s[t] = d.scale * acc;
          }
          std::vector<double> p = softmax(s);
          // A token only collects from queries within `window` steps of it
          // (HiKV's localized score); window 0 collects from all of them.
          for (size_t t = 0; t < vis.size(); ++t) {
            const int64_t dist = (int64_t)qp - x.pos[vis[t]];
            if (window > 0 && dist >= window) continue;
            added[vis[t]] += p[t];
          }
        }
      }
      if (pool > 1) {
        // SnapKV's pooling: the largest score over positions p .. p+pool-1
        // among the cached tokens (positions are distinct).
        std::vector<double> pooled(L);
        for (int n = 0; n < L; ++n) {
          pooled[n] = added[n];
          for (int m = 0; m < L; ++m) {
            const int64_t dp = (int64_t)x.pos[m] - x.pos[n];
            if (dp >= 0 && dp < pool) pooled[n] = std::max(pooled[n], added[m]);
          }
        }
        added = pooled;
      }
      for (int n = 0; n < L; ++n) x.imp[n] = (float)((double)x.imp[n] + added[n]);
    }
  return HIKV_REF_OK;
}
