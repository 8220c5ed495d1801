/*
 * hikv_ref -- CPU oracle for the importance-aware KV decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the slow, plain definition the
 * GPU library is checked against.  Only the test suite, the package smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, table or helper with the HIP library.
 *
 * Everything here works on host memory, one (batch, KV head) unit at a time,
 * in the order the pages state the method:
 *   append -> attention (per q-head) -> importance accumulation -> eviction.
 * Arithmetic is fp64; stored state (importance) keeps the cache's fp32 type.
 *
 * Sources (pages are cited by title and section):
 *  - HiKV: Hierarchical Importance-Aware KV Cache with Hardware Acceleration,
 *    Sec. II-A (P = softmax(QK^T), PV), Sec. III-B (importance score),
 *    Sec. III-C (Stage II: top-B_II channels of Q by magnitude), Algorithm 1.
 *  - KV Cache Compression and Dynamic Pruning in Production Serving,
 *    Sec. 3 "StreamingLLM" (sink + window set), Sec. 3 "H2O" (cumulative
 *    attention score, protected sinks/window, keep the top of the rest),
 *    Sec. 5 (GQA pooled importance).
 *  - Kelle (papercache summary), Sec. 2.2 (order of [k,v] pairs does not
 *    matter), Sec. 4.1 (per-head eviction by accumulated attention; prefill
 *    importance as attention column sums; initial and recent tokens kept).
 *  - Not All Heads Matter (HeadKV), Sec. 3.2 (per-head budgets).
 *  - HiKV Sec. III-B (dual bank: the score of a token sums the probabilities
 *    it receives while in the recent bank, then stays frozen; promotion into
 *    the important bank iff that score beats the bank's lowest) and
 *    Sec. III-D (bank initialisation from windowed prompt scores).
 *  - HiKV Sec. III-C and Algorithm 1 (Stage II V side: chunks of d_h entries
 *    of P, top-B_II per chunk, P.V over the kept rows).
 *  - Kelle Sec. 4.1 (Eq. 3) and Sec. 5.3 (importance as summed attention
 *    scores taken before the softmax).
 *  - "KV Cache Compression and Dynamic Pruning in Production Serving",
 *    SnapKV section (observation-window scores, 1-D max pooling).
 */
#ifndef HIKV_REF_H
#define HIKV_REF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HIKV_REF_F32 0
#define HIKV_REF_BF16 1

#define HIKV_REF_OK 0
#define HIKV_REF_EINVAL (-1)
#define HIKV_REF_ECAPACITY (-4)
#define HIKV_REF_EBUDGET (-5)

typedef struct {
  int32_t batch, n_q_heads, n_kv_heads, head_dim, capacity;
  int32_t kv_dtype; /* HIKV_REF_F32 | HIKV_REF_BF16 (q, k_new, v_new too) */
  float scale;      /* <= 0 -> 1/sqrt(head_dim) */
} hikv_ref_shape;

typedef struct {
  void *k, *v;      /* [B][Hkv][cap][D] */
  int32_t *pos;     /* [B][Hkv][cap] absolute position per slot */
  float *imp;       /* [B][Hkv][cap] cumulative importance */
  int32_t *len;     /* [B][Hkv] live slots are [0, len) */
} hikv_ref_cache;

/* Which tokens a step's attention probabilities are added to.
 * ALL: every live token (H2O's cumulative score).
 * RECENT: only the W' = min(n_recent, budget - n_sink) newest positions (the
 * protected window); everything older keeps a frozen score.  With n_sink 0
 * and n_recent = budget / 2 this is HiKV's dual bank (Sec. III-B): the window
 * is the recent bank, the rest the important bank, and each token's score is
 * the sum of the W' probabilities it received from its own step on. */
#define HIKV_REF_ACC_ALL 0
#define HIKV_REF_ACC_RECENT 1
/* LOGIT: every live token gains the pre-softmax logit scale * q.k it gets
 * from the group's queries (Kelle Sec. 5.3: the scores are summed without the
 * softmax); with Stage II on, the reduced logit. */
#define HIKV_REF_ACC_LOGIT 2

/* What Stage II does with the approximate probabilities on the V side.
 * TOPK: the k_T tokens with the largest approximate logit get an exact
 * (full-channel) softmax, renormalised over them, and P.V over them.
 * CHUNK: HiKV Sec. III-C literally: the approximate P over the live tokens in
 * position order is cut into chunks of D tokens (the last one shorter); each
 * chunk keeps its r largest entries (ties: lower position); the output is the
 * sum of those entries times their V rows, not renormalised. */
#define HIKV_REF_S2V_TOPK 0
#define HIKV_REF_S2V_CHUNK 1

typedef struct {
  const int32_t *budget; /* [B][Hkv] or NULL -> budget_all */
  int32_t budget_all, n_sink, n_recent;
  int32_t stage2_channels; /* r; 0 = Stage II off */
  int32_t stage2_tokens;   /* tokens kept for the exact softmax (k_T) */
  int32_t accumulate;      /* HIKV_REF_ACC_ALL | HIKV_REF_ACC_RECENT | HIKV_REF_ACC_LOGIT */
  int32_t stage2_v;        /* HIKV_REF_S2V_TOPK | HIKV_REF_S2V_CHUNK (used when r > 0) */
  /* Eviction granularity ("KV Cache Compression and Dynamic Pruning in
   * Production Serving", Sec. 5, PagedAttention block fragmentation): 0 or 1,
   * single tokens; P >= 2 (at most HIKV_REF_MAX_BLOCK), whole blocks of P
   * consecutive positions (block id = pos / P).  A block holding a protected
   * token is kept whole; the other blocks are ranked by the sum of their
   * tokens' importance and evicted lowest first (equal sums: the higher
   * block id first) while more than the budget's tokens are live, so a unit
   * may end below its budget, or above it when protected blocks hold more. */
  int32_t block_tokens;
} hikv_ref_policy;

#define HIKV_REF_MAX_BLOCK 1024

/* Optional per-step debug outputs; any pointer may be NULL. */
typedef struct {
  int32_t *sel_channels; /* [B][Hq][r]  chosen channels, ascending */
  int32_t *sel_tokens;   /* [B][Hq][k_T] positions of the exact-softmax set, ascending, -1 padded */
  int32_t *sel_count;    /* [B][Hq]     size of that set (CHUNK: tokens kept over all chunks) */
  double *approx_logits; /* [B][Hq][cap] Stage II approximate logit per pre-eviction slot */
  float *imp_pre_evict;  /* [B][Hkv][cap] importance after accumulation, pre-eviction slot order */
  uint8_t *kept;         /* [B][Hkv][cap] 1 if that pre-eviction slot survives eviction */
  double *prob_sum;      /* [B][Hkv] total importance added this step */
} hikv_ref_debug;

/* One decode step for every (b, j).  Returns 0, or the first unit error
 * (ECAPACITY / EBUDGET; that unit is left unchanged and its output rows are
 * zero), or EINVAL for a bad shape/policy (nothing is touched). */
int hikv_ref_decode_step(const hikv_ref_shape *shape, const hikv_ref_cache *cache,
                         const hikv_ref_policy *policy, const void *q, const void *k_new,
                         const void *v_new, const int32_t *new_pos, float *out,
                         hikv_ref_debug *dbg);

/* Compress every unit to its budget using the current importance;
 * newest_pos[b] anchors the recent window. */
int hikv_ref_evict(const hikv_ref_shape *shape, const hikv_ref_cache *cache,
                   const hikv_ref_policy *policy, const int32_t *newest_pos,
                   hikv_ref_debug *dbg);

/* Add prompt-side importance: for every observation query i (position
 * q_pos[b][i]) and q-head of the group, the causal softmax row over the
 * cached tokens (those with pos <= q_pos) is added to those tokens'
 * importance.  window == 0: every such entry counts (column sums);
 * window > 0: an entry counts only when 0 <= q_pos - pos < window.
 * pool > 1 (SnapKV's 1-D max pooling): a token at position p adds instead
 * the largest of this call's scores over the cached positions p .. p+pool-1. */
int hikv_ref_prefill_scores(const hikv_ref_shape *shape, const hikv_ref_cache *cache,
                            const void *q_obs /* [B][Hq][n_obs][D] */,
                            const int32_t *q_pos /* [B][n_obs] */, int32_t n_obs,
                            int32_t window, int32_t pool);

#ifdef __cplusplus
}
#endif
#endif
