/*
 * hikv.h -- C ABI of the importance-aware KV decode library (AMD MI355X, gfx950).
 *
 * One decode step of single-query attention over a budgeted, slot-indexed KV
 * cache, fused with importance-based eviction:
 *
 *   append the new (k, v) -> logits q.k for the G q-heads sharing each KV
 *   head -> softmax -> P.V -> add each cached token's attention probability
 *   (summed over the group) to its importance -> if the cache is over budget,
 *   evict the lowest-importance tokens, never the sinks or the recent window,
 *   and compact the survivors in place.
 *
 * Sources (pages are cited by title and section):
 *   [HiKV]  "HiKV: Hierarchical Importance-Aware KV Cache with Hardware
 *           Acceleration for LLM Decoding": Sec. II-A (decode GeMVs QK^T and
 *           PV, P = softmax(QK^T)), Sec. III-B (importance score from
 *           accumulated P; budget), Sec. III-C (Stage II: top-B_II channels of
 *           Q by magnitude guide the K loads), Algorithm 1.
 *   [Blog]  "KV Cache Compression and Dynamic Pruning in Production Serving":
 *           Sec. 3 StreamingLLM (sinks + rolling window), Sec. 3 H2O
 *           (cumulative attention score; evict the lowest while keeping sinks
 *           and the local window), Sec. 5 (GQA: pool importance over the
 *           q-heads of a KV group; ragged per-head lengths; compaction).
 *   [Kelle] "Kelle: Co-design KV Caching and eDRAM" summary: Sec. 2.2 (the
 *           order of [k, v] pairs does not change the output, so a slot cache
 *           needs no order), Sec. 4.1 (per-head eviction by accumulated
 *           attention; prefill importance as column sums of the prompt's
 *           attention; initial and recent tokens are kept).
 *   [HeadKV] "Not All Heads Matter": Sec. 3.2 (a budget per head).
 *
 * Conventions
 *   - Every data pointer is a DEVICE pointer owned by the caller, except the
 *     three descriptor structs, which live in host memory and are read during
 *     the call only.  The library keeps no pointer after a call returns.
 *   - All work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*; NULL = the null stream).  No call allocates device memory,
 *     synchronises or issues a memset, so a sequence of calls can be captured
 *     into a HIP graph.  Exception: hikv_device_status() synchronises.
 *   - Calls that share a cache or a workspace must be ordered on one stream.
 *   - Layouts are row-major; q-head h belongs to KV head h / G (G = Hq/Hkv).
 *   - Host-detectable errors are returned synchronously and enqueue nothing.
 *     Per-unit errors found on the device leave that (batch, KV head) unit
 *     unchanged, zero its output rows, and set a sticky status word in the
 *     workspace that hikv_device_status() reports.
 */
#ifndef HIKV_H
#define HIKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of K, V, q, k_new, v_new, q_obs. */
#define HIKV_F32 0
#define HIKV_BF16 1

/* Status codes. */
#define HIKV_OK 0
#define HIKV_EINVAL (-1)       /* null pointer, bad shape/policy, workspace too small */
#define HIKV_EUNSUPPORTED (-2) /* head_dim not 64/128, group size not 1/2/4/8, too many units, no gfx950;
                                  block_tokens >= 2 with Stage II, the multi-launch path or hikv_evict */
#define HIKV_EDEVICE (-3)      /* a HIP runtime call or kernel launch failed */
#define HIKV_ECAPACITY (-4)    /* device: len + 1 > capacity for some unit */
#define HIKV_EBUDGET (-5)      /* device: budget < n_sink or budget > capacity for some unit */

typedef struct hikv_shape {
  int32_t batch;       /* B >= 0 (0: every call is a no-op) */
  int32_t n_q_heads;   /* Hq, a multiple of n_kv_heads */
  int32_t n_kv_heads;  /* Hkv >= 1 */
  int32_t head_dim;    /* D: 64 or 128 */
  int32_t capacity;    /* slots per (batch, KV head) */
  int32_t kv_dtype;    /* HIKV_F32 or HIKV_BF16; q, k_new, v_new, q_obs use it too */
  float scale;         /* logit scale; <= 0 -> 1/sqrt(head_dim) */
} hikv_shape;

/* The cache.  One "unit" is a (batch b, KV head j) pair, u = b*Hkv + j.
 * Slots [0, len[u]) of a unit are live, in no particular order ([Kelle]
 * Sec. 2.2); pos holds each slot's absolute token position. */
typedef struct hikv_cache {
  void *k;        /* [B][Hkv][capacity][D] kv_dtype */
  void *v;        /* [B][Hkv][capacity][D] kv_dtype */
  int32_t *pos;   /* [B][Hkv][capacity] */
  float *imp;     /* [B][Hkv][capacity] cumulative importance ([Blog] Sec. 3 H2O) */
  int32_t *len;   /* [B][Hkv] */
  int32_t *evict; /* the cache's pending-eviction state (see hikv_decode_step): hikv_state_bytes()
                     bytes, 16-byte aligned, zero-filled together with a fresh cache */
} hikv_cache;

#define HIKV_ACC_ALL 0
#define HIKV_ACC_RECENT 1
#define HIKV_ACC_LOGIT 2

#define HIKV_S2V_TOPK 0
#define HIKV_S2V_CHUNK 1

typedef struct hikv_policy {
  const int32_t *budget;   /* [B][Hkv] device per-unit budgets ([HeadKV] Sec. 3.2), or NULL */
  int32_t budget_all;      /* budget of every unit when `budget` is NULL */
  int32_t n_sink;          /* S: positions 0..S-1 are never evicted */
  int32_t n_recent;        /* W: the W' = min(W, budget - S) newest positions are never evicted */
  int32_t stage2_channels; /* r: 0 = Stage II off; else 1..D channels per q-head ([HiKV] Sec. III-C) */
  int32_t stage2_tokens;   /* k_T >= 1: tokens in Stage II's exact softmax (used when r > 0) */
  const int32_t *len_hint; /* optional HOST copy of len[] as it is before this call, or NULL.
                              With at most 64 units the split-K tile plan is then computed on
                              the host and passed with the launch, which saves the kernels a
                              dependent device-memory round trip.  On the Stage II path with
                              budget == NULL, a hint under which no unit ends more than one
                              token over budget_all also leaves out the bulk-eviction launch.
                              A hint with len + 1 >
                              capacity or len < 0 is rejected (HIKV_EINVAL); a hint that
                              disagrees with the device's len[] sets HIKV_EINVAL in the
                              device status and that call's results are undefined. */
  const int32_t *budget_hint; /* optional HOST copy of budget[] (used with len_hint when budget
                              is not NULL), or NULL.  With both copies the host can tell a step
                              that cuts a unit by more than one token (the first step after a
                              prefill): the survivors' rows are then moved by a launch of many
                              workgroups per unit instead of one.  Results never depend on it. */
  int32_t accumulate;      /* which tokens a step's attention probabilities are added to:
                              HIKV_ACC_ALL: every live token (H2O's cumulative score).
                              HIKV_ACC_RECENT: only the W' newest positions (the window that
                              eviction protects); older tokens keep a frozen score.  With
                              n_sink 0 and n_recent = budget/2 this is HiKV's dual bank
                              ([HiKV] Sec. III-B): the window is the recent bank, the rest the
                              important bank, each score sums the W' probabilities a token
                              received from its own step on, and a token leaving the window
                              displaces the bank's lowest score iff its own is higher.
                              HIKV_ACC_LOGIT: every live token gains the pre-softmax logit
                              scale * q.k it gets from the group's q-heads ([Kelle] Sec. 4.1
                              Eq. 3 and Sec. 5.3: attention scores summed without the
                              softmax); with Stage II on, the reduced logit.  Scores can be
                              negative.  Any other value is HIKV_EINVAL. */
  int32_t stage2_v;        /* Stage II's V side (used when r > 0):
                              HIKV_S2V_TOPK: the k_T tokens with the largest reduced logit get
                              an exact full-channel softmax, renormalised over them, and P.V.
                              HIKV_S2V_CHUNK: [HiKV] Sec. III-C and Algorithm 1 literally: the
                              reduced-logit probabilities P of the live tokens, in position
                              order, are cut into chunks of D tokens (the last one shorter);
                              each chunk keeps its r largest entries (ties: lower position) and
                              the output is the sum of those entries times their V rows, not
                              renormalised (stage2_tokens is not used).  The position order is
                              found once per unit and step with a bitmap over windows of 2^18
                              positions: len * ceil(position span / 2^18) work per unit (one
                              pass while the live positions span at most 262144).  Any other
                              value is HIKV_EINVAL. */
  int32_t block_tokens;    /* eviction granularity ([Blog] Sec. 5, PagedAttention block
                              fragmentation): 0 or 1, single tokens; P in
                              2..HIKV_MAX_BLOCK_TOKENS, whole blocks of P consecutive positions
                              (block id = pos / P; positions >= 0).  A block holding a
                              protected token is kept whole; the others are ranked by the sum
                              of their tokens' importance and evicted lowest first (equal sums:
                              the higher block id first) while more than the budget's tokens
                              are live, so a unit can end below its budget, or above it when
                              protected blocks hold more tokens (the capacity must then hold
                              budget + 2 P).  Every eviction is a bulk cut; none is left
                              pending.  Stage I with the default launch sequence only
                              (stage2_channels > 0 or HIKV_PATH_MULTI_LAUNCH: HIKV_EUNSUPPORTED,
                              as for hikv_evict); other values are HIKV_EINVAL. */
} hikv_policy;

#define HIKV_MAX_BLOCK_TOKENS 1024

/* Optional outputs of hikv_decode_step for tests, inspection and profiling;
 * every field may be NULL. */
typedef struct hikv_debug {
  int32_t *sel_channels;   /* [B][Hq][r] Stage II chosen channels, ascending (device) */
  int32_t *sel_tokens;     /* [B][Hq][k_T] positions of the exact-softmax tokens, ascending, -1 padded
                              (device; not written with HIKV_S2V_CHUNK) */
  int32_t *sel_count;      /* [B][Hq] number of exact-softmax tokens, min(k_T, len + 1); with
                              HIKV_S2V_CHUNK the tokens kept over all chunks (device) */
  void *attend_start;      /* hipEvents (both or neither; caller-owned) that the dispatch of the step's */
  void *attend_stop;       /* attention launch records when it starts and ends executing (Stage I: the
                              launch over every live K and V row; Stage II: the reduced-channel logits
                              pass over every live K row) */
  int32_t stage1_path;     /* launch sequence: HIKV_PATH_AUTO (the library's choice) or
                              HIKV_PATH_MULTI_LAUNCH (Stage I: settle, attention tiles, combine,
                              accumulate and bulk eviction as separate launches; Stage II: channel
                              select, reduced-logit tiles, selection and exact pass, accumulate
                              and bulk eviction; both evicting in place; kept to compare
                              against).  Results are the same on every path.  Any other value is
                              HIKV_EINVAL. */
} hikv_debug;

#define HIKV_PATH_AUTO 0
#define HIKV_PATH_MULTI_LAUNCH 1

/* Bytes of hikv_cache.evict for this shape (a few words per unit).  0 on a
 * bad shape. */
size_t hikv_state_bytes(const hikv_shape *shape);

/* Bytes of device workspace the decode step and hikv_evict need for this
 * shape and policy.  The workspace must be zero-filled before its first use;
 * the library leaves it ready for the next call.  It holds scratch only (and
 * the status word): one workspace serves every cache of the shape, for calls
 * ordered on one stream.  0 on a bad shape. */
size_t hikv_workspace_bytes(const hikv_shape *shape, const hikv_policy *policy);

/* One decode step for every unit ([HiKV] Algorithm 1 with [Blog] Sec. 3 H2O
 * eviction; cfg. [Kelle] Sec. 4.1):
 *   1. append: slot len[u] <- (k_new[b][j], v_new[b][j]), pos = new_pos[b],
 *      importance 0; len[u] += 1;
 *   2. for every q-head h of KV head j: out[b][h] = softmax(scale * q.K^T) V
 *      over the live slots (the new token attends to itself);
 *      Stage II (r > 0): the logits use only the r channels of largest |q_d|
 *      (ties: lower channel); out = exact full-D softmax restricted to the
 *      k_T tokens with the largest reduced logit (ties: lower position);
 *   3. imp[slot] += sum over the group's q-heads of the slot's probability
 *      (Stage II: the reduced-logit softmax);
 *   4. if len[u] > budget: keep the protected tokens (pos < S or
 *      pos > new_pos[b] - W') and the budget - |protected| other tokens with
 *      the highest (importance, then lower position); compact them into
 *      slots [0, budget); len[u] = budget.
 * Pending eviction (Stage I, r == 0; and Stage II with the exact top-k_T V
 * side for bf16 K and V with D = 128 and k_T <= 2048, which runs in the same
 * two launches): when step 4 evicts exactly one token,
 * the call leaves the choice of the victim to the next call and does not
 * compact: len[u] stays budget + 1, and one of those slots, the victim, is
 * dead (its row, position and importance are stale); the choice is kept in
 * cache->evict.  The next decode step
 * neither attends to it nor counts it, and writes its new token there; a bulk
 * cut (more than one token over budget) removes it first.  hikv_settle()
 * resolves it (the cache then holds exactly the kept set, as in step 4) and
 * hikv_pending() reports the dead slot without changing anything; the other
 * Stage II variants and hikv_evict() settle first and evict in place.
 * Results (out, the kept set once settled) are those of step 4 in every case.  A unit whose budget + 2
 * exceeds the capacity therefore runs out of slots (HIKV_ECAPACITY) one call
 * after it reaches its budget.
 * q: [B][Hq][D]; k_new, v_new: [B][Hkv][D]; new_pos: [B] int32;
 * out: [B][Hq][D] float32.  `debug` may be NULL. */
int hikv_decode_step(const hikv_shape *shape, const hikv_cache *cache, const hikv_policy *policy,
                     const void *q, const void *k_new, const void *v_new,
                     const int32_t *new_pos, float *out, void *ws, size_t ws_bytes,
                     const hikv_debug *debug, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid it): hikv_decode_step
 * with the workspace taken from a static array the library holds on each GPU
 * (HIKV_STATIC_SCRATCH_BYTES, allocated with the library's code on that GPU
 * and held until the process ends) instead of a caller's buffer.  Nothing is
 * allocated or freed.  The call is rejected with HIKV_EINVAL when
 * hikv_workspace_bytes(shape, policy) exceeds HIKV_STATIC_SCRATCH_BYTES.
 * Device-side errors are recorded in *status (a caller-owned device int32,
 * sticky like the workspace's status word: zero it before the first call and
 * after reading a nonzero value).  Every call on one GPU uses that GPU's one
 * array: calls that overlap in time on one GPU (different streams, or host
 * threads enqueueing concurrently) race and must not be made; calls ordered
 * on one stream are safe, whatever their shapes.  The scratch keeps the last
 * call's contents; the call clears what must start at zero itself.  Results
 * are those of hikv_decode_step on the same inputs. */
#define HIKV_STATIC_SCRATCH_BYTES (128u << 20)
int hikv_decode_step_static(const hikv_shape *shape, const hikv_cache *cache, const hikv_policy *policy,
                            const void *q, const void *k_new, const void *v_new,
                            const int32_t *new_pos, float *out, int32_t *status,
                            const hikv_debug *debug, void *stream);

/* Compress every unit over its budget to exactly its budget with step 4 of
 * hikv_decode_step, using the current importance; newest_pos[b] anchors the
 * recent window ([Blog] Sec. 3 H2O; [Kelle] Sec. 4.1, prefill eviction).
 * A pending eviction is settled first. */
int hikv_evict(const hikv_shape *shape, const hikv_cache *cache, const hikv_policy *policy,
               const int32_t *newest_pos, void *ws, size_t ws_bytes, void *stream);

/* Resolve every unit's pending eviction (see hikv_decode_step): the unit's
 * last slot moves into the dead one (K and V rows, position, importance) and
 * len[u] drops by one, which is the in-place compaction of step 4 ([Kelle]
 * Sec. 2.2: slot order does not matter).  Units with none pending are left
 * alone.  `policy` and `ws` are those of the decode steps on this cache.
 * The pending state is part of the cache, so it stays with the cache across
 * workspaces.
 * Call it before reading the cache directly or handing it to
 * hikv_prefill_scores(). */
int hikv_settle(const hikv_shape *shape, const hikv_cache *cache, const hikv_policy *policy,
                void *ws, size_t ws_bytes, void *stream);

/* Write each unit's dead slot (-1 when no eviction is pending) to slot_out
 * ([B][Hkv] int32, device) without changing the cache or the workspace. */
int hikv_pending(const hikv_shape *shape, const hikv_cache *cache, const hikv_policy *policy,
                 const void *ws, size_t ws_bytes, int32_t *slot_out, void *stream);

/* Workspace bytes hikv_prefill_scores needs for n_obs observation queries. */
size_t hikv_prefill_workspace_bytes(const hikv_shape *shape, int32_t n_obs);

/* Add prompt-side importance ([Kelle] Sec. 4.1 prefill: column sums of the
 * prompt's attention; [HiKV] Sec. III-B/III-D: the windowed sum).  For every
 * observation query i at position q_pos[b][i] and every q-head of a KV group,
 * the causal softmax row over the unit's live tokens with pos <= q_pos is
 * formed; a token's share is added to its importance when window == 0, or
 * when 0 <= q_pos - pos < window.  q_obs: [B][Hq][n_obs][D]; q_pos: [B][n_obs].
 * pool > 1 applies SnapKV's 1-D max pooling ([Blog] SnapKV section): the
 * token at position p adds the largest of this call's scores over the live
 * positions p .. p+pool-1 instead of its own (0 or 1: no pooling).
 * Positions of a unit must be distinct.  bf16 caches run on the matrix cores
 * (capacity and n_obs at most 2^21: HIKV_EUNSUPPORTED beyond); fp32 caches
 * on the vector ALUs.  window < 0, pool < 0 or n_obs < 0: HIKV_EINVAL. */
int hikv_prefill_scores(const hikv_shape *shape, const hikv_cache *cache, const void *q_obs,
                        const int32_t *q_pos, int32_t n_obs, int32_t window, int32_t pool, void *ws,
                        size_t ws_bytes, void *stream);

/* Synchronise `stream`, return the first device-side error recorded in `ws`
 * since it was last cleared (HIKV_OK if none), and clear it when `clear`. */
int hikv_device_status(void *ws, int clear, void *stream);

/* Static description of a status code. */
const char *hikv_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif
