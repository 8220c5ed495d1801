// api.hip -- the C ABI (include/hikv.h): argument checks, workspace carving
// and the launch sequence of each entry point.  All launches go to the
// caller's stream; nothing here allocates, synchronises or memsets (except
// hikv_device_status, which is documented to synchronise).

#include <math.h>
#include <string.h>

#include <atomic>

#include "hikv_launch.h"

using namespace hikv;

// The allocation-free entry point's scratch (hikv_decode_step_static): one
// array per GPU the library runs on, held until the process ends.  Host code
// never uses the array's name as an address: each device's address is looked
// up once, with that device current, and kept (scratch_of_current_device).
static __device__ __attribute__((aligned(256))) char scratch[HIKV_STATIC_SCRATCH_BYTES];

namespace {

// gfx950 check, once per device.
int arch_ok() {
  static int cache[64];  // 0 unknown, 1 ok, -1 not gfx950
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return HIKV_EDEVICE;
  if (dev < 0 || dev >= 64) return HIKV_EUNSUPPORTED;
  if (cache[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return HIKV_EDEVICE;
    cache[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  return cache[dev] == 1 ? HIKV_OK : HIKV_EUNSUPPORTED;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(const hikv_shape *s) {
  if (!s) return HIKV_EINVAL;
  if (s->batch < 0 || s->n_kv_heads < 1 || s->n_q_heads < 1 || s->capacity < 1) return HIKV_EINVAL;
  if (s->n_q_heads % s->n_kv_heads) return HIKV_EINVAL;
  if (s->kv_dtype != HIKV_F32 && s->kv_dtype != HIKV_BF16) return HIKV_EINVAL;
  const int G = s->n_q_heads / s->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return HIKV_EUNSUPPORTED;
  if (s->head_dim != 64 && s->head_dim != 128) return HIKV_EUNSUPPORTED;
  if ((long long)s->batch * s->n_kv_heads > kMaxUnits) return HIKV_EUNSUPPORTED;
  return HIKV_OK;
}

int check_policy(const hikv_shape *s, const hikv_policy *p) {
  if (!p) return HIKV_EINVAL;
  if (p->n_sink < 0 || p->n_recent < 0) return HIKV_EINVAL;
  if (p->accumulate != HIKV_ACC_ALL && p->accumulate != HIKV_ACC_RECENT && p->accumulate != HIKV_ACC_LOGIT)
    return HIKV_EINVAL;
  if (p->stage2_channels < 0 || p->stage2_channels > s->head_dim) return HIKV_EINVAL;
  if (p->stage2_v != HIKV_S2V_TOPK && p->stage2_v != HIKV_S2V_CHUNK) return HIKV_EINVAL;
  if (p->stage2_channels > 0 && p->stage2_v == HIKV_S2V_TOPK && p->stage2_tokens < 1) return HIKV_EINVAL;
  if (p->block_tokens < 0 || p->block_tokens > HIKV_MAX_BLOCK_TOKENS) return HIKV_EINVAL;
  return HIKV_OK;
}

int check_cache(const hikv_cache *c) {
  if (!c || !c->k || !c->v || !c->pos || !c->imp || !c->len || !c->evict) return HIKV_EINVAL;
  if (!aligned16(c->k) || !aligned16(c->v) || !aligned16(c->evict)) return HIKV_EINVAL;
  return HIKV_OK;
}

WsSizes sizes_for(const hikv_shape *s, const hikv_policy *p) {
  const bool chunks = p && p->stage2_channels > 0 && p->stage2_v == HIKV_S2V_CHUNK;
  const int kT = (p && p->stage2_channels > 0 && !chunks) ? p->stage2_tokens : 0;  // 0: no exact top-k_T pass
  const bool blocks = p && p->block_tokens >= 2;
  return ws_sizes(s->batch, s->n_q_heads, s->n_kv_heads, s->head_dim, s->capacity, kT, chunks, chunks || blocks);
}

StepArgs make_args(const hikv_shape *s, const hikv_cache *c, const hikv_policy *p, const Ws &ws) {
  StepArgs a;
  memset(&a, 0, sizeof a);
  a.B = s->batch;
  a.Hq = s->n_q_heads;
  a.Hkv = s->n_kv_heads;
  a.D = s->head_dim;
  a.cap = s->capacity;
  a.G = s->n_q_heads / s->n_kv_heads;
  a.n_units = s->batch * s->n_kv_heads;
  const double scale = s->scale > 0.f ? (double)s->scale : 1.0 / sqrt((double)s->head_dim);
  a.scale_log2 = (float)(scale * 1.4426950408889634);
  a.k_cache = c->k;
  a.v_cache = c->v;
  a.k_w = c->k;
  a.v_w = c->v;
  a.pos = c->pos;
  a.imp = c->imp;
  a.len = c->len;
  a.evict = c->evict;
  a.budget = p->budget;
  a.budget_all = p->budget_all;
  a.n_sink = p->n_sink;
  a.n_recent = p->n_recent;
  a.acc_recent = p->accumulate == HIKV_ACC_RECENT;
  a.acc_logit = p->accumulate == HIKV_ACC_LOGIT;
  a.r = p->stage2_channels;
  a.s2_chunks = p->stage2_channels > 0 && p->stage2_v == HIKV_S2V_CHUNK;
  a.kT = (p->stage2_channels > 0 && !a.s2_chunks) ? p->stage2_tokens : 0;
  a.block = p->block_tokens >= 2 ? p->block_tokens : 0;
  a.ws = ws;
  return a;
}

inline int dev_err(hipError_t e) { return e == hipSuccess ? HIKV_OK : HIKV_EDEVICE; }

}  // namespace

extern "C" size_t hikv_state_bytes(const hikv_shape *shape) {
  if (check_shape(shape) != HIKV_OK) return 0;
  return sizeof(int32_t) * (size_t)shape->batch * shape->n_kv_heads * (size_t)state_words(shape->capacity);
}

extern "C" size_t hikv_workspace_bytes(const hikv_shape *shape, const hikv_policy *policy) {
  if (check_shape(shape) != HIKV_OK) return 0;
  if (policy && check_policy(shape, policy) != HIKV_OK) return 0;
  return sizes_for(shape, policy).total;
}

namespace {

// Host checks shared by the decode entry points (everything but the workspace).
int check_decode_args(const hikv_shape *shape, const hikv_cache *cache, const hikv_policy *policy,
                      const void *q, const void *k_new, const void *v_new, const int32_t *new_pos,
                      const float *out, const hikv_debug *debug) {
  int st = check_shape(shape);
  if (st != HIKV_OK) return st;
  if ((st = check_policy(shape, policy)) != HIKV_OK) return st;
  if (shape->batch == 0) return HIKV_OK;
  if ((st = check_cache(cache)) != HIKV_OK) return st;
  if (!q || !k_new || !v_new || !new_pos || !out) return HIKV_EINVAL;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new)) return HIKV_EINVAL;
  if (policy->len_hint) {
    const int U = shape->batch * shape->n_kv_heads;
    for (int u = 0; u < U; ++u)
      if (policy->len_hint[u] < 0 || policy->len_hint[u] + 1 > shape->capacity) return HIKV_EINVAL;
  }
  const int path = debug ? debug->stage1_path : HIKV_PATH_AUTO;
  if (path != HIKV_PATH_AUTO && path != HIKV_PATH_MULTI_LAUNCH) return HIKV_EINVAL;
  return HIKV_OK;
}

// The move launch of a bulk cut from the host's bound on each unit's moves
// (mvr): one workgroup per bulk_moves_per_wg moves of each unit, listed in
// a.hp.mvb, when the host plan covers every unit; else one row of workgroups
// per unit, sized for the largest bound.
void moves_plan(StepArgs &a, const int32_t *mvr, int dtype) {
  a.moves_flat = 0;
  if (!a.bulk_split || a.hp.n != a.n_units || a.n_units > kHostPlanUnits) return;
  const int per = bulk_moves_per_wg(a.D * (dtype == HIKV_BF16 ? 2 : 4));
  int base = 0;
  for (int u = 0; u < a.n_units; ++u) {
    a.hp.mvb[u] = base;
    base += (mvr[u] + per - 1) / per;
  }
  a.hp.mvb[a.n_units] = base;
  a.moves_flat = base > 0 ? 1 : 0;
}

__global__ void k_zero_words(int32_t *p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// The launch sequence of one decode step on a carved workspace.  clear_tickets:
// zero the per-unit counters first (a workspace whose previous contents are
// not this shape's own, before a path that counts tiles).
int run_decode(const hikv_shape *shape, const hikv_cache *cache, const hikv_policy *policy, const void *q,
               const void *k_new, const void *v_new, const int32_t *new_pos, float *out, const Ws &w,
               const hikv_debug *debug, void *stream, bool clear_tickets) {
  const int path = debug ? debug->stage1_path : HIKV_PATH_AUTO;
  StepArgs a = make_args(shape, cache, policy, w);
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_pos = new_pos;
  a.out = out;
  if (debug) {
    a.dbg_channels = debug->sel_channels;
    a.dbg_tokens = debug->sel_tokens;
    a.dbg_count = debug->sel_count;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int dt = shape->kv_dtype;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (debug && debug->attend_start && debug->attend_stop) {
    ev0 = static_cast<hipEvent_t>(debug->attend_start);
    ev1 = static_cast<hipEvent_t>(debug->attend_stop);
  }
  hipError_t e;
  // Block-granular eviction runs on the two-launch Stage I sequence only.
  if (a.block && (a.r > 0 || path == HIKV_PATH_MULTI_LAUNCH)) return HIKV_EUNSUPPORTED;
  if (clear_tickets && (a.r > 0 || path == HIKV_PATH_MULTI_LAUNCH)) {
    hipLaunchKernelGGL(k_zero_words, dim3(1), dim3(256), 0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<int32_t *>(a.ws.ticket), a.n_units);
    if ((e = hipGetLastError()) != hipSuccess) return dev_err(e);
  }
  if (a.r == 0) {
    if (path == HIKV_PATH_AUTO) {
      if (policy->len_hint) step_host_plan(a, dt, policy->len_hint);
      // With host copies of the lengths and budgets, a step that cuts some
      // unit by more than one token moves its survivors in a launch of its own.
      if (policy->len_hint && (!policy->budget || policy->budget_hint)) {
        a.bulk_known = 1;
        const int U = shape->batch * shape->n_kv_heads;
        int32_t mvr[kHostPlanUnits] = {};  // each unit's bound on its moves
        for (int u = 0; u < U; ++u) {
          const int beta = policy->budget ? policy->budget_hint[u] : policy->budget_all;
          const int len = policy->len_hint[u];
          if (a.block) {
            // Every eviction is a bulk cut of whole blocks: at most the
            // excess plus one block (and a dead slot left by a step of
            // single-token eviction) go, so at most that many rows move.
            if (len + 1 > beta) {
              a.bulk_split = 1;
              a.bulk_rows = max(a.bulk_rows, min(len + 1, len + 2 - beta + a.block));
              if (u < kHostPlanUnits) mvr[u] = min(len + 1, len + 2 - beta + a.block);
            }
            continue;
          }
          const int live = len + 1 - (len > beta ? 1 : 0);  // a unit over budget holds a dead slot
          if (live - beta > 1) {
            a.bulk_split = 1;
            // survivors at or above the budget: at most the budget, and at
            // most the len + 1 - beta slots there
            a.bulk_rows = max(a.bulk_rows, min(beta, len + 1 - beta));
            if (u < kHostPlanUnits) mvr[u] = min(beta, len + 1 - beta);
          }
        }
        moves_plan(a, mvr, dt);
      } else if (a.block) {  // any unit may be cut: the cut's launches always run
        a.bulk_split = 1;
        a.bulk_rows = a.cap;
      }
      return dev_err(launch_step(a, dt, s, ev0, ev1));
    }
    // The four-launch path evicts in place: an eviction a two-launch step
    // left pending is resolved first.
    if ((e = launch_settle(a, dt, nullptr, true, s)) != hipSuccess) return dev_err(e);
    if ((e = launch_attn_tiles(a, dt, true, false, s, ev0, ev1)) != hipSuccess) return dev_err(e);
    if ((e = launch_combine(a, true, s)) != hipSuccess) return dev_err(e);
  } else if (!a.s2_chunks && dt == HIKV_BF16 && a.D == 128 && a.kT <= kS2TwoMaxTokens &&
             path == HIKV_PATH_AUTO) {
    // Stage II with the exact top-k_T V side in two launches (like Stage I:
    // an eviction of one token is left pending).  Its bulk cut always leaves
    // the row moves to launches of their own; with the caller's lengths and
    // budgets they are launched only when some unit is cut in bulk.
    a.s2_two = 1;
    if (policy->len_hint) step_host_plan(a, dt, policy->len_hint);
    if (policy->len_hint && (!policy->budget || policy->budget_hint)) {
      a.bulk_known = 1;
      const int U = shape->batch * shape->n_kv_heads;
      int32_t mvr[kHostPlanUnits] = {};
      for (int u = 0; u < U; ++u) {
        const int beta = policy->budget ? policy->budget_hint[u] : policy->budget_all;
        const int len = policy->len_hint[u];
        const int live = len + 1 - (len > beta ? 1 : 0);
        if (live - beta > 1) {
          a.bulk_split = 1;
          a.bulk_rows = max(a.bulk_rows, min(beta, len + 1 - beta));
          if (u < kHostPlanUnits) mvr[u] = min(beta, len + 1 - beta);
        }
      }
      moves_plan(a, mvr, dt);
    } else {
      a.bulk_split = 1;
      a.bulk_rows = a.cap;
    }
    return dev_err(launch_step(a, dt, s, ev0, ev1));
  } else {
    // (the channel-select launch also settles a pending eviction first)
    if ((e = launch_stage2_channels(a, dt, s)) != hipSuccess) return dev_err(e);
    if ((e = launch_attn_tiles(a, dt, false, true, s, ev0, ev1)) != hipSuccess) return dev_err(e);
    // (no combine launch: the launches that need the unit statistics take
    // them from the tiles' partials themselves)
    if (a.s2_chunks) {
      if ((e = launch_chunk_pv(a, dt, s)) != hipSuccess) return dev_err(e);
    } else {
      if ((e = launch_stage2_exact(a, dt, s)) != hipSuccess) return dev_err(e);  // selection + exact pass
    }
  }
  // With the caller's lengths and one budget for every unit, the host knows
  // whether any unit ends more than one token over budget; if none does, the
  // bulk-eviction launch has nothing to do and is left out.
  if (policy->len_hint && !policy->budget) {
    a.no_bulk = 1;
    const int U = shape->batch * shape->n_kv_heads;
    for (int u = 0; u < U; ++u)
      if (policy->len_hint[u] + 1 - policy->budget_all > 1) a.no_bulk = 0;
  }
  if ((e = launch_accumulate(a, dt, s)) != hipSuccess) return dev_err(e);
  if (!a.no_bulk && (e = launch_bulk_evict(a, dt, new_pos, true, s)) != hipSuccess) return dev_err(e);
  return HIKV_OK;
}

std::atomic<void *> scratch_ptr[64];  // each device's address of `scratch` (below)

int scratch_of_current_device(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return HIKV_EDEVICE;
  if (dev < 0 || dev >= 64) return HIKV_EUNSUPPORTED;
  void *p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HIKV_EDEVICE;
    scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return HIKV_OK;
}

}  // namespace

extern "C" int hikv_decode_step(const hikv_shape *shape, const hikv_cache *cache,
                                const hikv_policy *policy, const void *q, const void *k_new,
                                const void *v_new, const int32_t *new_pos, float *out, void *ws,
                                size_t ws_bytes, const hikv_debug *debug, void *stream) {
  int st = check_decode_args(shape, cache, policy, q, k_new, v_new, new_pos, out, debug);
  if (st != HIKV_OK || shape->batch == 0) return st;
  if (!ws || !aligned16(ws)) return HIKV_EINVAL;
  const WsSizes sz = sizes_for(shape, policy);
  if (ws_bytes < sz.total) return HIKV_EINVAL;
  if ((st = arch_ok()) != HIKV_OK) return st;
  return run_decode(shape, cache, policy, q, k_new, v_new, new_pos, out, ws_carve(ws, sz), debug, stream, false);
}

extern "C" int hikv_decode_step_static(const hikv_shape *shape, const hikv_cache *cache,
                                       const hikv_policy *policy, const void *q, const void *k_new,
                                       const void *v_new, const int32_t *new_pos, float *out,
                                       int32_t *status, const hikv_debug *debug, void *stream) {
  int st = check_decode_args(shape, cache, policy, q, k_new, v_new, new_pos, out, debug);
  if (st != HIKV_OK || shape->batch == 0) return st;
  if (!status || (reinterpret_cast<uintptr_t>(status) & 3u)) return HIKV_EINVAL;
  const WsSizes sz = sizes_for(shape, policy);
  if (sz.total > (size_t)HIKV_STATIC_SCRATCH_BYTES) return HIKV_EINVAL;
  if ((st = arch_ok()) != HIKV_OK) return st;
  void *base = nullptr;
  if ((st = scratch_of_current_device(&base)) != HIKV_OK) return st;
  Ws w = ws_carve(base, sz);
  w.status = status;  // device-side errors go to the caller's word
  return run_decode(shape, cache, policy, q, k_new, v_new, new_pos, out, w, debug, stream, true);
}

extern "C" int hikv_evict(const hikv_shape *shape, const hikv_cache *cache,
                          const hikv_policy *policy, const int32_t *newest_pos, void *ws,
                          size_t ws_bytes, void *stream) {
  int st = check_shape(shape);
  if (st != HIKV_OK) return st;
  if ((st = check_policy(shape, policy)) != HIKV_OK) return st;
  if (shape->batch == 0) return HIKV_OK;
  if ((st = check_cache(cache)) != HIKV_OK) return st;
  if (!newest_pos || !ws || !aligned16(ws)) return HIKV_EINVAL;
  if (policy->block_tokens >= 2) return HIKV_EUNSUPPORTED;  // block-granular eviction: decode steps only
  const WsSizes sz = sizes_for(shape, policy);
  if (ws_bytes < sz.total) return HIKV_EINVAL;
  if ((st = arch_ok()) != HIKV_OK) return st;
  StepArgs a = make_args(shape, cache, policy, ws_carve(ws, sz));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_settle(a, shape->kv_dtype, nullptr, true, s);
  if (e != hipSuccess) return dev_err(e);
  return dev_err(launch_bulk_evict(a, shape->kv_dtype, newest_pos, false, s));
}

namespace {
int settle_common(const hikv_shape *shape, const hikv_cache *cache, const hikv_policy *policy,
                  const void *ws, size_t ws_bytes, int32_t *slot_out, bool apply, void *stream) {
  int st = check_shape(shape);
  if (st != HIKV_OK) return st;
  if ((st = check_policy(shape, policy)) != HIKV_OK) return st;
  if (shape->batch == 0) return HIKV_OK;
  if ((st = check_cache(cache)) != HIKV_OK) return st;
  if (!ws || !aligned16(ws) || (!apply && !slot_out)) return HIKV_EINVAL;
  const WsSizes sz = sizes_for(shape, policy);
  if (ws_bytes < sz.total) return HIKV_EINVAL;
  if ((st = arch_ok()) != HIKV_OK) return st;
  StepArgs a = make_args(shape, cache, policy, ws_carve(const_cast<void *>(ws), sz));
  return dev_err(launch_settle(a, shape->kv_dtype, slot_out, apply, static_cast<hipStream_t>(stream)));
}
}  // namespace

extern "C" int hikv_settle(const hikv_shape *shape, const hikv_cache *cache, const hikv_policy *policy,
                           void *ws, size_t ws_bytes, void *stream) {
  return settle_common(shape, cache, policy, ws, ws_bytes, nullptr, true, stream);
}

extern "C" int hikv_pending(const hikv_shape *shape, const hikv_cache *cache, const hikv_policy *policy,
                            const void *ws, size_t ws_bytes, int32_t *slot_out, void *stream) {
  return settle_common(shape, cache, policy, ws, ws_bytes, slot_out, false, stream);
}

extern "C" size_t hikv_prefill_workspace_bytes(const hikv_shape *shape, int32_t n_obs) {
  if (check_shape(shape) != HIKV_OK || n_obs < 0) return 0;
  const size_t U = (size_t)shape->batch * shape->n_kv_heads;
  const size_t G = (size_t)(shape->n_q_heads / shape->n_kv_heads);
  const size_t nobs = n_obs > 0 ? (size_t)n_obs : 1;
  const size_t nkt = ((size_t)shape->capacity + 63) / 64, nqt = (nobs + 63) / 64;
  return 256 + align256(sizeof(float) * U * G * nobs * 2) + align256(sizeof(int32_t) * U * nkt * 2) +
         align256(sizeof(int32_t) * (size_t)shape->batch * nqt * 2) +
         3 * align256(sizeof(int32_t) * U * (size_t)shape->capacity);
}

extern "C" int hikv_prefill_scores(const hikv_shape *shape, const hikv_cache *cache,
                                   const void *q_obs, const int32_t *q_pos, int32_t n_obs,
                                   int32_t window, int32_t pool, void *ws, size_t ws_bytes,
                                   void *stream) {
  int st = check_shape(shape);
  if (st != HIKV_OK) return st;
  if (n_obs < 0 || window < 0 || pool < 0) return HIKV_EINVAL;
  if (shape->batch == 0 || n_obs == 0) return HIKV_OK;
  if ((st = check_cache(cache)) != HIKV_OK) return st;
  if (!q_obs || !q_pos || !ws || !aligned16(q_obs) || !aligned16(ws)) return HIKV_EINVAL;
  if (ws_bytes < hikv_prefill_workspace_bytes(shape, n_obs)) return HIKV_EINVAL;
  // the matrix-core passes track at most 32768 tiles of 64 (keys or queries)
  if (shape->kv_dtype == HIKV_BF16 && ((long long)shape->capacity > 32768LL * 64 || (long long)n_obs > 32768LL * 64))
    return HIKV_EUNSUPPORTED;
  if ((st = arch_ok()) != HIKV_OK) return st;
  PrefillArgs p;
  memset(&p, 0, sizeof p);
  p.B = shape->batch;
  p.Hq = shape->n_q_heads;
  p.Hkv = shape->n_kv_heads;
  p.D = shape->head_dim;
  p.cap = shape->capacity;
  p.G = p.Hq / p.Hkv;
  p.n_units = p.B * p.Hkv;
  p.n_obs = n_obs;
  p.window = window;
  p.pool = pool;
  const double scale = shape->scale > 0.f ? (double)shape->scale : 1.0 / sqrt((double)shape->head_dim);
  p.scale_log2 = (float)(scale * 1.4426950408889634);
  p.k_cache = cache->k;
  p.pos = cache->pos;
  p.imp = cache->imp;
  p.len = cache->len;
  p.q_obs = q_obs;
  p.q_pos = q_pos;
  p.status = static_cast<int32_t *>(ws);
  p.stats = reinterpret_cast<float *>(static_cast<char *>(ws) + 256);
  {
    const size_t U = (size_t)p.n_units, nkt = ((size_t)p.cap + 63) / 64;
    char *r = static_cast<char *>(ws) + 256 + align256(sizeof(float) * U * p.G * (size_t)n_obs * 2);
    p.krange = reinterpret_cast<int32_t *>(r);
    r += align256(sizeof(int32_t) * U * nkt * 2);
    p.qrange = reinterpret_cast<int32_t *>(r);
    r += align256(sizeof(int32_t) * (size_t)p.B * (((size_t)n_obs + 63) / 64) * 2);
    const size_t per = align256(sizeof(int32_t) * U * (size_t)p.cap);
    p.padd = reinterpret_cast<float *>(r);
    p.pord = reinterpret_cast<int32_t *>(r + per);
    p.prank = reinterpret_cast<int32_t *>(r + 2 * per);
  }
  return dev_err(launch_prefill(p, shape->kv_dtype, static_cast<hipStream_t>(stream)));
}

extern "C" int hikv_device_status(void *ws, int clear, void *stream) {
  if (!ws) return HIKV_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(s) != hipSuccess) return HIKV_EDEVICE;
  int32_t v = 0;
  if (hipMemcpy(&v, ws, sizeof v, hipMemcpyDeviceToHost) != hipSuccess) return HIKV_EDEVICE;
  if (clear && v != 0) {
    const int32_t z = 0;
    if (hipMemcpy(ws, &z, sizeof z, hipMemcpyHostToDevice) != hipSuccess) return HIKV_EDEVICE;
  }
  return v;
}

extern "C" const char *hikv_status_string(int status) {
  switch (status) {
    case HIKV_OK: return "ok";
    case HIKV_EINVAL: return "invalid argument";
    case HIKV_EUNSUPPORTED: return "unsupported shape or device";
    case HIKV_EDEVICE: return "HIP runtime or launch failure";
    case HIKV_ECAPACITY: return "cache capacity exceeded";
    case HIKV_EBUDGET: return "budget below sink count or above capacity";
    default: return "unknown status";
  }
}
