// hikv_launch.h -- host-side launchers of the HIP kernels (internal).
#pragma once

#include "hikv_common.h"

namespace hikv {

// Split-K decode attention over the live slots of every unit (append
// included).  with_v=false: logits + softmax statistics only (Stage II's
// reduced-channel pass).  ev0/ev1 (may be null): events recorded around it.
hipError_t launch_attn_tiles(const StepArgs &a, int dtype, bool with_v, bool masked,
                             hipStream_t s, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
// Per (unit, q-head): merge tile partials; write out (when with_v) and stats.
hipError_t launch_combine(const StepArgs &a, bool with_v, hipStream_t s);
// Per tile: importance += probabilities; steady-state single eviction.
hipError_t launch_accumulate(const StepArgs &a, int dtype, hipStream_t s);
// Per unit: radix-select eviction of every token over budget + compaction.
// newest = new_pos (decode) or newest_pos (hikv_evict); from_decode selects
// which units are eligible (those the decode step processed).
hipError_t launch_bulk_evict(const StepArgs &a, int dtype, const int32_t *newest,
                             bool from_decode, hipStream_t s);

// The Stage I step in two launches (attention tiles, then statistics,
// output, importance and eviction).
// ev0/ev1 (may be null): events recorded around the attention launch.
hipError_t launch_step(const StepArgs &a, int dtype, hipStream_t s, hipEvent_t ev0 = nullptr,
                       hipEvent_t ev1 = nullptr);
// The pending eviction a two-launch step leaves: its slot per unit to
// slot_out (device [n_units], may be null; -1 when none) and, with apply, the
// unit compacted as if evicted in place.
hipError_t launch_settle(const StepArgs &a, int dtype, int32_t *slot_out, bool apply, hipStream_t s);
// Host-side tile plan from a host copy of len[] (fills a.hp); false when it
// does not apply (too many units), in which case the kernels derive it.
bool step_host_plan(StepArgs &a, int dtype, const int32_t *len_hint);

// Stage II.
hipError_t launch_stage2_channels(const StepArgs &a, int dtype, hipStream_t s);
hipError_t launch_stage2_exact(const StepArgs &a, int dtype, hipStream_t s);
hipError_t launch_chunk_pv(const StepArgs &a, int dtype, hipStream_t s);
// The position order of the units a block-granular eviction cuts (ws.order).
hipError_t launch_pos_rank(const StepArgs &a, hipStream_t s);

// Prefill scores.
struct PrefillArgs {
  int B, Hq, Hkv, D, cap, G, n_units, n_obs, window, pool;
  float scale_log2;
  const void *k_cache;
  const int32_t *pos;
  float *imp;
  const int32_t *len;
  const void *q_obs;
  const int32_t *q_pos;
  float *stats;       // [U][G][n_obs][2]
  int32_t *krange;    // [U][ceil(cap/64)][2] lowest, highest position of each 64-slot tile
  int32_t *qrange;    // [B][ceil(n_obs/64)][2] lowest, highest position of each 64-query tile
  float *padd;        // [U][cap] this call's score per slot (pooling only)
  int32_t *pord;      // [U][cap] slots in position order (pooling only)
  int32_t *prank;     // [U][cap] each slot's rank in that order (pooling only)
  int32_t *status;
};
hipError_t launch_prefill(const PrefillArgs &p, int dtype, hipStream_t s);

}  // namespace hikv
