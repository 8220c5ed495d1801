// hikv_common.h -- device helpers and the workspace layout shared by the HIP
// kernels of the importance-aware KV decode library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hikv.h"

namespace hikv {

constexpr int kWave = 64;
constexpr int kMaxUnits = 4096;     // (batch, KV head) units per call
constexpr int kTileMin = 64;        // smallest split-K tile, tokens
constexpr int kTilesTarget = 512;   // split-K tiles aimed for per step (2 per CU)
constexpr int kMaxGrid = 2048;      // upper bound on resident workgroups (256 CUs x 8)
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kImpChunk = 2048;     // tokens per importance block of the step's second launch

// Importance blocks per unit in the step's second launch.
__host__ __device__ inline int imp_blocks(int cap) { return (cap + kImpChunk - 1) / kImpChunk; }

// Per-unit record of the cache's pending eviction (hikv_cache.evict), in
// int32 words: [0] the number n of candidates (0: none pending), [1] the dead
// slot as the attention launch of the current step found it, then from word 4
// one 4-word candidate per importance block of the step that left it: the
// block's lowest eviction key (low, high word) and that key's slot.
__host__ __device__ inline int state_words(int cap) { return 4 * (imp_blocks(cap) + 1); }

// ---------------------------------------------------------------------------
// Workspace layout.  Offsets are 256-byte aligned; everything is derived from
// the shape and policy alone, so the host can size it without the device.
// Scratch only (and a sticky status word): one workspace can serve every
// cache of one shape, call after call on one stream.
// ---------------------------------------------------------------------------
struct Ws {
  int32_t *status;      // [1] sticky first device-side error
  int32_t *tinfo;       // [max_tiles][4] per-tile record from the attention launch
  float *fz_newimp;     // [n_units] the new token's importance this step
  uint32_t *ticket;     // [n_units] last-tile-arrives counters (self-resetting)
  int32_t *plan;        // [n_units + 4]: tile base per unit (exclusive prefix), then
                        //   [n_units] = total tiles, [+1] = tile size T
  float *stats;         // [n_units][G][2] softmax max and sum per q-head (multi-kernel path)
  float *part_ml;       // [max_tiles][G][2] per-tile partial max / sum
  float *part_acc;      // [max_tiles][G][D] per-tile partial P.V (unnormalised)
  float *logits;        // [n_units][cap][G] this step's logits: scaled, log2 domain (multi-kernel
                        //   and Stage II paths) or raw q.k (two-launch step; maxima raw too)
  uint64_t *tile_key;   // [max_tiles] lowest eviction key per tile
  int32_t *tile_slot;   // [max_tiles] its slot
  int32_t *holes;       // [n_units][cap] bulk compaction: evicted slots below budget
  int32_t *movers;      // [n_units][cap] bulk compaction: survivors at/above budget
  uint32_t *chmask;     // [B*Hq][D/32] Stage II channel mask
  int32_t *tsel;        // [B*Hq][k_T] Stage II exact-softmax slots
  int32_t *tcount;      // [B*Hq]
  int32_t *urec;        // [n_units][4] per-unit plan of the step: first tile, tiles, tokens
  uint64_t *bkeys;      // [n_units][cap] bulk eviction: every slot's eviction key
                        //   (UINT64_MAX for a protected token)
  int32_t *nmoves;      // [n_units] bulk eviction: rows the move launch relocates (0: none)
  float *chunk_acc;     // [n_units][ceil(cap/D)][G][D] Stage II chunked V side: each chunk's P.V
  int32_t *chunk_cnt;   // [n_units][ceil(cap/D)][G] tokens each chunk kept per q-head
  int32_t *order;       // [n_units][cap] Stage II chunked V side: the live slots in position order
  uint32_t *uhist;      // [n_units][kBulkHistWords] bulk cut: the unit's key histogram (kBulkBins
                        //   words), then its record (kBulkRec: candidates, bin, need, count, mode)
  int32_t *bsel;        // [n_units][4] bulk cut: tokens to evict, budget, tokens, flag (1: cut in bulk)
  float *logits2;       // [n_units][cap][G] Stage II in two launches: the exact logits (raw q.k)
  uint64_t *s2keys;     // [n_units][G][cap] Stage II in two launches: selection keys of long units
  uint64_t *cand;       // [n_units][kBulkCand] bulk cut: the keys of the threshold's bin
  int32_t *cslot;       // [n_units][kBulkCand] ... and their slots
  uint64_t *ebits;      // [n_units][ceil(cap / 64)] bulk cut: the slots whose keys lie below the bin
};

constexpr int kWsParts = 29;
// Bulk cut: a histogram of the eviction keys' top kBulkBits bits per unit,
// and the keys of the bin that holds the threshold, gathered when at most
// kBulkCand.
constexpr int kBulkBits = 11, kBulkBins = 1 << kBulkBits, kBulkShift = 64 - kBulkBits;
constexpr int kBulkCand = 4096;
constexpr int kBulkRec = kBulkBins;             // the record's first word in a unit's uhist row
constexpr int kBulkHistWords = kBulkBins + 64;  // a unit's uhist row (16-byte multiple)
struct WsSizes {
  size_t off[kWsParts];
  size_t total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline int max_tiles_for(int n_units) { return kMaxGrid + n_units + 8; }

inline WsSizes ws_sizes(int B, int Hq, int Hkv, int D, int cap, int kT, bool chunks, bool order) {
  const size_t U = (size_t)B * Hkv, G = (size_t)(Hq / Hkv), MT = (size_t)max_tiles_for((int)U);
  const size_t NC = chunks ? (size_t)((cap + D - 1) / D) : 0;
  const size_t sz[kWsParts] = {
      512,                             // status (+ spare)
      sizeof(int32_t) * 4 * MT,        // tinfo
      sizeof(float) * U,               // fz_newimp
      sizeof(uint32_t) * U,            // ticket
      sizeof(int32_t) * (U + 4),       // plan
      sizeof(float) * U * G * 2,       // stats
      sizeof(float) * MT * G * 2,      // part_ml
      sizeof(float) * MT * G * D,      // part_acc
      sizeof(float) * U * cap * G,     // logits
      sizeof(uint64_t) * MT,           // tile_key
      sizeof(int32_t) * MT,            // tile_slot
      sizeof(int32_t) * U * cap,       // holes
      sizeof(int32_t) * U * cap,       // movers
      sizeof(uint32_t) * B * Hq * ((D + 31) / 32),  // chmask
      sizeof(int32_t) * B * Hq * (size_t)(kT > 0 ? kT : 1),  // tsel
      sizeof(int32_t) * B * Hq,        // tcount
      sizeof(int32_t) * 4 * U,         // urec
      sizeof(uint64_t) * U * cap,      // bkeys
      sizeof(int32_t) * U,             // nmoves
      sizeof(float) * U * NC * G * D,  // chunk_acc
      sizeof(int32_t) * U * NC * G,    // chunk_cnt
      order ? sizeof(int32_t) * U * cap : 0,   // order (chunked Stage II V side, block eviction)
      sizeof(uint32_t) * U * (size_t)kBulkHistWords,  // uhist
      sizeof(int32_t) * 4 * U,         // bsel
      (kT > 0 && !chunks) ? sizeof(float) * U * cap * G : 0,     // logits2
      (kT > 0 && !chunks) ? sizeof(uint64_t) * U * G * cap : 0,  // s2keys
      sizeof(uint64_t) * U * kBulkCand,  // cand
      sizeof(int32_t) * U * kBulkCand,   // cslot
      sizeof(uint64_t) * U * (size_t)((cap + 63) / 64),  // ebits
  };
  WsSizes w;
  size_t o = 0;
  for (int i = 0; i < kWsParts; ++i) {
    w.off[i] = o;
    o += align256(sz[i]);
  }
  w.total = o;
  return w;
}

inline Ws ws_carve(void *base, const WsSizes &s) {
  char *b = static_cast<char *>(base);
  Ws w;
  w.status = reinterpret_cast<int32_t *>(b + s.off[0]);
  w.tinfo = reinterpret_cast<int32_t *>(b + s.off[1]);
  w.fz_newimp = reinterpret_cast<float *>(b + s.off[2]);
  w.ticket = reinterpret_cast<uint32_t *>(b + s.off[3]);
  w.plan = reinterpret_cast<int32_t *>(b + s.off[4]);
  w.stats = reinterpret_cast<float *>(b + s.off[5]);
  w.part_ml = reinterpret_cast<float *>(b + s.off[6]);
  w.part_acc = reinterpret_cast<float *>(b + s.off[7]);
  w.logits = reinterpret_cast<float *>(b + s.off[8]);
  w.tile_key = reinterpret_cast<uint64_t *>(b + s.off[9]);
  w.tile_slot = reinterpret_cast<int32_t *>(b + s.off[10]);
  w.holes = reinterpret_cast<int32_t *>(b + s.off[11]);
  w.movers = reinterpret_cast<int32_t *>(b + s.off[12]);
  w.chmask = reinterpret_cast<uint32_t *>(b + s.off[13]);
  w.tsel = reinterpret_cast<int32_t *>(b + s.off[14]);
  w.tcount = reinterpret_cast<int32_t *>(b + s.off[15]);
  w.urec = reinterpret_cast<int32_t *>(b + s.off[16]);
  w.bkeys = reinterpret_cast<uint64_t *>(b + s.off[17]);
  w.nmoves = reinterpret_cast<int32_t *>(b + s.off[18]);
  w.chunk_acc = reinterpret_cast<float *>(b + s.off[19]);
  w.chunk_cnt = reinterpret_cast<int32_t *>(b + s.off[20]);
  w.order = reinterpret_cast<int32_t *>(b + s.off[21]);
  w.uhist = reinterpret_cast<uint32_t *>(b + s.off[22]);
  w.bsel = reinterpret_cast<int32_t *>(b + s.off[23]);
  w.logits2 = reinterpret_cast<float *>(b + s.off[24]);
  w.s2keys = reinterpret_cast<uint64_t *>(b + s.off[25]);
  w.cand = reinterpret_cast<uint64_t *>(b + s.off[26]);
  w.cslot = reinterpret_cast<int32_t *>(b + s.off[27]);
  w.ebits = reinterpret_cast<uint64_t *>(b + s.off[28]);
  return w;
}

// Tile plan computed on the host from a caller-supplied copy of len[] (the
// kernels then skip deriving it from device memory).  n == 0: no host plan.
constexpr int kHostPlanUnits = 64;
// Stage II in two launches lists its selected tokens in LDS: k_T up to this.
constexpr int kS2TwoMaxTokens = 2048;
struct HostPlan {
  int32_t n, T, ntiles;
  int32_t base[kHostPlanUnits + 1];  // first tile of each unit; base[n] = ntiles
  int32_t L[kHostPlanUnits];         // tokens after the append (0: unit not planned)
  // A bulk cut's row moves, one workgroup per chunk of bulk_moves_per_wg moves
  // of each unit's bound: the first chunk of each unit; mvb[n] = chunks.
  int32_t mvb[kHostPlanUnits + 1];
};

// Row moves one workgroup of the bulk cut's move launch makes (256 threads,
// 16 bytes of a row per thread, four rows per thread group).
constexpr int bulk_moves_per_wg(int rb) { return (256 / (rb / 16)) * 4; }

// Everything a decode-step kernel needs, passed by value.
struct StepArgs {
  int B, Hq, Hkv, D, cap, G, n_units;
  float scale_log2;          // logit scale * log2(e): logits live in the log2 domain
  const void *k_cache;       // K [U][cap][D]
  const void *v_cache;
  void *k_w, *v_w;           // same pointers, writable
  int32_t *pos;
  float *imp;
  int32_t *len;
  int32_t *evict;            // [U][state_words(cap)] pending eviction (cache state)
  const int32_t *budget;     // may be null
  int32_t budget_all, n_sink, n_recent;
  int32_t acc_recent;        // importance accumulates only inside the protected window (HiKV dual bank)
  int32_t acc_logit;         // importance accumulates pre-softmax logits (Kelle)
  int32_t r, kT;             // Stage II
  int32_t s2_chunks;         // Stage II V side: HiKV's per-chunk top-r of P (else exact top-k_T)
  int32_t no_bulk;           // the host skipped the bulk-eviction launch (length hint): flag a unit that needed it
  int32_t bulk_split;        // a bulk cut leaves its row moves to a launch of many workgroups per unit
  int32_t bulk_rows;         // with bulk_split: the host's bound on the rows any unit's cut moves
  int32_t bulk_known;        // the host foresaw every bulk cut of the step (lengths and budgets known)
  int32_t block;             // block-granular eviction: positions per block (>= 2), or 0 (single tokens)
  int32_t s2_two;            // Stage II (exact top-k_T V side) in the two-launch sequence
  int32_t moves_flat;        // the move launch runs one workgroup per chunk of hp.mvb
  const void *q, *k_new, *v_new;
  const int32_t *new_pos;
  float *out;
  int32_t *dbg_channels, *dbg_tokens, *dbg_count;
  Ws ws;
  HostPlan hp;
};

// ---------------------------------------------------------------------------
// Small device helpers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void set_status(int32_t *status, int32_t code) {
  atomicCAS(status, 0, code);
}

// The kernel-argument lines a launch's prologue reads, pulled into the scalar
// cache together.  Left to the code, each scalar load is issued where its
// value is first needed, and the prologue waits for one cache miss after
// another (the plan's words, then the flags, then the pointers); touched
// together they cost one round trip.  Lines: the first 512 bytes of StepArgs
// (every field before the host plan), the hidden arguments after it, and the
// host-plan words of unit uh.  Loads and their wait are in one asm block; the
// registers they fill are scratch, declared clobbered.
static_assert(offsetof(StepArgs, hp) <= 512, "the fields before the host plan span eight 64-byte lines");
__device__ __forceinline__ void kernarg_warm(int uh) {
  const uint64_t kp = (uint64_t)__builtin_amdgcn_kernarg_segment_ptr();
  const uint64_t pa = kp + offsetof(StepArgs, hp) + offsetof(HostPlan, base) + 4 * (uint64_t)uh;
  const uint64_t pb = kp + offsetof(StepArgs, hp) + offsetof(HostPlan, L) + 4 * (uint64_t)uh;
  asm volatile(
      "s_load_dword s40, %0, 0x0\n\t"
      "s_load_dword s41, %0, 0x40\n\t"
      "s_load_dword s42, %0, 0x80\n\t"
      "s_load_dword s43, %0, 0xc0\n\t"
      "s_load_dword s44, %0, 0x100\n\t"
      "s_load_dword s45, %0, 0x140\n\t"
      "s_load_dword s46, %0, 0x180\n\t"
      "s_load_dword s47, %0, 0x1c0\n\t"
      "s_load_dword s48, %0, %3\n\t"
      "s_load_dword s49, %0, %4\n\t"
      "s_load_dword s50, %1, 0x0\n\t"
      "s_load_dword s51, %2, 0x0\n\t"
      "s_waitcnt lgkmcnt(0)"
      :
      : "s"(kp), "s"(pa), "s"(pb), "i"(sizeof(StepArgs)), "i"(sizeof(StepArgs) + 64)
      : "s40", "s41", "s42", "s43", "s44", "s45", "s46", "s47", "s48", "s49", "s50", "s51", "memory");
}

// A bulk cut's per-unit histograms and records start at zero: the attention
// launch, which precedes every launch that adds to them, clears them.
__device__ __forceinline__ void bulk_hist_clear(const StepArgs &a) {
  const int n = a.n_units * (kBulkHistWords / 4);
  uint4 *p = reinterpret_cast<uint4 *>(a.ws.uhist);
  for (int i = (int)(blockIdx.x * blockDim.x + threadIdx.x); i < n; i += (int)(gridDim.x * blockDim.x))
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}

// All-reduce across the LPR consecutive lanes that hold one token row.
// quad_perm xor1 / xor2, then half-row and row mirrors (DPP, full rate), then
// cross-row swizzles for rows wider than 16 lanes.
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
  if constexpr (LPR >= 2) v += dpp<0xB1>(v);
  if constexpr (LPR >= 4) v += dpp<0x4E>(v);
  if constexpr (LPR >= 8) v += dpp<0x141>(v);
  if constexpr (LPR >= 16) v += dpp<0x140>(v);
  if constexpr (LPR >= 32) v += __shfl_xor(v, 16);
  if constexpr (LPR >= 64) v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// bf16 pair (one uint32) -> two floats.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Monotone map float -> uint32 (total order of the float values).
__device__ __forceinline__ uint32_t ord_f32(float f) {
  uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inverse of ord_f32.
__device__ __forceinline__ float unord_f32(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o ^ 0x80000000u) : ~o);
}

// Eviction key: smaller = evicted first.  Lower importance first; among
// equal importance the higher position first (so the lower one is kept).
__device__ __forceinline__ uint64_t evict_key(float imp, int32_t pos) {
  return ((uint64_t)ord_f32(imp) << 32) | (uint64_t)(~(uint32_t)pos);
}

// Stores, loads and a counter increment that are coherent across the whole
// device (all XCDs' L2 caches) without a cache-wide write-back.  The stores
// write through to memory: a kernel's results stored this way leave little
// for the write-back at its end, which the next launch waits for.
__device__ __forceinline__ void store_agent(int32_t *p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_agent(const int32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ticket_agent(uint32_t *p) {
  return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent_f(float *p, float v) {
  store_agent(reinterpret_cast<int32_t *>(p), __float_as_int(v));
}

__device__ __forceinline__ int unit_budget(const StepArgs &a, int u) {
  return a.budget ? a.budget[u] : a.budget_all;
}

// Budget / capacity validity of a unit before a decode step.
__device__ __forceinline__ int32_t unit_error(const StepArgs &a, int u, int len_now, int add) {
  const int beta = unit_budget(a, u);
  if (len_now + add > a.cap || len_now < 0) return HIKV_ECAPACITY;
  if (beta < a.n_sink || beta > a.cap) return HIKV_EBUDGET;
  return 0;
}

}  // namespace hikv
