// hikv_dev.h -- device helpers of the two-launch step's split-K attention kernels:
// plans, global->LDS staging, lane reductions, eviction keys, the
// pending-eviction lookup and matrix-core operands.
#pragma once

#include "hikv_common.h"

namespace hikv {


constexpr int kThreads = 256;

__device__ __forceinline__ void st_ag(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_ag(int32_t *p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_ag(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_ag(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_ag(const int32_t *p) {
  return __hip_atomic_load(const_cast<int32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_ag(const uint64_t *p) {
  return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Load a wave-uniform value through the vector memory path.  A scalar load
// shares its counter (lgkmcnt) with the kernel-argument loads, so the first
// wait for an argument would also wait for this round trip.  z is a zero the
// compiler cannot see through (vzero(), taken once before any load: the asm
// that makes it may otherwise wait for loads in flight).
__device__ __forceinline__ int vzero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}
template <typename T>
__device__ __forceinline__ T ld_vec(const T *p, int z) {
  return p[z];
}
// A load of global memory through a uniform pointer the compiler cannot
// trace to its origin, so that it is neither merged with another load of the
// same address nor split into per-branch loads.
template <typename T>
__device__ __forceinline__ T ld_opaque(const T *p, int z) {
  using GP = const __attribute__((address_space(1))) T *;
  GP g = (GP)p;
  asm("" : "+s"(g));
  return g[z];
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

struct Plan {
  int valid, u, s, nt, t0, t1, L, T;
};

// Every wave computes the same plan; lanes own contiguous unit ranges, so the
// tile ids of a unit are consecutive.
__device__ inline Plan wave_plan(const StepArgs &a, int tile, int ntarget, bool write_rec) {
  const int lane = threadIdx.x & 63;
  const int U = a.n_units;
  const int per = (U + 63) >> 6;
  const int u0 = lane * per;
  long long tot = 0;
  for (int k = 0; k < per; ++k) {
    const int u = u0 + k;
    if (u < U) {
      const int len = a.len[u];
      if (!unit_error(a, u, len, 1)) tot += len + 1;
    }
  }
  tot = wave_sum(tot);
  const long long tt = (tot + ntarget - 1) / ntarget;
  int T = (int)((tt + 15) / 16 * 16);
  if (T < 16) T = 16;
  int mine = 0;
  for (int k = 0; k < per; ++k) {
    const int u = u0 + k;
    if (u < U) {
      const int len = a.len[u];
      if (!unit_error(a, u, len, 1)) mine += (len + 1 + T - 1) / T;
    }
  }
  int incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int x = __shfl_up(incl, off);
    if (lane >= off) incl += x;
  }
  const int excl = incl - mine;
  const bool own = (tile >= excl) && (tile < incl);
  const uint64_t m = __ballot(own);
  Plan p;
  p.T = T;
  p.valid = m != 0ull;
  int info[4] = {0, 0, 0, 0};
  if (write_rec) {  // the per-unit records the second launch reads
    int bse = excl;
    for (int k = 0; k < per; ++k) {
      const int u = u0 + k;
      if (u >= U) break;
      const int len = a.len[u];
      const int L = unit_error(a, u, len, 1) ? 0 : len + 1;
      const int n = (L + T - 1) / T;
      reinterpret_cast<int4 *>(a.ws.urec)[u] = make_int4(bse, n, L, 0);
      bse += n;
    }
  }
  if (own) {
    int bse = excl;
    for (int k = 0; k < per; ++k) {
      const int u = u0 + k;
      if (u >= U) break;
      const int len = a.len[u];
      const int L = unit_error(a, u, len, 1) ? 0 : len + 1;
      const int n = (L + T - 1) / T;
      if (tile >= bse && tile < bse + n) {
        info[0] = u;
        info[1] = tile - bse;
        info[2] = n;
        info[3] = L;
      }
      bse += n;
    }
  }
  const int src = p.valid ? (int)__builtin_ctzll(m) : 0;
  p.u = __shfl(info[0], src);
  p.s = __shfl(info[1], src);
  p.nt = __shfl(info[2], src);
  p.L = __shfl(info[3], src);
  p.t0 = p.s * T;
  p.t1 = min(p.t0 + T, p.L);
  return p;
}

// Plan from the kernel arguments (host-computed from the caller's copy of
// len[]).  Lane i holds unit i's end tile and length (bend, Lv: loaded by the
// caller before it knows whether there is a host plan, so that the lookup
// costs one round trip); the unit is the number of units that end at or
// before the tile.
__device__ inline Plan host_plan(const StepArgs &a, int tile, int bend, int Lv) {
  const int lane = threadIdx.x & 63;
  const int n = a.hp.n;
  const int u = __popcll(__ballot(lane < n && bend <= tile));
  Plan p;
  p.T = a.hp.T;
  p.valid = u < n;
  const int uu = p.valid ? u : 0;
  const int b0 = uu ? __builtin_amdgcn_readlane(bend, uu - 1) : 0;
  p.u = uu;
  p.s = tile - b0;
  p.nt = __builtin_amdgcn_readlane(bend, uu) - b0;
  p.L = __builtin_amdgcn_readlane(Lv, uu);
  p.t0 = p.s * p.T;
  p.t1 = min(p.t0 + p.T, p.L);
  return p;
}

template <int EL, int D, int G>
struct ALay {
  static constexpr int RB = D * EL;             // bytes per token row
  static constexpr int CH = 16 / EL;            // channels per lane
  static constexpr int LPR = D / CH;            // lanes per token row
  static constexpr int TPW = kWave / LPR;       // rows per wave instruction
  static constexpr int SUBB = 8192;             // bytes of K (and of V) per sub-chunk
  static constexpr int NSUB = 3;                // sub-chunks per LDS chunk
  static constexpr int TS = SUBB / RB;          // tokens per sub-chunk
  static constexpr int TC = TS * NSUB;          // tokens per LDS chunk (one tile normally)
  static constexpr int UR = TS / 4 / TPW;       // row groups per wave per sub-chunk
  static constexpr int NI = SUBB / 4096;        // DMA instructions per wave per sub-chunk, K or V
};

// Cache policy of the K and V row loads: non-temporal.  A step reads every
// live row once, and the rows of all the layers of a model far exceed the
// caches; marked as streaming they do not push out the small per-token arrays
// (importance, positions, logits) that the same layer's next step reads again.
constexpr int kRowCpol = 2;

// Stage one sub-chunk of K and V rows into LDS with the global->LDS DMA.
// Every lane issues exactly NI loads for K and NI for V (constant vmcnt
// bookkeeping); lanes past the tile read a clamped valid row into unused
// buffer space; the new token's row (slot Lold, not yet in the cache) comes
// from k_new / v_new.
// SWZ (256-byte rows): the 16-byte chunk p of LDS row r holds source chunk
// p ^ (r & 15), so that reads of one chunk column across 16 rows spread over
// all LDS banks.
template <int RB, int NI, bool SWZ = false>
__device__ __forceinline__ void stage_sub(char *kb, char *vb, const char *kc, const char *vc,
                                          const char *kn, const char *vn, int c0, int nrows,
                                          int t0, int Lold, int wave, int lane) {
  static_assert(!SWZ || RB == 256, "the swizzle is written for 256-byte rows");
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int off = ((i * 4 + wave) << 10) + (lane << 4);
    const int row = off / RB;
    const int col = SWZ ? ((((off - row * RB) >> 4) ^ (row & 15)) << 4) : off - row * RB;
    const int n = (row < nrows) ? c0 + row : t0;  // t0 is always a live row of the tile
    const char *ks = (n == Lold) ? kn + col : kc + (size_t)n * RB + col;
    const char *vs = (n == Lold) ? vn + col : vc + (size_t)n * RB + col;
    __builtin_amdgcn_global_load_lds(ks, kb + ((i * 4 + wave) << 10), 16, 0, kRowCpol);
    __builtin_amdgcn_global_load_lds(vs, vb + ((i * 4 + wave) << 10), 16, 0, kRowCpol);
  }
}

// The same staging done by LW of the workgroup's waves only (wave index wl
// among them): each issues 8 / LW loads for K and as many for V per sub-chunk.
template <int LW>
__device__ __forceinline__ void stage_sub_by(char *kb, char *vb, const char *kc, const char *vc,
                                             const char *kn, const char *vn, int c0, int nrows,
                                             int t0, int Lold, int wl, int lane) {
  constexpr int RB = 256;
  if (nrows == 32 && (unsigned)(Lold - c0) >= 32u) {
    // Every row is a cache row (the usual case): one base per sub-chunk and
    // per-lane offsets, which do not change from one sub-chunk to the next.
    const char *kbase = kc + (size_t)c0 * RB, *vbase = vc + (size_t)c0 * RB;
#pragma unroll
    for (int i = 0; i < 8 / LW; ++i) {
      const int piece = i * LW + wl;
      const int row = piece * 4 + (lane >> 4);
      const uint32_t o = (uint32_t)(row * RB) + ((((uint32_t)lane & 15u) ^ ((uint32_t)row & 15u)) << 4);
      __builtin_amdgcn_global_load_lds(kbase + o, kb + (piece << 10), 16, 0, kRowCpol);
      __builtin_amdgcn_global_load_lds(vbase + o, vb + (piece << 10), 16, 0, kRowCpol);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 8 / LW; ++i) {
    const int piece = i * LW + wl;  // 1 KB piece of the 8 KB sub-chunk: four 256-byte rows
    const int off = (piece << 10) + (lane << 4);
    const int row = off / RB;
    const int col = (((off - row * RB) >> 4) ^ (row & 15)) << 4;
    const int n = (row < nrows) ? c0 + row : t0;  // t0 is always a live row of the tile
    const char *ks = (n == Lold) ? kn + col : kc + (size_t)n * RB + col;
    const char *vs = (n == Lold) ? vn + col : vc + (size_t)n * RB + col;
    __builtin_amdgcn_global_load_lds(ks, kb + (piece << 10), 16, 0, kRowCpol);
    __builtin_amdgcn_global_load_lds(vs, vb + (piece << 10), 16, 0, kRowCpol);
  }
}

// LDS reads of rows that arrived by DMA.  Written as one asm block so that the
// compiler, which cannot tell the three sub-chunk buffers apart, does not
// insert a vmcnt(0) before them (the explicit vmcnt chain already covers the
// sub-chunk being read); the block waits for its own reads.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) char *)p;
}
__device__ __forceinline__ void lds_read_rows(uint4 &k0, uint4 &k1, uint4 &v0, uint4 &v1, uint32_t ak0,
                                              uint32_t ak1, uint32_t av0, uint32_t av1) {
  u32x4 a, b, c, d;
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d)
      : "v"(ak0), "v"(ak1), "v"(av0), "v"(av1)
      : "memory");
  k0 = make_uint4(a.x, a.y, a.z, a.w);
  k1 = make_uint4(b.x, b.y, b.z, b.w);
  v0 = make_uint4(c.x, c.y, c.z, c.w);
  v1 = make_uint4(d.x, d.y, d.z, d.w);
}

__device__ __forceinline__ void dma16(const void *src, void *lds_dst) {
  __builtin_amdgcn_global_load_lds(src, lds_dst, 16, 0, 0);
}
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
// Ends the wave here, so that the code after it does not merge with this path
// at a common exit (where the compiler would wait for both paths' loads).
__device__ __forceinline__ void end_wave() { __builtin_amdgcn_endpgm(); }

// Reductions across the token rows of a wave.  A token row is LPR lanes wide
// and the rows of a wave are lanes i, i ^ LPR, i ^ 2 LPR, ...  The permlane
// swaps exchange 32- and 16-lane halves between two registers without LDS;
// applied to two different values at once and followed by one add, each
// swap halves the registers still to reduce (a reduce-scatter).  The swaps
// are asm: the compiler builtin, given one value for both operands, treats
// its two results as equal.
__device__ __forceinline__ void permlane16_swap(float &a, float &b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane32_swap(float &a, float &b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}

// Reduce N values per lane over the rows of a wave (rows LPR = 8, 16 or 32
// lanes wide).  S = 1 swap step for 32-lane rows, else 2.  Afterwards v[i],
// i < N >> S, holds in lane part p = lane >> (6 - S) the reduction of value
// i + p * (N >> S); rows of 8 lanes are finished with DPP (row_ror:8), and
// there lanes l and l ^ 8 hold the same results.
template <int LPR>
constexpr int swap_steps() { return LPR >= 32 ? 1 : 2; }
template <int LPR, bool MAX, int N>
__device__ __forceinline__ void rows_reduce(float (&v)[N]) {
  constexpr int S = swap_steps<LPR>();
  static_assert(N % (1 << S) == 0, "values must split over the lane parts");
  auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    float x = v[i], y = v[i + N / 2];
    permlane32_swap(x, y);
    v[i] = op(x, y);
  }
  if constexpr (S == 2) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      float x = v[i], y = v[i + N / 4];
      permlane16_swap(x, y);
      v[i] = op(x, y);
    }
  }
  if constexpr (LPR == 8) {
#pragma unroll
    for (int i = 0; i < (N >> S); ++i)
      v[i] = op(v[i], __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v[i]), 0x128,
                                                                            0xf, 0xf, false)));
  }
}

// All-reduce over the lanes of a wave that are congruent modulo M (M a power
// of two): DPP within 16-lane rows (xor 1, xor 2, then rotations by 4 and 8,
// which combine the row's lanes of one residue), permlane swaps across rows.
// No data goes through LDS.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
template <int STEP>
__device__ __forceinline__ uint32_t dpp_step(uint32_t v) {
  if constexpr (STEP == 1) return dpp_u<0xB1>(v);        // quad_perm [1,0,3,2]
  else if constexpr (STEP == 2) return dpp_u<0x4E>(v);   // quad_perm [2,3,0,1]
  else if constexpr (STEP == 4) return dpp_u<0x124>(v);  // row_ror:4
  else return dpp_u<0x128>(v);                           // row_ror:8
}
__device__ __forceinline__ void swap16_u(uint32_t &a, uint32_t &b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap32_u(uint32_t &a, uint32_t &b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
template <int M, typename Op>
__device__ __forceinline__ float lanes_reduce(float v, Op op) {
  auto step = [&](auto tag) {
    constexpr int S = decltype(tag)::value;
    v = op(v, __uint_as_float(dpp_step<S>(__float_as_uint(v))));
  };
  if constexpr (M <= 1) step(std::integral_constant<int, 1>{});
  if constexpr (M <= 2) step(std::integral_constant<int, 2>{});
  if constexpr (M <= 4) step(std::integral_constant<int, 4>{});
  if constexpr (M <= 8) step(std::integral_constant<int, 8>{});
  if constexpr (M <= 16) {
    uint32_t a = __float_as_uint(v), b = a;
    swap16_u(a, b);
    v = op(__uint_as_float(a), __uint_as_float(b));
  }
  if constexpr (M <= 32) {
    uint32_t a = __float_as_uint(v), b = a;
    swap32_u(a, b);
    v = op(__uint_as_float(a), __uint_as_float(b));
  }
  return v;
}
template <int M>
__device__ __forceinline__ float lanes_max(float v) {
  return lanes_reduce<M>(v, [](float x, float y) { return fmaxf(x, y); });
}
template <int M>
__device__ __forceinline__ float lanes_sum(float v) {
  return lanes_reduce<M>(v, [](float x, float y) { return x + y; });
}

// The smallest 64-bit eviction key of the wave, with the slot that holds it.
struct KeySlot {
  uint32_t hi, lo, slot;
};
__device__ __forceinline__ KeySlot key_min(KeySlot a, KeySlot b) {
  const bool take_b = (b.hi < a.hi) || (b.hi == a.hi && b.lo < a.lo);
  return take_b ? b : a;
}
__device__ __forceinline__ void wave_min_key(uint64_t &key, int &slot) {
  KeySlot x{(uint32_t)(key >> 32), (uint32_t)key, (uint32_t)slot};
  auto step = [&](auto tag) {
    constexpr int S = decltype(tag)::value;
    x = key_min(x, KeySlot{dpp_step<S>(x.hi), dpp_step<S>(x.lo), dpp_step<S>(x.slot)});
  };
  step(std::integral_constant<int, 1>{});
  step(std::integral_constant<int, 2>{});
  step(std::integral_constant<int, 4>{});
  step(std::integral_constant<int, 8>{});
  {
    KeySlot a = x, b = x;
    swap16_u(a.hi, b.hi);
    swap16_u(a.lo, b.lo);
    swap16_u(a.slot, b.slot);
    x = key_min(a, b);
  }
  {
    KeySlot a = x, b = x;
    swap32_u(a.hi, b.hi);
    swap32_u(a.lo, b.lo);
    swap32_u(a.slot, b.slot);
    x = key_min(a, b);
  }
  key = ((uint64_t)x.hi << 32) | x.lo;
  slot = (int)x.slot;
}

// The value lane l holds (l wave-uniform).
__device__ __forceinline__ float lane_value(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// ---------------------------------------------------------------------------
// Pending eviction.  A two-launch step that evicts one token leaves the choice
// of the victim to the next call: it stores, in the unit's record of the
// cache's pending-eviction state (hikv_cache.evict), the number n of its
// importance blocks and each block's lowest eviction key and its slot.  The
// evicted slot is the one whose key is the smallest; until a later call
// resolves it, the slot is dead.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int pend_stride(const StepArgs &a) { return imp_blocks(a.cap); }
// The unit's record: [0] count, [1] dead slot, candidates from word 4.
__device__ __forceinline__ int32_t *unit_state(const StepArgs &a, int u) {
  return a.evict + (size_t)u * state_words(a.cap);
}

// The lookup in the attention launch goes through LDS, 64 records of 16 bytes
// at a time: lane 0 fetches the header (count, slot) and lanes 1..63 the
// first 63 candidates; later rounds fetch 64 candidates each.
struct PendLds {
  int32_t rec[kWave][4];
  int32_t dead[4];
};

// Wave 0 of a tile, before its first rows: the first 16-byte records of unit
// u's state, by DMA (no register loads whose waits the compiler would place),
// issued ahead of the rows so that the first wait covers them.
__device__ __forceinline__ void pend_fetch(const StepArgs &a, int u, PendLds &pd, int lane) {
  const int nbm = pend_stride(a);
  const int32_t *rec = unit_state(a, u);
  __builtin_amdgcn_global_load_lds(rec + 4 * min(lane, nbm), &pd.rec[0][0], 16, 0, 0);
}

// Wave 0, once the fetch has landed: the dead slot (-1 if none), left in
// pd.dead[0] for the other waves of the tile; with record, also stored for
// the second launch of the step.  More than 63 candidates take a round trip
// per further 64.
__device__ __forceinline__ int pend_resolve(const StepArgs &a, int u, PendLds &pd, int lane, bool record) {
  const int nbm = pend_stride(a);
  int n;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(n) : "v"(lds_addr(&pd.rec[0][0])) : "memory");
  n = __builtin_amdgcn_readfirstlane(min(n, nbm));
  uint64_t key = ~0ull;
  int slot = -1;
  // Record r (r >= 1) of the state is candidate r - 1; round base holds
  // records base .. base + 63.
  for (int base = 0; base <= n; base += kWave) {
    if (base > 0) {
      __builtin_amdgcn_global_load_lds(unit_state(a, u) + 4 * min(base + lane, nbm), &pd.rec[0][0], 16, 0, 0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    u32x4 e;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(e) : "v"(lds_addr(&pd.rec[lane][0])) : "memory");
    const int r = base + lane;
    const uint64_t k = ((uint64_t)e.y << 32) | e.x;
    if (r >= 1 && r <= n && k < key) {
      key = k;
      slot = (int)e.z;
    }
  }
  wave_min_key(key, slot);
  const int d = (key == ~0ull) ? -1 : slot;
  if (lane == 0) {
    pd.dead[0] = d;
    if (record) store_agent(unit_state(a, u) + 1, d);
  }
  // The LDS write is complete before the barrier that follows (a DMA barrier
  // does not wait for LDS operations).
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  return d;
}
__device__ __forceinline__ int pend_read(PendLds &pd) {
  int d;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(d) : "v"(lds_addr(&pd.dead[0])) : "memory");
  return __builtin_amdgcn_readfirstlane(d);
}

// Workgroup barrier for LDS data only.  __syncthreads() also waits for every
// global load and store of the wave to complete, which costs a memory round
// trip when none of them matter to the LDS exchange.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Workgroup barrier for data that arrived by global->LDS DMA.  The caller has
// already waited for its own DMA with an explicit vmcnt; __syncthreads() would
// add a full vmcnt(0) and serialise the sub-chunk pipeline.
__device__ __forceinline__ void dma_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Units a device-side error excludes from the step: zero their output rows
// and record the first error (device-derived plans only; with a host plan the
// second launch does this).
template <int G, int D>
__device__ void error_sweep(const StepArgs &a) {
  for (int u = threadIdx.x; u < a.n_units; u += kThreads) {
    const int err = unit_error(a, u, a.len[u], 1);
    if (err) {
      set_status(a.ws.status, err);
      const int b = u / a.Hkv, j = u - b * a.Hkv;
      for (int i = 0; i < G * D; ++i) a.out[((size_t)(b * a.Hq + j * G)) * D + i] = 0.f;
    }
  }
}


// ---------------------------------------------------------------------------
// K1 for bf16 K and V with D = 128: the same tiles, staging and outputs, with
// q.k and P.V on the matrix cores (v_mfma_f32_16x16x16_bf16).
//
// Per 32-token sub-chunk, wave w takes token group w & 1 (16 rows) and
// channel half w >> 1 of P.V.  q.k is S = K Q^T (A = 16 K rows, B = the
// group's queries, zero-padded to 16 columns), so each lane ends with the
// scores of 4 tokens for one head -- exactly P's layout as the A operand of
// P.V.  V enters as the B operand through LDS transpose reads.  P (fp32)
// goes in as a bf16 pair hi + lo, which keeps it to about 16 bits.
// Each head keeps one running maximum per wave, so the tokens of a wave need
// no merge; the tile partial combines the two token groups.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Byte offset of element (row, ch) in a sub-chunk of 256-byte rows staged
// with the swizzle of stage_sub.
__device__ __forceinline__ uint32_t swz_off(int row, int ch) {
  return (uint32_t)(row * 256 + ((((ch >> 3) ^ (row & 15)) << 4) | ((ch & 7) << 1)));
}

// The twelve LDS reads of one sub-chunk for one wave: eight 8-byte K reads
// (q.k A operand) and four transpose reads of V (P.V B operand), at
// immediate offsets from per-lane addresses, then one wait.  asm, for the
// reason given at lds_read_rows.
template <int KOFF, int VOFF>
__device__ __forceinline__ void mfma_operands(uint64_t (&o)[12], const uint32_t (&ad)[12]) {
  asm volatile(
      "ds_read_b64 %0, %12 offset:%24\n\t"
      "ds_read_b64 %1, %13 offset:%24\n\t"
      "ds_read_b64 %2, %14 offset:%24\n\t"
      "ds_read_b64 %3, %15 offset:%24\n\t"
      "ds_read_b64 %4, %16 offset:%24\n\t"
      "ds_read_b64 %5, %17 offset:%24\n\t"
      "ds_read_b64 %6, %18 offset:%24\n\t"
      "ds_read_b64 %7, %19 offset:%24\n\t"
      "ds_read_b64_tr_b16 %8, %20 offset:%25\n\t"
      "ds_read_b64_tr_b16 %9, %21 offset:%25\n\t"
      "ds_read_b64_tr_b16 %10, %22 offset:%25\n\t"
      "ds_read_b64_tr_b16 %11, %23 offset:%25\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]),
        "=&v"(o[7]), "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7]),
        "v"(ad[8]), "v"(ad[9]), "v"(ad[10]), "v"(ad[11]), "i"(KOFF), "i"(VOFF)
      : "memory");
}

// Wait until the sub-chunk being consumed has landed: at most k * STEP loads
// (those of the k sub-chunks issued after it, 0 <= k <= K) may be outstanding.
// Eight 8-byte LDS reads 32 bytes apart from one per-lane address, one wait.
// asm: the array was filled by DMA, and a compiler-visible read of DMA'd LDS
// makes the compiler wait for every load in flight, the ring's included.
__device__ __forceinline__ void lds_read8_b64(uint64_t (&o)[8], uint32_t addr) {
  asm volatile(
      "ds_read_b64 %0, %8\n\t"
      "ds_read_b64 %1, %8 offset:32\n\t"
      "ds_read_b64 %2, %8 offset:64\n\t"
      "ds_read_b64 %3, %8 offset:96\n\t"
      "ds_read_b64 %4, %8 offset:128\n\t"
      "ds_read_b64 %5, %8 offset:160\n\t"
      "ds_read_b64 %6, %8 offset:192\n\t"
      "ds_read_b64 %7, %8 offset:224\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
      : "v"(addr)
      : "memory");
}

// Stage II's attention launch stages K only: a sub-chunk of 64 rows of 256
// bytes (16 KB, the swizzle of stage_sub), issued by LW waves (wave wl among
// them), 16 / LW loads each.
template <int LW>
__device__ __forceinline__ void stage_k_by(char *kb, const char *kc, const char *kn, int c0, int nrows, int t0,
                                           int Lold, int wl, int lane) {
  constexpr int RB = 256;
#pragma unroll
  for (int i = 0; i < 16 / LW; ++i) {
    const int piece = i * LW + wl;  // 1 KB piece of the 16 KB sub-chunk: four rows
    const int off = (piece << 10) + (lane << 4);
    const int row = off / RB;
    const int col = (((off - row * RB) >> 4) ^ (row & 15)) << 4;
    const int n = (row < nrows) ? c0 + row : t0;  // t0 is always a live row of the tile
    const char *ks = (n == Lold) ? kn + col : kc + (size_t)n * RB + col;
    __builtin_amdgcn_global_load_lds(ks, kb + (piece << 10), 16, 0, kRowCpol);
  }
}

// The eight 8-byte K reads of one wave's 16 rows (the q.k A operand), at an
// immediate offset (the ring buffer), then one wait; asm, for the reason given
// at lds_read_rows.
template <int OFF>
__device__ __forceinline__ void mfma_k_operands(uint64_t (&o)[8], const uint32_t (&ad)[8]) {
  asm volatile(
      "ds_read_b64 %0, %8 offset:%16\n\t"
      "ds_read_b64 %1, %9 offset:%16\n\t"
      "ds_read_b64 %2, %10 offset:%16\n\t"
      "ds_read_b64 %3, %11 offset:%16\n\t"
      "ds_read_b64 %4, %12 offset:%16\n\t"
      "ds_read_b64 %5, %13 offset:%16\n\t"
      "ds_read_b64 %6, %14 offset:%16\n\t"
      "ds_read_b64 %7, %15 offset:%16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7]), "i"(OFF)
      : "memory");
}

// LDS accesses the compiler must not order against the DMA ring (it would
// wait for every load in flight): one 32-bit write, no wait; one 32-bit and
// two 16-bit reads with their wait.
__device__ __forceinline__ void lds_write_b32(uint32_t addr, float v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ float lds_read_f32(uint32_t addr) {
  float x;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(x) : "v"(addr) : "memory");
  return x;
}
__device__ __forceinline__ void lds_read_u16x2(uint32_t &a, uint32_t &b, uint32_t addr_a, uint32_t addr_b) {
  asm volatile("ds_read_u16 %0, %2\n\tds_read_u16 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(a), "=&v"(b) : "v"(addr_a), "v"(addr_b) : "memory");
}
__device__ __forceinline__ uint64_t lds_read_u64(uint32_t addr) {
  uint64_t x;
  asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(x) : "v"(addr) : "memory");
  return x;
}
__device__ __forceinline__ uint4 lds_read_u128(uint32_t addr) {
  uint4 x;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(x) : "v"(addr) : "memory");
  return x;
}

// Wave-wide scan and reductions with DPP (GFX9 row shifts within rows of 16
// lanes, then the row broadcasts of lanes 15 and 31), in place of shuffle
// chains through the LDS crossbar.  A lane whose DPP source lies outside its
// row keeps the identity (`old`).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t v) {
  v += dpp_u32<0x111>(0u, v);       // row_shr:1
  v += dpp_u32<0x112>(0u, v);       // row_shr:2
  v += dpp_u32<0x114>(0u, v);       // row_shr:4
  v += dpp_u32<0x118>(0u, v);       // row_shr:8
  v += dpp_u32<0x142, 0xA>(0u, v);  // row_bcast:15 into rows 1 and 3
  v += dpp_u32<0x143, 0xC>(0u, v);  // row_bcast:31 into rows 2 and 3
  return v;
}
// Maximum and sum over the wave (every lane gets the result).
__device__ __forceinline__ float wave_max_dpp(float v) {
  const uint32_t ninf = __float_as_uint(-INFINITY);
  v = fmaxf(v, __uint_as_float(dpp_u32<0x111>(ninf, __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x112>(ninf, __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x114>(ninf, __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x118>(ninf, __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x142, 0xA>(ninf, __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x143, 0xC>(ninf, __float_as_uint(v))));
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += __uint_as_float(dpp_u32<0x111>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x112>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x114>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x118>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x142, 0xA>(0u, __float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x143, 0xC>(0u, __float_as_uint(v)));
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}

template <int STEP, int K>
__device__ __forceinline__ void vm_wait_ahead(int k) {
  if constexpr (K == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    if (k >= K) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(K * STEP) : "memory");
    else vm_wait_ahead<STEP, K - 1>(k);
  }
}

__device__ __forceinline__ f32x4_t mfma16(bf16x4_t a, bf16x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Two 16x16x16 products summed by one 16x16x32 instruction: lane (qd, hl)
// holds terms 8 qd .. 8 qd + 7 of the longer sum, here the terms of (a0, b0)
// and then those of (a1, b1); a sum does not depend on which lane holds which
// of its terms, so c + a0 b0 + a1 b1 comes out of one instruction.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4_t mfma32_2(bf16x4_t a0, bf16x4_t a1, bf16x4_t b0, bf16x4_t b1, f32x4_t c) {
  const bf16x8_t a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
  const bf16x8_t b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// q.k of a 16-row K operand (eight 4-channel pieces per lane) against the
// queries: four 32-channel instructions in two independent chains (the K
// pieces are rd[0..7]).
template <int N>
__device__ __forceinline__ f32x4_t qk16(const uint64_t (&rd)[N], const bf16x4_t (&qb)[8]) {
  static_assert(N >= 8, "eight K pieces");
  f32x4_t s0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
  for (int j = 0; j < 4; j += 2) {
    s0 = mfma32_2(__builtin_bit_cast(bf16x4_t, rd[2 * j]), __builtin_bit_cast(bf16x4_t, rd[2 * j + 1]), qb[2 * j],
                  qb[2 * j + 1], s0);
    s1 = mfma32_2(__builtin_bit_cast(bf16x4_t, rd[2 * j + 2]), __builtin_bit_cast(bf16x4_t, rd[2 * j + 3]),
                  qb[2 * j + 2], qb[2 * j + 3], s1);
  }
  return s0 + s1;
}


}  // namespace hikv
