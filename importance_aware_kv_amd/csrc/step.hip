// step.hip -- the Stage I decode step in two launches.
//
// Method (pages cited by title and section): decode attention GeMVs ("HiKV",
// Sec. II-A); importance = accumulated attention, pooled over the q-heads of
// a KV group ("KV Cache Compression and Dynamic Pruning in Production
// Serving", Sec. 3 H2O, Sec. 5); eviction of the lowest importance outside the
// protected sinks and recent window (same page, Sec. 3); per-head eviction in
// an unordered slot cache where the new token takes the evicted slot ("Kelle"
// summary, Sec. 2.2 and Sec. 4.1).
//
// K1 k_attend -- one workgroup per split-K tile; the grid is one resident
//   round of workgroups.  Every wave derives the same ragged tile plan from
//   len[] and the budgets (tiles of equal length whatever the per-head mix);
//   the tile's K and V rows are staged into LDS with the global->LDS DMA
//   (16 B per lane) as three sub-chunks issued together and consumed as each
//   lands; q.k is reduced over a token row's lanes with DPP and every row
//   keeps an online softmax; the tile writes its logits, (max, sum) per head
//   and P.V partial.
// K2 k_finalize -- the same tiles.  The launch boundary makes K1's writes
//   visible, so each tile reads its unit's partials with plain loads: unit
//   softmax statistics, a slice of the output (tiles of a unit split the
//   G*D outputs), the importance of its own tokens and its lowest eviction
//   key.  The last tile of the unit to finish (atomic ticket) picks the
//   victim and writes the new token straight into the victim's slot, so no
//   row is ever moved in the steady state.  A unit that must shed more than
//   one token (first step after a prefill) is compacted by its last tile with
//   a radix select.

#include "hikv_block.h"
#include "hikv_launch.h"

namespace hikv {

namespace {

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

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Per-tile description K1 hands to K2 (16 bytes).
struct TileRec {
  int32_t u_s;     // unit << 12 | tile index within the unit; -1: no tile
  int32_t nt;      // tiles of the unit
  int32_t t0_len;  // first token << 0 (t0); length packed in L below
  int32_t L_t1;    // unused (kept for alignment)
};

struct Plan {
  int valid, u, s, nt, t0, t1, L, T;
};

// Every wave computes the same plan; lanes own contiguous unit ranges, so the
// tile ids of a unit are consecutive.
__device__ Plan wave_plan(const StepArgs &a, int tile, int ntarget) {
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
// len[]): a uniform binary search over the tile bases.
__device__ Plan host_plan(const StepArgs &a, int tile) {
  Plan p;
  p.T = a.hp.T;
  p.valid = tile < a.hp.ntiles;
  p.u = p.s = p.nt = p.t0 = p.t1 = p.L = 0;
  if (!p.valid) return p;
  int lo = 0, hi = a.hp.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.hp.base[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  p.u = lo;
  p.s = tile - a.hp.base[lo];
  p.nt = a.hp.base[lo + 1] - a.hp.base[lo];
  p.L = a.hp.L[lo];
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

// Stage one sub-chunk of K and V rows into LDS with the global->LDS DMA.
// Every lane issues exactly NI loads for K and NI for V (constant vmcnt
// bookkeeping); lanes past the tile read a clamped valid row into unused
// buffer space; the new token's row (slot Lold, not yet in the cache) comes
// from k_new / v_new.
template <int RB, int NI>
__device__ __forceinline__ void stage_sub(char *kb, char *vb, const char *kc, const char *vc,
                                          const char *kn, const char *vn, int c0, int nrows,
                                          int t0, int Lold, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int off = ((i * 4 + wave) << 10) + (lane << 4);
    const int row = off / RB, col = off - row * RB;
    const int n = (row < nrows) ? c0 + row : t0;  // t0 is always a live row of the tile
    const char *ks = (n == Lold) ? kn + col : kc + (size_t)n * RB + col;
    const char *vs = (n == Lold) ? vn + col : vc + (size_t)n * RB + col;
    __builtin_amdgcn_global_load_lds(ks, kb + ((i * 4 + wave) << 10), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vs, vb + ((i * 4 + wave) << 10), 16, 0, 0);
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// K1: split-K attention tiles.
// ---------------------------------------------------------------------------
template <int EL, int D, int G>
__global__ __launch_bounds__(kThreads) void k_attend(StepArgs a) {
  using LY = ALay<EL, D, G>;
  constexpr int CH = LY::CH, LPR = LY::LPR, TPW = LY::TPW, UR = LY::UR, TS = LY::TS, NSUB = LY::NSUB,
                TC = LY::TC, NI = LY::NI, SUBB = LY::SUBB;
  constexpr int RB = LY::RB;
  // LDS: NSUB sub-chunks, each K then V.
  __shared__ __attribute__((aligned(16))) char smem[NSUB * 2 * SUBB];
  __shared__ float sm_ml[4][G][2];
  float(*sm_acc)[G][D] = reinterpret_cast<float(*)[G][D]>(smem);  // reused after the chunks
  static_assert(4 * G * D * 4 <= NSUB * 2 * SUBB, "merge scratch must fit in the stage");
  static_assert(NSUB == 3, "the vmcnt chain below is written for three sub-chunks");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int U = a.n_units;
  const Plan pl = a.hp.n ? host_plan(a, blockIdx.x) : wave_plan(a, blockIdx.x, (int)gridDim.x - U);

  if (blockIdx.x == 0) {  // units skipped by a device-side error
    for (int u = tid; u < U; u += kThreads) {
      const int err = unit_error(a, u, a.len[u], 1);
      if (err) {
        set_status(a.ws.status, err);
        const int b = u / a.Hkv, j = u - b * a.Hkv;
        for (int i = 0; i < G * D; ++i) a.out[((size_t)(b * a.Hq + j * G)) * D + i] = 0.f;
      }
    }
  }
  if (tid == 0 && !a.hp.n) {  // hand the device-derived plan to the second launch
    int4 rec = make_int4(-1, 0, 0, 0);
    if (pl.valid) rec = make_int4(pl.u, pl.s, pl.nt, pl.L);
    reinterpret_cast<int4 *>(a.ws.tinfo)[blockIdx.x] = rec;
    if (blockIdx.x == 0) a.ws.plan[0] = pl.T;
  }
  if (!pl.valid) return;
  // A host plan must describe the device's lengths.
  const int len_dev = a.hp.n ? a.len[pl.u] : pl.L - 1;

  const int u = pl.u, b = u / a.Hkv, j = u - b * a.Hkv;
  const int Lold = pl.L - 1, t0 = pl.t0, t1 = pl.t1;
  const int tile = blockIdx.x;
  const int r = lane / LPR, c = lane - r * LPR;
  const char *kc = static_cast<const char *>(a.k_cache) + (size_t)u * a.cap * RB;
  const char *vc = static_cast<const char *>(a.v_cache) + (size_t)u * a.cap * RB;
  const char *kn = static_cast<const char *>(a.k_new) + (size_t)u * RB;
  const char *vn = static_cast<const char *>(a.v_new) + (size_t)u * RB;
  float *lg = a.ws.logits + (size_t)u * a.cap * G;

  uint4 qf[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
    qf[g] = *reinterpret_cast<const uint4 *>(static_cast<const char *>(a.q) +
                                             ((size_t)(b * a.Hq + j * G + g) * D + c * CH) * EL);
  float m[G], l[G], acc[G][CH];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < CH; ++e) acc[g][e] = 0.f;
  }
  for (int cbase = t0; cbase < t1; cbase += TC) {
    if (cbase != t0) __syncthreads();  // every wave is done with the previous chunk
    // All sub-chunks of the chunk go out at once; each is consumed as it lands.
#pragma unroll
    for (int sc = 0; sc < NSUB; ++sc) {
      const int c0 = cbase + sc * TS;
      stage_sub<RB, NI>(smem + sc * 2 * SUBB, smem + sc * 2 * SUBB + SUBB, kc, vc, kn, vn, c0,
                        max(0, min(TS, t1 - c0)), t0, Lold, wave, lane);
    }
#pragma unroll
    for (int sc = 0; sc < NSUB; ++sc) {
      const int c0 = cbase + sc * TS;
      if (sc == 0) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NI * (NSUB - 1)) : "memory");
      else if (sc == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NI * (NSUB - 2)) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (c0 >= t1) continue;  // uniform: nothing left in this chunk
      const char *kb = smem + sc * 2 * SUBB;
      const char *vb = kb + SUBB;
      const int nrows = min(TS, t1 - c0);
      float sl[UR][G];
      uint4 vf[UR];
#pragma unroll
      for (int i = 0; i < UR; ++i) {
        const int row = wave * (TS / 4) + i * TPW + r;
        const bool ok = row < nrows;
        const uint4 kf = *reinterpret_cast<const uint4 *>(kb + row * RB + c * 16);
        vf[i] = *reinterpret_cast<const uint4 *>(vb + row * RB + c * 16);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float d;
          if constexpr (EL == 2) {
            d = dot2_bf16(qf[g].x, kf.x, 0.f);
            d = dot2_bf16(qf[g].y, kf.y, d);
            d = dot2_bf16(qf[g].z, kf.z, d);
            d = dot2_bf16(qf[g].w, kf.w, d);
          } else {
            d = __uint_as_float(qf[g].x) * __uint_as_float(kf.x);
            d = fmaf(__uint_as_float(qf[g].y), __uint_as_float(kf.y), d);
            d = fmaf(__uint_as_float(qf[g].z), __uint_as_float(kf.z), d);
            d = fmaf(__uint_as_float(qf[g].w), __uint_as_float(kf.w), d);
          }
          d = row_sum<LPR>(d) * a.scale_log2;
          sl[i][g] = ok ? d : -INFINITY;
        }
        if (c == 0 && ok) {
          float *dst = lg + (size_t)(c0 + row) * G;
          if constexpr (G % 4 == 0) {
#pragma unroll
            for (int g = 0; g < G; g += 4)
              *reinterpret_cast<float4 *>(dst + g) = make_float4(sl[i][g], sl[i][g + 1], sl[i][g + 2], sl[i][g + 3]);
          } else if constexpr (G == 2) {
            *reinterpret_cast<float2 *>(dst) = make_float2(sl[i][0], sl[i][1]);
          } else {
            dst[0] = sl[i][0];
          }
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float mx = m[g];
#pragma unroll
        for (int i = 0; i < UR; ++i) mx = fmaxf(mx, sl[i][g]);
        const float mxs = (mx == -INFINITY) ? 0.f : mx;
        const float corr = fast_exp2(m[g] - mxs);
        float ls = l[g] * corr;
#pragma unroll
        for (int e = 0; e < CH; ++e) acc[g][e] *= corr;
#pragma unroll
        for (int i = 0; i < UR; ++i) {
          const float p = fast_exp2(sl[i][g] - mxs);
          ls += p;
          if constexpr (EL == 2) {
            const uint32_t *vw = reinterpret_cast<const uint32_t *>(&vf[i]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[g][2 * e] = fmaf(p, bf_lo(vw[e]), acc[g][2 * e]);
              acc[g][2 * e + 1] = fmaf(p, bf_hi(vw[e]), acc[g][2 * e + 1]);
            }
          } else {
            const float *vv = reinterpret_cast<const float *>(&vf[i]);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[g][e] = fmaf(p, vv[e], acc[g][e]);
          }
        }
        l[g] = ls;
        m[g] = mx;
      }
    }
  }
  if (a.hp.n && tid == 0 && len_dev != pl.L - 1) set_status(a.ws.status, HIKV_EINVAL);
  // Merge the NS = 4 * TPW row streams into the tile partial.
  constexpr int NS = 4 * TPW;
  constexpr bool kLdsMerge = NS * G * D * 4 + NS * G * 8 + G * 8 <= NSUB * 2 * SUBB;
  __syncthreads();  // the staging buffers become merge scratch
  if constexpr (kLdsMerge) {
    // Every stream writes its (m, l, P.V) to LDS; no cross-lane shuffles.
    float *s_acc = reinterpret_cast<float *>(smem);   // [NS][G][D]
    float *s_m = s_acc + NS * G * D;                  // [NS][G]
    float *s_l = s_m + NS * G;                        // [NS][G]
    float *s_M = s_l + NS * G;                        // [G] tile max, then [G] tile sum
    const int sid = wave * TPW + r;
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < CH; e += 4)
        *reinterpret_cast<float4 *>(s_acc + (sid * G + g) * D + c * CH + e) =
            make_float4(acc[g][e], acc[g][e + 1], acc[g][e + 2], acc[g][e + 3]);
      if (c == 0) {
        s_m[sid * G + g] = m[g];
        s_l[sid * G + g] = l[g];
      }
    }
    __syncthreads();
    if (tid < G) {
      float M = -INFINITY;
      for (int q = 0; q < NS; ++q) M = fmaxf(M, s_m[q * G + tid]);
      const float Ms = (M == -INFINITY) ? 0.f : M;
      float lv = 0.f;
      for (int q = 0; q < NS; ++q) {
        const float f = fast_exp2(s_m[q * G + tid] - Ms);
        s_m[q * G + tid] = f;  // becomes the stream's rescale factor
        lv += s_l[q * G + tid] * f;
      }
      s_M[tid] = M;
      s_M[G + tid] = lv;
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += kThreads) {
      const int g = idx / D;
      float av = 0.f;
#pragma unroll
      for (int q = 0; q < NS; ++q) av += s_acc[(q * G) * D + idx] * s_m[q * G + g];
      a.ws.part_acc[(size_t)tile * G * D + idx] = av;
      if (idx - g * D == 0)
        *reinterpret_cast<float2 *>(a.ws.part_ml + ((size_t)tile * G + g) * 2) = make_float2(s_M[g], s_M[G + g]);
    }
  } else {
    // Rows of each wave through shuffles, then the waves through LDS.
#pragma unroll
    for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mo = __shfl_xor(m[g], off), lo = __shfl_xor(l[g], off);
        const float mx = fmaxf(m[g], mo);
        const float mxs = (mx == -INFINITY) ? 0.f : mx;
        const float ea = fast_exp2(m[g] - mxs), eb = fast_exp2(mo - mxs);
        l[g] = l[g] * ea + lo * eb;
#pragma unroll
        for (int e = 0; e < CH; ++e) acc[g][e] = acc[g][e] * ea + __shfl_xor(acc[g][e], off) * eb;
        m[g] = mx;
      }
    }
    if (r == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < CH; ++e) sm_acc[wave][g][c * CH + e] = acc[g][e];
      if (c == 0)
#pragma unroll
        for (int g = 0; g < G; ++g) {
          sm_ml[wave][g][0] = m[g];
          sm_ml[wave][g][1] = l[g];
        }
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += kThreads) {
      const int g = idx / D, d = idx - g * D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_ml[w][g][0]);
      const float Ms = (M == -INFINITY) ? 0.f : M;
      float av = 0.f, lv = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float e = fast_exp2(sm_ml[w][g][0] - Ms);
        av += sm_acc[w][g][d] * e;
        lv += sm_ml[w][g][1] * e;
      }
      a.ws.part_acc[((size_t)tile * G + g) * D + d] = av;
      if (d == 0) *reinterpret_cast<float2 *>(a.ws.part_ml + ((size_t)tile * G + g) * 2) = make_float2(M, lv);
    }
  }
}

// ---------------------------------------------------------------------------
// K2: unit statistics, output, importance, eviction.
// ---------------------------------------------------------------------------
template <int EL, int D, int G>
__global__ __launch_bounds__(kThreads) void k_finalize(StepArgs a) {
  constexpr int RB = D * EL;
  __shared__ float sm_stat[G][2];
  __shared__ uint64_t sk[4];
  __shared__ int ss[4];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int u, s, nt, L, T;
  if (a.hp.n) {
    const Plan pl = host_plan(a, blockIdx.x);
    if (!pl.valid) return;
    u = pl.u, s = pl.s, nt = pl.nt, L = pl.L, T = pl.T;
    if (unit_error(a, u, L - 1, 1)) return;  // device-side error: unit left alone
  } else {
    const int4 rec = reinterpret_cast<const int4 *>(a.ws.tinfo)[blockIdx.x];
    if (rec.x < 0) return;
    u = rec.x, s = rec.y, nt = rec.z, L = rec.w;
    T = a.ws.plan[0];
  }
  const int b = u / a.Hkv, j = u - b * a.Hkv;
  const int Lold = L - 1, t0 = s * T, t1 = min(t0 + T, L);
  const int tile = blockIdx.x, tb = tile - s;
  const int beta = unit_budget(a, u);
  const int S = a.n_sink, Wp = min(a.n_recent, beta - S), newest = a.new_pos[b];
  const bool over = L > beta;
  const int n_evict = over ? L - beta : 0;
  const bool bulk = n_evict > 1;
  const float *lg = a.ws.logits + (size_t)u * a.cap * G;
  float *impw = a.imp + (size_t)u * a.cap;
  int32_t *posw = a.pos + (size_t)u * a.cap;

  // Own tokens' operands first (independent of the unit statistics).
  const int n_first = t0 + tid;
  float imp_first = 0.f;
  int pos_first = newest;
  float lg_first[G];
  if (n_first < t1) {
#pragma unroll
    for (int g = 0; g < G; ++g) lg_first[g] = lg[(size_t)n_first * G + g];
    if (n_first != Lold) {
      imp_first = impw[n_first];
      pos_first = posw[n_first];
    }
  }

  // Unit statistics per head (a wave per head, lanes over tiles).
  for (int g = wave; g < G; g += 4) {
    float Mx = -INFINITY, ls = 0.f;
    for (int t0r = 0; t0r < nt; t0r += 256) {
      float2 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int t = t0r + lane + 64 * k;
        v[k] = (t < nt) ? *reinterpret_cast<const float2 *>(a.ws.part_ml + ((size_t)(tb + t) * G + g) * 2)
                        : make_float2(-INFINITY, 0.f);
      }
      float mr = fmaxf(fmaxf(v[0].x, v[1].x), fmaxf(v[2].x, v[3].x));
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mr = fmaxf(mr, __shfl_xor(mr, off));
      const float mn = fmaxf(Mx, mr);
      const float mns = (mn == -INFINITY) ? 0.f : mn;
      float part = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) part += v[k].y * fast_exp2(v[k].x - mns);
      part = wave_sum(part);
      ls = ls * fast_exp2(Mx - mns) + part;
      Mx = mn;
    }
    if (lane == 0) {
      sm_stat[g][0] = Mx;
      sm_stat[g][1] = ls;
    }
  }
  __syncthreads();

  // This tile's slice of the output.  Lanes run over the unit's tiles (LO
  // lanes per output, loads issued first), a butterfly over those lanes sums
  // them in a fixed order.
  {
    const int per = (G * D + nt - 1) / nt;
    const int o0 = min(s * per, G * D), o1 = min(o0 + per, G * D);
    const int n_o = o1 - o0;
    int LO = 1;
    while (LO < nt && LO < 64) LO <<= 1;
    const int OW = 64 / LO;                 // outputs per wave per round
    const int sub = lane / LO, tl = lane - sub * LO;
    for (int ob = wave * OW; ob < n_o; ob += 4 * OW) {
      const int oo = ob + sub;
      const bool ok_o = oo < n_o;
      const int o = o0 + (ok_o ? oo : 0), g = o / D;
      const float Ms = (sm_stat[g][0] == -INFINITY) ? 0.f : sm_stat[g][0];
      float av = 0.f;
      for (int tb0 = 0; tb0 < nt; tb0 += 4 * LO) {
        float va[4], vm[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int t = tb0 + tl + k * LO;
          const bool ok = ok_o && t < nt;
          va[k] = ok ? a.ws.part_acc[((size_t)(tb + t) * G) * D + o] : 0.f;
          vm[k] = ok ? a.ws.part_ml[((size_t)(tb + t) * G + g) * 2] : -INFINITY;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) av += va[k] * fast_exp2(vm[k] - Ms);
      }
      for (int off = LO / 2; off > 0; off >>= 1) av += __shfl_xor(av, off);
      if (ok_o && tl == 0) a.out[((size_t)(b * a.Hq + j * G)) * D + o] = av / sm_stat[g][1];
    }
  }

  // Importance of this tile's tokens; lowest eviction key among candidates.
  float Mg[G], ILg[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    Mg[g] = sm_stat[g][0];
    ILg[g] = 1.f / sm_stat[g][1];
  }
  uint64_t best = ~0ull;
  int best_slot = -1;
  for (int n = n_first; n < t1; n += kThreads) {
    const bool first = n == n_first;
    float p = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) p += fast_exp2((first ? lg_first[g] : lg[(size_t)n * G + g]) - Mg[g]) * ILg[g];
    const float io = first ? imp_first : ((n == Lold) ? 0.f : impw[n]);
    const int pn = first ? pos_first : ((n == Lold) ? newest : posw[n]);
    const float iv = io + p;
    // Agent-scope (write-through) stores: the unit's last tile may overwrite
    // the victim's slot in this launch, and a dirty copy in this XCD's L2
    // must not be written back over it later.
    if (n == Lold) st_ag(a.ws.fz_newimp + u, iv);
    else st_ag(impw + n, iv);
    if (over && !((pn < S) || (pn > newest - Wp))) {
      const uint64_t k = evict_key(iv, pn);
      if (k < best) {
        best = k;
        best_slot = n;
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t ko = __shfl_xor(best, off);
    const int so = __shfl_xor(best_slot, off);
    if (ko < best) {
      best = ko;
      best_slot = so;
    }
  }
  if (lane == 0) {
    sk[wave] = best;
    ss[wave] = best_slot;
  }
  __syncthreads();
  if (tid == 0) {
    uint64_t kk = sk[0];
    int vs = ss[0];
    for (int w = 1; w < 4; ++w)
      if (sk[w] < kk) {
        kk = sk[w];
        vs = ss[w];
      }
    st_ag(a.ws.tile_key + tile, kk);
    st_ag(a.ws.tile_slot + tile, vs);
  }
  wait_vmem();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(a.ws.ticket + u, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (uint32_t)(nt - 1);
  }
  __syncthreads();
  if (!s_last) return;

  // ---------------- tail: the unit's last tile ----------------
  asm volatile("" ::: "memory");
  const char *kn = static_cast<const char *>(a.k_new) + (size_t)u * RB;
  const char *vn = static_cast<const char *>(a.v_new) + (size_t)u * RB;
  char *kw = static_cast<char *>(a.k_w) + (size_t)u * a.cap * RB;
  char *vw = static_cast<char *>(a.v_w) + (size_t)u * a.cap * RB;
  const float newimp = ld_ag(a.ws.fz_newimp + u);
  int dst = Lold;  // slot that receives the new token; -1 when it is evicted itself
  if (n_evict == 1) {
    if (wave == 0) {
      uint64_t kk = ~0ull;
      int vs = -1;
      for (int t = lane; t < nt; t += 64) {
        const uint64_t k = ld_ag(a.ws.tile_key + tb + t);
        const int sl = ld_ag(a.ws.tile_slot + tb + t);
        if (k < kk) {
          kk = k;
          vs = sl;
        }
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const uint64_t ko = __shfl_xor(kk, off);
        const int so = __shfl_xor(vs, off);
        if (ko < kk) {
          kk = ko;
          vs = so;
        }
      }
      if (lane == 0) s_last = vs;
    }
    __syncthreads();
    dst = (s_last == Lold) ? -1 : s_last;
  }
  if (dst >= 0) {
    for (int i = tid; i < RB / 16; i += kThreads) {
      reinterpret_cast<uint4 *>(kw + (size_t)dst * RB)[i] = reinterpret_cast<const uint4 *>(kn)[i];
      reinterpret_cast<uint4 *>(vw + (size_t)dst * RB)[i] = reinterpret_cast<const uint4 *>(vn)[i];
    }
    if (tid == 0) {
      posw[dst] = newest;
      impw[dst] = newimp;
    }
  }
  if (!bulk) {
    if (tid == 0 && a.len[u] != L - n_evict) a.len[u] = L - n_evict;
  } else {
    // The unit now holds L contiguous slots: select the n_evict lowest keys
    // among the unprotected tokens and compact.
    __syncthreads();
    __shared__ uint32_t hist[256];
    __shared__ int sc[kThreads];
    __shared__ RadixState rs;
    auto cand_key = [&](int n, uint64_t &key) -> bool {
      const int pn = (n == Lold) ? newest : posw[n];
      if ((pn < S) || (pn > newest - Wp)) return false;
      key = evict_key((n == Lold) ? newimp : ld_ag(impw + n), pn);
      return true;
    };
    radix_select_smallest<kThreads>(L, n_evict, cand_key, hist, &rs);
    const uint64_t prefix = rs.prefix;
    const int shift = rs.shift;
    auto evicted = [&](int n) -> bool {
      uint64_t key;
      if (!cand_key(n, key)) return false;
      return (key >> shift) <= (prefix >> shift);
    };
    const int per = (L + kThreads - 1) / kThreads;
    const int n0 = min(tid * per, L), n1 = min(n0 + per, L);
    int nh = 0, nm = 0;
    for (int n = n0; n < n1; ++n) {
      const bool e = evicted(n);
      nh += (n < beta && e);
      nm += (n >= beta && !e);
    }
    int tot_h, tot_m;
    int oh = block_excl_scan<kThreads>(nh, sc, &tot_h);
    int om = block_excl_scan<kThreads>(nm, sc, &tot_m);
    int32_t *holes = a.ws.holes + (size_t)u * a.cap;
    int32_t *movers = a.ws.movers + (size_t)u * a.cap;
    for (int n = n0; n < n1; ++n) {
      const bool e = evicted(n);
      if (n < beta && e) holes[oh++] = n;
      if (n >= beta && !e) movers[om++] = n;
    }
    __syncthreads();
    if (tot_h == tot_m) {
      constexpr int CPR = RB / 16;
      for (int idx = tid; idx < tot_m * CPR; idx += kThreads) {
        const int i = idx / CPR, ci = idx - i * CPR;
        const int src = movers[i], dd = holes[i];
        reinterpret_cast<uint4 *>(kw + (size_t)dd * RB)[ci] = reinterpret_cast<const uint4 *>(kw + (size_t)src * RB)[ci];
        reinterpret_cast<uint4 *>(vw + (size_t)dd * RB)[ci] = reinterpret_cast<const uint4 *>(vw + (size_t)src * RB)[ci];
      }
      for (int i = tid; i < tot_m; i += kThreads) {
        const int src = movers[i], dd = holes[i];
        posw[dd] = (src == Lold) ? newest : posw[src];
        impw[dd] = (src == Lold) ? newimp : ld_ag(impw + src);
      }
      if (tid == 0) a.len[u] = beta;
    } else if (tid == 0) {
      set_status(a.ws.status, HIKV_EINVAL);
    }
  }
  if (tid == 0) a.ws.ticket[u] = 0;
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
template <int EL, int D, int G>
static int attend_grid(int n_units) {
  static int per_cu_cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (per_cu_cache[dev] == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_attend<EL, D, G>, kThreads, 0) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    per_cu_cache[dev] = per_cu * cus;
  }
  // One resident round of tiles, and at least 64 tiles beyond one per unit.
  return min(max(per_cu_cache[dev], n_units + 64), kMaxGrid);
}

template <int EL, int D, int G>
static hipError_t step_go(const StepArgs &a, hipStream_t s) {
  const int g = attend_grid<EL, D, G>(a.n_units);
  if (g <= 0) return hipErrorInvalidValue;
  const dim3 grid(g), block(kThreads);
  hipLaunchKernelGGL((k_attend<EL, D, G>), grid, block, 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_finalize<EL, D, G>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int EL, int D>
static hipError_t step_g(const StepArgs &a, hipStream_t s) {
  switch (a.G) {
    case 1: return step_go<EL, D, 1>(a, s);
    case 2: return step_go<EL, D, 2>(a, s);
    case 4: return step_go<EL, D, 4>(a, s);
    case 8: return step_go<EL, D, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// Fill a.hp from a host copy of len[] exactly as the kernels would derive the
// plan from the device copy.  Returns false when no host plan applies.
template <int EL, int D, int G>
static bool host_plan_fill(StepArgs &a, const int32_t *len_hint) {
  const int U = a.n_units;
  if (U > kHostPlanUnits) return false;
  const int g = attend_grid<EL, D, G>(U);
  if (g <= U) return false;
  long long tot = 0;
  for (int u = 0; u < U; ++u) tot += len_hint[u] + 1;
  const int ntarget = g - U;
  const long long tt = (tot + ntarget - 1) / ntarget;
  int T = (int)((tt + 15) / 16 * 16);
  if (T < 16) T = 16;
  int base = 0;
  for (int u = 0; u < U; ++u) {
    a.hp.base[u] = base;
    a.hp.L[u] = len_hint[u] + 1;
    base += (a.hp.L[u] + T - 1) / T;
  }
  a.hp.base[U] = base;
  a.hp.ntiles = base;
  a.hp.T = T;
  a.hp.n = U;
  return base <= g;  // every tile gets a workgroup
}

template <int EL, int D>
static bool host_plan_g(StepArgs &a, const int32_t *len_hint) {
  switch (a.G) {
    case 1: return host_plan_fill<EL, D, 1>(a, len_hint);
    case 2: return host_plan_fill<EL, D, 2>(a, len_hint);
    case 4: return host_plan_fill<EL, D, 4>(a, len_hint);
    case 8: return host_plan_fill<EL, D, 8>(a, len_hint);
    default: return false;
  }
}

bool step_host_plan(StepArgs &a, int dtype, const int32_t *len_hint) {
  a.hp.n = 0;
  bool ok = false;
  if (dtype == HIKV_BF16) {
    if (a.D == 128) ok = host_plan_g<2, 128>(a, len_hint);
    else if (a.D == 64) ok = host_plan_g<2, 64>(a, len_hint);
  } else {
    if (a.D == 128) ok = host_plan_g<4, 128>(a, len_hint);
    else if (a.D == 64) ok = host_plan_g<4, 64>(a, len_hint);
  }
  if (!ok) a.hp.n = 0;
  return ok;
}

hipError_t launch_step(const StepArgs &a, int dtype, hipStream_t s) {
  if (dtype == HIKV_BF16) {
    if (a.D == 128) return step_g<2, 128>(a, s);
    if (a.D == 64) return step_g<2, 64>(a, s);
  } else {
    if (a.D == 128) return step_g<4, 128>(a, s);
    if (a.D == 64) return step_g<4, 64>(a, s);
  }
  return hipErrorInvalidValue;
}


}  // namespace hikv
