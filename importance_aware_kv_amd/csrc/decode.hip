// decode.hip -- decode-step kernels: split-K attention tiles, tile merge,
// importance accumulation with the steady single eviction, and bulk
// radix-select eviction with in-place compaction.
//
// Method (pages cited by title and section):
//  * decode GeMVs: logits q.K^T, P = softmax, O = P.V -- "HiKV", Sec. II-A.
//  * importance: every cached token accumulates the attention probability it
//    receives, summed over the q-heads that share its KV head -- "KV Cache
//    Compression and Dynamic Pruning in Production Serving", Sec. 3 (H2O)
//    and Sec. 5 (GQA pooling); "HiKV", Sec. III-B.
//  * eviction: over budget, drop the lowest-importance tokens but never the
//    first S positions nor the W' newest ones (same blog page, Sec. 3,
//    StreamingLLM and H2O); per KV head ("Kelle" summary, Sec. 4.1).
//  * slots are unordered, so a survivor can fill any hole ("Kelle" summary,
//    Sec. 2.2): compaction moves survivors from above the budget into the
//    holes below it.
//
// MI355X mapping.  A token row of K (or V) is D*el bytes; LPR lanes hold one
// row with 16 bytes each (bf16 D=128: 16 lanes x 8 channels), so one wave64
// load instruction fetches TPW full rows, perfectly coalesced.  The q.k dot
// product is reduced over the row's lanes with DPP (quad_perm, row mirrors),
// which leaves the logit in every lane of the row; each row then runs its own
// online softmax over the tokens it sees, so the inner loop needs no LDS and
// no barrier.  Rows, waves and finally tiles are merged with the usual
// max/rescale rule.  Logits are kept in the log2 domain (scale * log2 e) so
// every exponential is a single v_exp_f32.

#include <hip/hip_ext.h>

#include "hikv_block.h"
#include "hikv_launch.h"
#include "hikv_stats.h"

namespace hikv {

// ---------------------------------------------------------------------------
// Split-K tile plan.  Units are cut into tiles of T tokens, T chosen so the
// whole step yields about kTilesTarget tiles (>= 2 per CU) whatever the mix
// of per-head lengths: ragged budgets are balanced by construction.  Every
// workgroup of the attention kernel derives the same plan from len[]; block 0
// also stores it for the later kernels of the step.
// ---------------------------------------------------------------------------
struct TileInfo {
  int u, t0, t1, L, valid;
};

struct PlanShared {
  int sc[256];
  long long ll[256];
  int info[5];
};

__device__ TileInfo plan_locate(const StepArgs &a, int tile, bool store, PlanShared &ps) {
  const int tid = threadIdx.x;
  const int U = a.n_units;
  const int per = (U + 255) / 256;
  const int u0 = min(tid * per, U), u1 = min(u0 + per, U);
  long long mine = 0;
  for (int u = u0; u < u1; ++u) {
    const int len = a.len[u];
    const int err = unit_error(a, u, len, 1);
    if (err) {
      if (store) set_status(a.ws.status, err);
      continue;
    }
    mine += len + 1;
  }
  const long long total = block_sum_ll<256>(mine, ps.ll);
  long long tt = (total + kTilesTarget - 1) / kTilesTarget;
  int T = (int)(((tt + kTileMin - 1) / kTileMin) * kTileMin);
  if (T < kTileMin) T = kTileMin;
  int my_tiles = 0;
  for (int u = u0; u < u1; ++u) {
    const int len = a.len[u];
    if (unit_error(a, u, len, 1)) continue;
    my_tiles += (len + 1 + T - 1) / T;
  }
  int total_tiles;
  const int base = block_excl_scan<256>(my_tiles, ps.sc, &total_tiles);
  if (tid == 0) ps.info[4] = 0;
  __syncthreads();
  int bcur = base;
  for (int u = u0; u < u1; ++u) {
    const int len = a.len[u];
    const int nt = unit_error(a, u, len, 1) ? 0 : (len + 1 + T - 1) / T;
    if (store) a.ws.plan[u] = bcur;
    if (tile >= bcur && tile < bcur + nt) {
      const int lt = tile - bcur;
      ps.info[0] = u;
      ps.info[1] = lt * T;
      ps.info[2] = min(lt * T + T, len + 1);
      ps.info[3] = len + 1;
      ps.info[4] = 1;
    }
    bcur += nt;
  }
  if (store && tid == 0) {
    a.ws.plan[U] = total_tiles;
    a.ws.plan[U + 1] = T;
  }
  __syncthreads();
  TileInfo ti;
  ti.valid = ps.info[4];
  ti.u = ps.info[0];
  ti.t0 = ps.info[1];
  ti.t1 = ps.info[2];
  ti.L = ps.info[3];
  return ti;
}

// The unit of a tile: the last unit whose first tile is at or before it
// (a unit without tiles shares its successor's first tile).  Called by whole
// waves with a uniform tile: every lane loads its share of the table at once
// (from clamped addresses) and the wave counts, one round trip for up to 256
// units instead of a dependent load per step of a binary search.
__device__ __forceinline__ int plan_unit(const int32_t *plan, int U, int tile) {
  const int lane = threadIdx.x & 63;
  int cnt = 0;
  for (int i0 = 0; i0 < U; i0 += 256) {
    int v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = plan[min(i0 + 64 * q + lane, U - 1)];
#pragma unroll
    for (int q = 0; q < 4; ++q) cnt += __popcll(__ballot(i0 + 64 * q + lane < U && v[q] <= tile));
  }
  return cnt - 1;  // plan[0] = 0: at least one
}
__device__ __forceinline__ int plan_ntiles(const int32_t *plan, int U, int u) {
  return plan[u + 1 < U ? u + 1 : U] - plan[u];
}

// ---------------------------------------------------------------------------
// Kernel A: split-K attention tiles.
// ---------------------------------------------------------------------------
template <int EL, int D, int G>
struct Lay {
  static constexpr int CH = 16 / EL;            // channels per lane
  static constexpr int LPR = D / CH;            // lanes per token row
  static constexpr int TPW = kWave / LPR;       // rows per wave instruction
  static constexpr int TOKW = (G >= 8) ? 8 : 16;
  static constexpr int U = (TOKW / TPW) > 0 ? TOKW / TPW : 1;  // row groups in flight
};

template <int EL, int D, int G, bool WITH_V, bool MASKED>
__global__ __launch_bounds__(256) void k_attn_tiles(StepArgs a) {
  using LY = Lay<EL, D, G>;
  constexpr int CH = LY::CH, LPR = LY::LPR, TPW = LY::TPW, U = LY::U;
  constexpr int RB = D * EL;  // row bytes
  __shared__ PlanShared ps;
  __shared__ float sm_ml[4][G][2];
  __shared__ float sm_acc[WITH_V ? 4 : 1][G][WITH_V ? D : 1];

  const TileInfo ti = plan_locate(a, blockIdx.x, blockIdx.x == 0, ps);
  if (!ti.valid) return;
  const int u = ti.u, b = u / a.Hkv, j = u - b * a.Hkv;
  const int Lold = ti.L - 1, t0 = ti.t0, t1 = ti.t1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane / LPR, c = lane - r * LPR;

  const char *kc = static_cast<const char *>(a.k_cache) + (size_t)u * a.cap * RB;
  const char *vc = static_cast<const char *>(a.v_cache) + (size_t)u * a.cap * RB;
  const char *kn = static_cast<const char *>(a.k_new) + (size_t)u * RB;
  const char *vn = static_cast<const char *>(a.v_new) + (size_t)u * RB;

  // Append: the tile holding slot Lold copies the new row in (nobody else
  // reads that slot during this kernel; this tile reads it from k_new).
  if (t0 <= Lold && Lold < t1) {
    for (int i = tid; i < RB / 16; i += 256) {
      reinterpret_cast<uint4 *>(static_cast<char *>(a.k_w) + ((size_t)u * a.cap + Lold) * RB)[i] =
          reinterpret_cast<const uint4 *>(kn)[i];
      reinterpret_cast<uint4 *>(static_cast<char *>(a.v_w) + ((size_t)u * a.cap + Lold) * RB)[i] =
          reinterpret_cast<const uint4 *>(vn)[i];
    }
    if (tid == 0) a.pos[(size_t)u * a.cap + Lold] = a.new_pos[b];
  }

  // q fragments of the group's G heads (channels c*CH .. c*CH+CH-1).
  uint4 qf[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int h = j * G + g;
    qf[g] = *reinterpret_cast<const uint4 *>(static_cast<const char *>(a.q) +
                                             ((size_t)(b * a.Hq + h) * D + c * CH) * EL);
    if constexpr (MASKED) {
      const uint32_t w = a.ws.chmask[(size_t)(b * a.Hq + h) * (D / 32) + (c * CH) / 32];
      const uint32_t bits = (w >> ((c * CH) & 31)) & ((1u << CH) - 1u);
      uint32_t *qw = reinterpret_cast<uint32_t *>(&qf[g]);
      if constexpr (EL == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t m = ((bits >> (2 * e)) & 1u ? 0x0000ffffu : 0u) |
                             ((bits >> (2 * e + 1)) & 1u ? 0xffff0000u : 0u);
          qw[e] &= m;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) qw[e] = ((bits >> e) & 1u) ? qw[e] : 0u;
      }
    }
  }

  float m[G], l[G], acc[G][WITH_V ? CH : 1];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < (WITH_V ? CH : 1); ++e) acc[g][e] = 0.f;
  }
  float *lg = a.ws.logits + (size_t)u * a.cap * G;

  for (int base = t0 + wave * TPW * U; base < t1; base += 4 * TPW * U) {
    uint4 kf[U], vf[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int n = base + i * TPW + r;
      const bool ok = n < t1;
      const char *krow = (n == Lold) ? kn : kc + (size_t)n * RB;
      kf[i] = ok ? *reinterpret_cast<const uint4 *>(krow + c * 16) : make_uint4(0, 0, 0, 0);
      if constexpr (WITH_V) {
        const char *vrow = (n == Lold) ? vn : vc + (size_t)n * RB;
        vf[i] = ok ? *reinterpret_cast<const uint4 *>(vrow + c * 16) : make_uint4(0, 0, 0, 0);
      }
    }
    float s[U][G];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int n = base + i * TPW + r;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d;
        if constexpr (EL == 2) {
          d = dot2_bf16(qf[g].x, kf[i].x, 0.f);
          d = dot2_bf16(qf[g].y, kf[i].y, d);
          d = dot2_bf16(qf[g].z, kf[i].z, d);
          d = dot2_bf16(qf[g].w, kf[i].w, d);
        } else {
          d = __uint_as_float(qf[g].x) * __uint_as_float(kf[i].x);
          d = fmaf(__uint_as_float(qf[g].y), __uint_as_float(kf[i].y), d);
          d = fmaf(__uint_as_float(qf[g].z), __uint_as_float(kf[i].z), d);
          d = fmaf(__uint_as_float(qf[g].w), __uint_as_float(kf[i].w), d);
        }
        d = row_sum<LPR>(d) * a.scale_log2;
        s[i][g] = (n < t1) ? d : -INFINITY;
      }
      if (c == 0 && n < t1) {
        float *dst = lg + (size_t)n * G;
        if constexpr (G % 4 == 0) {
#pragma unroll
          for (int g = 0; g < G; g += 4)
            *reinterpret_cast<float4 *>(dst + g) = make_float4(s[i][g], s[i][g + 1], s[i][g + 2], s[i][g + 3]);
        } else if constexpr (G == 2) {
          *reinterpret_cast<float2 *>(dst) = make_float2(s[i][0], s[i][1]);
        } else {
          dst[0] = s[i][0];
        }
      }
    }
    // Online softmax of this row's U tokens.
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = m[g];
#pragma unroll
      for (int i = 0; i < U; ++i) mx = fmaxf(mx, s[i][g]);
      const float mxs = (mx == -INFINITY) ? 0.f : mx;
      const float corr = fast_exp2(m[g] - mxs);
      float lsum = l[g] * corr;
      if constexpr (WITH_V) {
#pragma unroll
        for (int e = 0; e < CH; ++e) acc[g][e] *= corr;
      }
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const float p = fast_exp2(s[i][g] - mxs);
        lsum += p;
        if constexpr (WITH_V) {
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
      }
      l[g] = lsum;
      m[g] = mx;
    }
  }

  // Merge the TPW rows of each wave (rows are LPR lanes apart).
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(m[g], off);
      const float lo = __shfl_xor(l[g], off);
      const float mx = fmaxf(m[g], mo);
      const float mxs = (mx == -INFINITY) ? 0.f : mx;
      const float ea = fast_exp2(m[g] - mxs), eb = fast_exp2(mo - mxs);
      l[g] = l[g] * ea + lo * eb;
      if constexpr (WITH_V) {
#pragma unroll
        for (int e = 0; e < CH; ++e) acc[g][e] = acc[g][e] * ea + __shfl_xor(acc[g][e], off) * eb;
      }
      m[g] = mx;
    }
  }
  // Merge the 4 waves through LDS and write the tile partial.
  if (r == 0) {
    if constexpr (WITH_V) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < CH; ++e) sm_acc[wave][g][c * CH + e] = acc[g][e];
    }
    if (c == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        sm_ml[wave][g][0] = m[g];
        sm_ml[wave][g][1] = l[g];
      }
    }
  }
  __syncthreads();
  const int tile = blockIdx.x;
  if constexpr (WITH_V) {
    for (int idx = tid; idx < G * D; idx += 256) {
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
      if (d == 0) {
        a.ws.part_ml[((size_t)tile * G + g) * 2] = M;
        a.ws.part_ml[((size_t)tile * G + g) * 2 + 1] = lv;
      }
    }
  } else {
    if (tid < G) {
      const int g = tid;
      float M = -INFINITY;
      for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_ml[w][g][0]);
      const float Ms = (M == -INFINITY) ? 0.f : M;
      float lv = 0.f;
      for (int w = 0; w < 4; ++w) lv += sm_ml[w][g][1] * fast_exp2(sm_ml[w][g][0] - Ms);
      a.ws.part_ml[((size_t)tile * G + g) * 2] = M;
      a.ws.part_ml[((size_t)tile * G + g) * 2 + 1] = lv;
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel B: per unit, merge the tile partials of each q-head.
// ---------------------------------------------------------------------------
template <int D, int G, bool WITH_V>
__global__ __launch_bounds__(256) void k_combine(StepArgs a) {
  const int u = blockIdx.x, tid = threadIdx.x;
  const int U = a.n_units;
  const int b = u / a.Hkv, j = u - b * a.Hkv;
  __shared__ float sM[G], sL[G];
  const int t_begin = a.ws.plan[u];
  const int t_end = (u + 1 < U) ? a.ws.plan[u + 1] : a.ws.plan[U];
  if (t_end <= t_begin) {  // unit skipped by a device-side error
    if constexpr (WITH_V)
      for (int idx = tid; idx < G * D; idx += 256)
        a.out[((size_t)(b * a.Hq + j * G)) * D + idx] = 0.f;
    return;
  }
  if (tid < G) {
    const int g = tid;
    float M = -INFINITY;
    for (int t = t_begin; t < t_end; ++t) M = fmaxf(M, a.ws.part_ml[((size_t)t * G + g) * 2]);
    const float Ms = (M == -INFINITY) ? 0.f : M;
    float ls = 0.f;
    for (int t = t_begin; t < t_end; ++t)
      ls += a.ws.part_ml[((size_t)t * G + g) * 2 + 1] * fast_exp2(a.ws.part_ml[((size_t)t * G + g) * 2] - Ms);
    sM[g] = M;
    sL[g] = ls;
    a.ws.stats[((size_t)u * G + g) * 2] = M;
    a.ws.stats[((size_t)u * G + g) * 2 + 1] = ls;
  }
  __syncthreads();
  if constexpr (WITH_V) {
    for (int idx = tid; idx < G * D; idx += 256) {
      const int g = idx / D, d = idx - g * D;
      const float Ms = (sM[g] == -INFINITY) ? 0.f : sM[g];
      float av = 0.f;
      for (int t = t_begin; t < t_end; ++t)
        av += a.ws.part_acc[((size_t)t * G + g) * D + d] *
              fast_exp2(a.ws.part_ml[((size_t)t * G + g) * 2] - Ms);
      a.out[((size_t)(b * a.Hq + j * G + g)) * D + d] = av / sL[g];
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel C: importance accumulation + steady-state single eviction.
// The last tile of a unit to finish (atomic ticket) picks the victim from the
// per-tile minima and moves the last slot into it; units that must shed more
// than one token are left to the bulk kernel.
// ---------------------------------------------------------------------------
template <int G, int EL, int D>
__global__ __launch_bounds__(256) void k_accumulate(StepArgs a) {
  const int U = a.n_units, tile = blockIdx.x, tid = threadIdx.x;
  const int total_tiles = a.ws.plan[U];
  if (tile >= total_tiles) return;
  const int T = a.ws.plan[U + 1];
  const int u = plan_unit(a.ws.plan, U, tile);
  const int ntile_u = plan_ntiles(a.ws.plan, U, u);
  const int lt = tile - a.ws.plan[u];
  const int b = u / a.Hkv;
  const int L = a.len[u] + 1;
  const int beta = unit_budget(a, u);
  const int S = a.n_sink;
  const int Wp = min(a.n_recent, beta - S);
  const int newest = a.new_pos[b];
  const bool over = L > beta;
  const int t0 = lt * T, t1 = min(t0 + T, L);
  // More than one token over budget needs the bulk eviction, which the host
  // leaves out when the caller's lengths say that no unit needs it.
  if (a.no_bulk && L - beta > 1 && lt == 0 && tid == 0) set_status(a.ws.status, HIKV_EINVAL);
  // HiKV's chunked V side: the unit's first tile adds up the chunks' P.V
  // partials in chunk order (the launch boundary made them visible).
  if (a.s2_chunks && lt == 0) {
    const int Dd = a.D;
    const size_t NC = (size_t)((a.cap + Dd - 1) / Dd);
    const int nc = (L + Dd - 1) / Dd;
    float *outp = a.out + ((size_t)b * a.Hq + (size_t)(u - b * a.Hkv) * G) * Dd;
    const float *ca = a.ws.chunk_acc + (size_t)u * NC * G * Dd;
    for (int i = tid; i < G * Dd; i += 256) {
      float sum = 0.f;
      for (int c0 = 0; c0 < nc; c0 += 8) {  // eight loads in flight, added in chunk order
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = c0 + e < nc ? ca[(size_t)(c0 + e) * G * Dd + i] : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += v[e];
      }
      outp[i] = sum;
    }
    if (a.dbg_count && tid < G) {
      int k = 0;
      for (int cc = 0; cc < nc; ++cc) k += a.ws.chunk_cnt[((size_t)u * NC + cc) * G + tid];
      a.dbg_count[(size_t)b * a.Hq + (size_t)(u - b * a.Hkv) * G + tid] = k;
    }
  }

  float M[G], IL[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float Sg;
    unit_softmax_stats(a, u, g, M[g], Sg);
    IL[g] = 1.f / Sg;
  }
  const float *lg = a.ws.logits + (size_t)u * a.cap * G;
  float *imp = a.imp + (size_t)u * a.cap;
  const int32_t *pos = a.pos + (size_t)u * a.cap;
  uint64_t best = ~0ull;
  int best_slot = -1;
  for (int n = t0 + tid; n < t1; n += 256) {
    float p = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g)  // Kelle's score: the logit itself (stored in log2 units)
      p += a.acc_logit ? lg[(size_t)n * G + g] * 0.69314718055994531f : fast_exp2(lg[(size_t)n * G + g] - M[g]) * IL[g];
    const bool is_new = n == L - 1;
    const int pn = (over || a.acc_recent) ? pos[n] : 0;
    // HiKV's dual bank: only the recent window accumulates; older scores are
    // frozen and not rewritten (the new token's slot is always written).
    const bool acc = !a.acc_recent || pn > newest - Wp;
    const float iv = (is_new ? 0.f : imp[n]) + (acc ? p : 0.f);
    // Written through to memory: the unit's last tile may move slot L - 1's
    // value into the victim's slot, and no slot may be left dirty in two
    // caches.
    if (acc || is_new) store_agent_f(imp + n, iv);
    if (over) {
      const bool prot = (pn < S) || (pn > newest - Wp);
      if (!prot) {
        const uint64_t k = evict_key(iv, pn);
        if (k < best) {
          best = k;
          best_slot = n;
        }
      }
    }
  }
  // Block min of (key, slot).
  __shared__ uint64_t sk[256];
  __shared__ int ss[256];
  __shared__ int last_flag;
  sk[tid] = best;
  ss[tid] = best_slot;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off && sk[tid + off] < sk[tid]) {
      sk[tid] = sk[tid + off];
      ss[tid] = ss[tid + off];
    }
    __syncthreads();
  }
  // The tile's lowest key goes out with device-coherent stores, and every
  // store of the tile is complete before its ticket is taken; the unit's
  // last tile then reads them all with device-coherent loads.  (No cache-wide
  // write-back: a fence here costs more than the whole kernel's work.)
  if (tid == 0) {
    __hip_atomic_store(&a.ws.tile_key[tile], sk[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    store_agent(&a.ws.tile_slot[tile], ss[0]);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) last_flag = ticket_agent(&a.ws.ticket[u]) == (uint32_t)(ntile_u - 1);
  __syncthreads();
  if (!last_flag) return;
  if (over && L - beta == 1) {
    const int tb = a.ws.plan[u];
    if (tid == 0) {
      uint64_t kk = ~0ull;
      int vs = -1;
      for (int t = tb; t < tb + ntile_u; ++t) {
        const uint64_t k = __hip_atomic_load(&a.ws.tile_key[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (k < kk) {
          kk = k;
          vs = load_agent(&a.ws.tile_slot[t]);
        }
      }
      last_flag = vs;  // reuse as victim slot broadcast
    }
    __syncthreads();
    const int v = last_flag;
    const int last = L - 1;
    if (v >= 0 && v != last) {
      constexpr int RB = D * EL;
      char *kw = static_cast<char *>(a.k_w) + (size_t)u * a.cap * RB;
      char *vw = static_cast<char *>(a.v_w) + (size_t)u * a.cap * RB;
      for (int i = tid; i < RB / 16; i += 256) {
        reinterpret_cast<uint4 *>(kw + (size_t)v * RB)[i] = reinterpret_cast<const uint4 *>(kw + (size_t)last * RB)[i];
        reinterpret_cast<uint4 *>(vw + (size_t)v * RB)[i] = reinterpret_cast<const uint4 *>(vw + (size_t)last * RB)[i];
      }
      if (tid == 0) {
        a.pos[(size_t)u * a.cap + v] = pos[last];
        store_agent_f(a.imp + (size_t)u * a.cap + v, __int_as_float(load_agent(reinterpret_cast<const int32_t *>(imp + last))));
      }
    }
    if (tid == 0) a.len[u] = (v >= 0) ? L - 1 : L;
  } else {
    if (tid == 0) a.len[u] = L;
  }
  if (tid == 0) a.ws.ticket[u] = 0;
}

// ---------------------------------------------------------------------------
// Kernel D: bulk eviction of one unit per workgroup.  Radix select (8-bit
// digits, most significant first) finds the boundary of the k lowest
// eviction keys among the unprotected tokens, stopping as soon as the
// boundary bucket is taken whole; then holes below the budget are matched in
// slot order with survivors above it and rows are moved.
// ---------------------------------------------------------------------------
constexpr int kBulkThreads = 1024;

template <int EL, int D>
__global__ __launch_bounds__(kBulkThreads) void k_bulk_evict(StepArgs a, const int32_t *newest_pos,
                                                             int from_decode) {
  const int u = blockIdx.x, tid = threadIdx.x;
  const int b = u / a.Hkv;
  const int L = a.len[u];
  const int beta = unit_budget(a, u);
  if (from_decode) {
    // Units the decode step skipped (device error) have no tiles.
    const int U = a.n_units;
    const int nt = ((u + 1 < U) ? a.ws.plan[u + 1] : a.ws.plan[U]) - a.ws.plan[u];
    if (nt <= 0) return;
  } else {
    if (beta < a.n_sink || beta > a.cap || L > a.cap || L < 0) {
      if (tid == 0) set_status(a.ws.status, HIKV_EBUDGET);
      return;
    }
  }
  if (L <= beta) return;
  const int S = a.n_sink;
  const int Wp = min(a.n_recent, beta - S);
  const int newest = newest_pos[b];
  const float *imp = a.imp + (size_t)u * a.cap;
  const int32_t *pos = a.pos + (size_t)u * a.cap;
  const int k_evict = L - beta;

  // Every slot's eviction key (UINT64_MAX for a protected token), then the
  // selection and compaction.
  uint64_t *keys = a.ws.bkeys + (size_t)u * a.cap;
  constexpr int KB = 8;
  for (int base = 0; base < L; base += kBulkThreads * KB) {
    int pk[KB];
    float ik[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int n = min(base + tid + j * kBulkThreads, L - 1);
      pk[j] = pos[n];
      ik[j] = imp[n];
    }
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int n = base + tid + j * kBulkThreads;
      if (n < L) keys[n] = ((pk[j] < S) || (pk[j] > newest - Wp)) ? ~0ull : evict_key(ik[j], pk[j]);
    }
  }
  __syncthreads();
  __shared__ uint32_t hist[256];
  __shared__ __attribute__((aligned(16))) uint32_t whist[kBulkThreads / 64 * 256];
  __shared__ int sc[kBulkThreads];
  __shared__ RadixState rs;
  constexpr int RB = D * EL;
  bulk_compact<kBulkThreads, RB>(keys, L, beta, k_evict, static_cast<char *>(a.k_w) + (size_t)u * a.cap * RB,
                                 static_cast<char *>(a.v_w) + (size_t)u * a.cap * RB,
                                 a.pos + (size_t)u * a.cap, a.imp + (size_t)u * a.cap,
                                 a.ws.holes + (size_t)u * a.cap, a.ws.movers + (size_t)u * a.cap, a.len + u,
                                 a.ws.status, hist, whist, sc, &rs);
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
template <int EL, int D>
static hipError_t attn_dispatch_g(const StepArgs &a, bool with_v, bool masked, hipStream_t s,
                                 hipEvent_t ev0, hipEvent_t ev1) {
  const dim3 grid(max_tiles_for(a.n_units)), block(256);
  // With events, the dispatch itself records them around the kernel's execution.
  auto go = [&](void (*kern)(StepArgs)) {
    if (ev0 && ev1) hipExtLaunchKernelGGL(kern, grid, block, 0, s, ev0, ev1, 0, a);
    else hipLaunchKernelGGL(kern, grid, block, 0, s, a);
  };
#define HIKV_ATTN(GG)                                                 \
  case GG:                                                            \
    if (with_v && !masked) go(k_attn_tiles<EL, D, GG, true, false>);  \
    else if (!with_v && masked) go(k_attn_tiles<EL, D, GG, false, true>); \
    else if (!with_v && !masked) go(k_attn_tiles<EL, D, GG, false, false>); \
    else go(k_attn_tiles<EL, D, GG, true, true>);                     \
    break;
  switch (a.G) {
    HIKV_ATTN(1)
    HIKV_ATTN(2)
    HIKV_ATTN(4)
    HIKV_ATTN(8)
    default: return hipErrorInvalidValue;
  }
#undef HIKV_ATTN
  return hipGetLastError();
}

hipError_t launch_attn_tiles(const StepArgs &a, int dtype, bool with_v, bool masked, hipStream_t s,
                             hipEvent_t ev0, hipEvent_t ev1) {
  if (dtype == HIKV_BF16) {
    if (a.D == 128) return attn_dispatch_g<2, 128>(a, with_v, masked, s, ev0, ev1);
    if (a.D == 64) return attn_dispatch_g<2, 64>(a, with_v, masked, s, ev0, ev1);
  } else {
    if (a.D == 128) return attn_dispatch_g<4, 128>(a, with_v, masked, s, ev0, ev1);
    if (a.D == 64) return attn_dispatch_g<4, 64>(a, with_v, masked, s, ev0, ev1);
  }
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t combine_dispatch(const StepArgs &a, bool with_v, hipStream_t s) {
  const dim3 grid(a.n_units), block(256);
#define HIKV_COMB(GG)                                                                            \
  case GG:                                                                                       \
    if (with_v) hipLaunchKernelGGL((k_combine<D, GG, true>), grid, block, 0, s, a);              \
    else hipLaunchKernelGGL((k_combine<D, GG, false>), grid, block, 0, s, a);                    \
    break;
  switch (a.G) {
    HIKV_COMB(1)
    HIKV_COMB(2)
    HIKV_COMB(4)
    HIKV_COMB(8)
    default: return hipErrorInvalidValue;
  }
#undef HIKV_COMB
  return hipGetLastError();
}

hipError_t launch_combine(const StepArgs &a, bool with_v, hipStream_t s) {
  if (a.D == 128) return combine_dispatch<128>(a, with_v, s);
  if (a.D == 64) return combine_dispatch<64>(a, with_v, s);
  return hipErrorInvalidValue;
}

template <int EL, int D>
static hipError_t accum_dispatch(const StepArgs &a, hipStream_t s) {
  const dim3 grid(max_tiles_for(a.n_units)), block(256);
  switch (a.G) {
    case 1: hipLaunchKernelGGL((k_accumulate<1, EL, D>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_accumulate<2, EL, D>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_accumulate<4, EL, D>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((k_accumulate<8, EL, D>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_accumulate(const StepArgs &a, int dtype, hipStream_t s) {
  if (dtype == HIKV_BF16) {
    if (a.D == 128) return accum_dispatch<2, 128>(a, s);
    if (a.D == 64) return accum_dispatch<2, 64>(a, s);
  } else {
    if (a.D == 128) return accum_dispatch<4, 128>(a, s);
    if (a.D == 64) return accum_dispatch<4, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bulk_evict(const StepArgs &a, int dtype, const int32_t *newest, bool from_decode,
                             hipStream_t s) {
  const dim3 grid(a.n_units), block(kBulkThreads);
  const int fd = from_decode ? 1 : 0;
  if (dtype == HIKV_BF16) {
    if (a.D == 128) hipLaunchKernelGGL((k_bulk_evict<2, 128>), grid, block, 0, s, a, newest, fd);
    else if (a.D == 64) hipLaunchKernelGGL((k_bulk_evict<2, 64>), grid, block, 0, s, a, newest, fd);
    else return hipErrorInvalidValue;
  } else {
    if (a.D == 128) hipLaunchKernelGGL((k_bulk_evict<4, 128>), grid, block, 0, s, a, newest, fd);
    else if (a.D == 64) hipLaunchKernelGGL((k_bulk_evict<4, 64>), grid, block, 0, s, a, newest, fd);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hikv
