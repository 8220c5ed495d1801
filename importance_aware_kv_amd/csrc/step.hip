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
// K2 k_finalize -- importance blocks (2048 tokens of a unit each) and output
//   blocks.  The launch boundary makes K1's writes visible.  An importance
//   block turns its tokens' logits into probabilities with the unit's
//   statistics, adds them to the importance (with the HiKV dual bank only
//   inside the recent window), and leaves its lowest eviction key in the
//   cache's pending-eviction record; the next call's attention launch takes
//   the lowest of those as the victim, skips it, and the new token is then
//   written into its slot, so no row moves in the steady state.  A unit that
//   must shed more than one token (the first step after a prefill) is cut in
//   bulk by a radix select; with the caller's lengths and budgets the cut is
//   spread over the unit's importance blocks (keys, and a key histogram for
//   the unit) and finished by three more launches (k_bulk_mark: the bin of
//   the threshold, the slots below it and the bin's keys; k_bulk_select: the
//   threshold and the lists of rows to move; k_bulk_moves: the moves).
//   Output blocks combine the tiles' partials.

#include <hip/hip_ext.h>

#include <type_traits>

#include "hikv_block.h"
#include "hikv_dev.h"
#include "hikv_launch.h"

namespace hikv {


// ---------------------------------------------------------------------------
// K1: split-K attention tiles.
// ---------------------------------------------------------------------------
template <int EL, int D, int G>
__global__ __launch_bounds__(kThreads) void k_attend(StepArgs a) {
  using LY = ALay<EL, D, G>;
  constexpr int CH = LY::CH, LPR = LY::LPR, TPW = LY::TPW, UR = LY::UR, TS = LY::TS, NSUB = LY::NSUB,
                TC = LY::TC, NI = LY::NI, SUBB = LY::SUBB;
  constexpr int RB = LY::RB;
  constexpr int QB = G * D * EL;  // the group's queries, bytes
  static_assert(QB <= 4 * 1024, "one q DMA instruction per wave");
  // LDS: NSUB sub-chunks, each K then V; the group's queries.
  __shared__ __attribute__((aligned(16))) char smem[NSUB * 2 * SUBB];
  __shared__ __attribute__((aligned(16))) char qs[QB];
  __shared__ __attribute__((aligned(16))) float lgs[TC * G];  // the chunk's logits
  __shared__ float sm_ml[4][G][2];
  __shared__ __attribute__((aligned(16))) PendLds pd;
  float(*sm_acc)[G][D] = reinterpret_cast<float(*)[G][D]>(smem);  // reused after the chunks
  static_assert(4 * G * D * 4 <= NSUB * 2 * SUBB, "merge scratch must fit in the stage");
  static_assert(NSUB == 3, "the vmcnt chain below is written for three sub-chunks");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int U = a.n_units;
  // The host plan's words are loaded before its presence is known (the kernel
  // arguments are always readable); the device plan's path uses them too, after
  // its own loads, so that the compiler issues them ahead of the branch.
  const int hp_bend = a.hp.base[lane + 1], hp_len = a.hp.L[lane];
  kernarg_warm(0);  // (after the plan's vector loads are issued)
  Plan pl;
  if (a.hp.n) {
    pl = host_plan(a, blockIdx.x, hp_bend, hp_len);
  } else {
    pl = wave_plan(a, blockIdx.x, (int)gridDim.x - U, blockIdx.x == 0 && wave == 0);
    asm volatile("" ::"v"(hp_bend), "v"(hp_len));
  }

  if (!pl.valid) {
    if (a.bulk_split) bulk_hist_clear(a);  // (on every way out: the grid covers it)
    if (blockIdx.x == 0 && !a.hp.n) error_sweep<G, D>(a);
    return;
  }

  const int u = pl.u, b = u / a.Hkv, j = u - b * a.Hkv;
  const int Lold = pl.L - 1, t0 = pl.t0, t1 = pl.t1;
  const int tile = blockIdx.x;
  const int r = lane / LPR, c = lane - r * LPR;
  const char *kc = static_cast<const char *>(a.k_cache) + (size_t)u * a.cap * RB;
  const char *vc = static_cast<const char *>(a.v_cache) + (size_t)u * a.cap * RB;
  const char *kn = static_cast<const char *>(a.k_new) + (size_t)u * RB;
  const char *vn = static_cast<const char *>(a.v_new) + (size_t)u * RB;
  float *lg = a.ws.logits + (size_t)u * a.cap * G;

  // The pending eviction's candidates and the group's queries go to LDS
  // ahead of the first rows, so every wait below also covers them.
  if (wave == 0) pend_fetch(a, u, pd, lane);
  int dead = -1;  // the pending eviction's slot: masked
  {
    const int off = wave * 1024 + lane * 16;
    const char *qsrc = static_cast<const char *>(a.q) + (size_t)(b * a.Hq + j * G) * D * EL;
    if (off < QB) dma16(qsrc + off, qs + wave * 1024);
  }
  const float cs = a.scale_log2, tau = 8.f / cs;
  float m[G], l[G], acc[G][CH];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < CH; ++e) acc[g][e] = 0.f;
  }
  for (int cbase = t0; cbase < t1; cbase += TC) {
    if (cbase != t0) lds_barrier();  // every wave is done with the previous chunk
#pragma unroll
    for (int sc = 0; sc < NSUB; ++sc) {
      const int c0 = cbase + sc * TS;
      stage_sub<RB, NI>(smem + sc * 2 * SUBB, smem + sc * 2 * SUBB + SUBB, kc, vc, kn, vn, c0,
                        max(0, min(TS, t1 - c0)), t0, Lold, wave, lane);
    }
    uint4 qf[G];
#pragma unroll
    for (int sc = 0; sc < NSUB; ++sc) {
      float sl[UR][G];
      const int c0 = cbase + sc * TS;
      if (sc == 0) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NI * (NSUB - 1)) : "memory");
      else if (sc == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NI * (NSUB - 2)) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      const bool first = cbase == t0 && sc == 0;
      if (first && wave == 0) pend_resolve(a, u, pd, lane, t0 == 0);
      dma_barrier();
      if (first) dead = pend_read(pd);
      if (sc == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) qf[g] = *reinterpret_cast<const uint4 *>(qs + (g * D + c * CH) * EL);
      }
      const int nrows = min(TS, t1 - c0);  // <= 0: nothing left in this chunk
      const char *kb = smem + sc * 2 * SUBB;
      const char *vb = kb + SUBB;
      static_assert(UR == 2, "two row groups per wave per sub-chunk");
      uint4 kf2[UR], vf[UR];
      {
        const int row0 = wave * (TS / 4) + r, row1 = row0 + TPW;
        lds_read_rows(kf2[0], kf2[1], vf[0], vf[1], lds_addr(kb + row0 * RB + c * 16),
                      lds_addr(kb + row1 * RB + c * 16), lds_addr(vb + row0 * RB + c * 16),
                      lds_addr(vb + row1 * RB + c * 16));
      }
#pragma unroll
      for (int i = 0; i < UR; ++i) {
        const int row = wave * (TS / 4) + i * TPW + r;
        const bool ok = row < nrows && c0 + row != dead;
        const uint4 kf = kf2[i];
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
          d = row_sum<LPR>(d);  // raw q.k; the scale enters in the exponent
          sl[i][g] = ok ? d : -INFINITY;
        }
        if (c == 0) {  // staged in LDS, written out once the chunk is done
          float *dst = lgs + (sc * TS + row) * G;
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
        // Each row keeps a reference maximum m (raw q.k) and p = 2^((s - m) c).
        // The reference moves (with a rescale of l and acc) only when the
        // row's maximum passes it by more than 8 / c, i.e. when p could
        // exceed 2^8; the branch is taken by the whole wave or not at all.
        float mx = m[g];
#pragma unroll
        for (int i = 0; i < UR; ++i) mx = fmaxf(mx, sl[i][g]);
        if (__ballot(mx > m[g] + tau) != 0ull) {
          const float corr = (mx == -INFINITY) ? 1.f : fast_exp2((m[g] - mx) * cs);
          l[g] *= corr;
#pragma unroll
          for (int e = 0; e < CH; ++e) acc[g][e] *= corr;
          m[g] = mx;
        }
        const float mc = (m[g] == -INFINITY) ? 0.f : m[g] * cs;
        float ls = l[g];
#pragma unroll
        for (int i = 0; i < UR; ++i) {
          const float p = fast_exp2(fmaf(sl[i][g], cs, -mc));
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
      }
      // Keep this sub-chunk's arithmetic ahead of the next sub-chunk's wait:
      // the empty asm statements consume the running state, and asm volatile
      // statements keep their order (otherwise the compiler defers the
      // softmax and P.V of every sub-chunk until the last one has landed).
#pragma unroll
      for (int g = 0; g < G; ++g) {
        asm volatile("" : "+v"(m[g]), "+v"(l[g]));
#pragma unroll
        for (int e = 0; e < CH; ++e) asm volatile("" : "+v"(acc[g][e]));
      }
      sched_fence();
    }
    // The chunk's logits: each wave writes the rows it computed (global
    // stores issued between the waits above would hold back the vmcnt chain).
    {
      constexpr int WR = (TS / 4) * G;  // floats per wave per sub-chunk
#pragma unroll
      for (int q0 = 0; q0 < NSUB * WR; q0 += kWave) {
        const int q = q0 + lane;
        const int sc = q / WR, w = q - sc * WR;
        const int row = wave * (TS / 4) + w / G;
        const int n = cbase + sc * TS + row;
        if (q < NSUB * WR && n < t1) store_agent_f(lg + (size_t)n * G + (w % G), lgs[(sc * TS + row) * G + (w % G)]);
      }
    }
  }
  // Tile partial.  Each token row kept its own running maximum; the rows of a
  // wave are rescaled to the wave's maximum and summed in registers, then the
  // four waves are combined through LDS.
  constexpr int S = swap_steps<LPR>(), PW = kWave >> S;  // lanes per part
  constexpr int GP = G < 4 ? 4 : G;                        // heads, padded
  constexpr int NV = G * CH;
  float mw[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) mw[g] = g < G ? m[g] : -INFINITY;
  rows_reduce<LPR, true>(mw);
  float Mw[G];  // the wave's maximum per head, in every lane
#pragma unroll
  for (int g = 0; g < G; ++g)
    Mw[g] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mw[g % (GP >> S)]),
                                                                (g / (GP >> S)) * PW));
  float vals[NV], lw[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    if (g < G) {
      const float f = fast_exp2((m[g] - ((Mw[g] == -INFINITY) ? 0.f : Mw[g])) * cs);
      lw[g] = l[g] * f;
#pragma unroll
      for (int e = 0; e < CH; ++e) vals[g * CH + e] = acc[g][e] * f;
    } else {
      lw[g] = 0.f;
    }
  }
  rows_reduce<LPR, false>(vals);
  rows_reduce<LPR, false>(lw);
  lds_barrier();  // every wave is done with the staging buffers: they become merge scratch
  {
    const int part = lane / PW, cc = lane % LPR;
    if (LPR != 8 || (lane & 8) == 0) {
#pragma unroll
      for (int i = 0; i < (NV >> S); ++i) {
        const int vi = i + part * (NV >> S);
        sm_acc[wave][vi / CH][cc * CH + vi % CH] = vals[i];
      }
      if (cc == 0) {
#pragma unroll
        for (int i = 0; i < (GP >> S); ++i) {
          const int gi = i + part * (GP >> S);
          if (gi < G) sm_ml[wave][gi][1] = lw[i];
        }
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) sm_ml[wave][g][0] = Mw[g];
    }
  }
  lds_barrier();
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int g = idx / D, d = idx - g * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_ml[w][g][0]);
    const float Ms = (M == -INFINITY) ? 0.f : M;
    float av = 0.f, lv = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float e = fast_exp2((sm_ml[w][g][0] - Ms) * cs);
      av += sm_acc[w][g][d] * e;
      lv += sm_ml[w][g][1] * e;
    }
    store_agent_f(a.ws.part_acc + ((size_t)tile * G + g) * D + d, av);
    if (d == 0) {
      store_agent_f(a.ws.part_ml + ((size_t)tile * G + g) * 2, M);
      store_agent_f(a.ws.part_ml + ((size_t)tile * G + g) * 2 + 1, lv);
    }
  }
  if (a.bulk_split) bulk_hist_clear(a);  // (on every way out: the grid covers it)
  if (blockIdx.x == 0 && !a.hp.n) error_sweep<G, D>(a);
}

template <int G, int NSUB>
__global__ __launch_bounds__(kThreads) void k_attend_mfma(StepArgs a) {
  constexpr int EL = 2, D = 128, RB = D * EL, SUBB = 8192, TS = SUBB / RB, NI = SUBB / 4096;
  constexpr int QB = G * D * EL;
  static_assert(TS == 32 && G <= 8, "two 16-token groups per sub-chunk; at most 8 heads per group");
  __shared__ __attribute__((aligned(16))) char smem[NSUB * 2 * SUBB];
  __shared__ __attribute__((aligned(16))) char qs[QB];
  __shared__ __attribute__((aligned(16))) float lgs[2 * 16 * G];  // logits of a sub-chunk, per token group
  __shared__ float sm_ml[4][G][2];
  __shared__ __attribute__((aligned(16))) PendLds pd;
  float(*sm_acc)[G][64] = reinterpret_cast<float(*)[G][64]>(smem);  // reused after the loop
  static_assert(4 * G * 64 * 4 <= NSUB * 2 * SUBB, "merge scratch must fit in the stage");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int U = a.n_units;
  // The host plan's words are loaded before its presence is known (the kernel
  // arguments are always readable); the device plan's path uses them too, after
  // its own loads, so that the compiler issues them ahead of the branch.
  const int hp_bend = a.hp.base[lane + 1], hp_len = a.hp.L[lane];
  kernarg_warm(0);  // (after the plan's vector loads are issued)
  Plan pl;
  if (a.hp.n) {
    pl = host_plan(a, blockIdx.x, hp_bend, hp_len);
  } else {
    pl = wave_plan(a, blockIdx.x, (int)gridDim.x - U, blockIdx.x == 0 && wave == 0);
    asm volatile("" ::"v"(hp_bend), "v"(hp_len));
  }
  if (!pl.valid) {
    if (a.bulk_split) bulk_hist_clear(a);  // (on every way out: the grid covers it)
    if (blockIdx.x == 0 && !a.hp.n) error_sweep<G, D>(a);
    return;
  }
  const int u = pl.u, b = u / a.Hkv, j = u - b * a.Hkv;
  const int Lold = pl.L - 1, t0 = pl.t0, t1 = pl.t1;
  const int tile = blockIdx.x;
  const char *kc = static_cast<const char *>(a.k_cache) + (size_t)u * a.cap * RB;
  const char *vc = static_cast<const char *>(a.v_cache) + (size_t)u * a.cap * RB;
  const char *kn = static_cast<const char *>(a.k_new) + (size_t)u * RB;
  const char *vn = static_cast<const char *>(a.v_new) + (size_t)u * RB;
  float *lg = a.ws.logits + (size_t)u * a.cap * G;
  // The plan's loads are all consumed by now.  A wait the compiler can see
  // (vmcnt(0) only) tells it so; otherwise it waits for them, and with them
  // for every DMA issued below, at the first reuse of their registers.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  // The pending eviction's candidates, then q, ahead of the rows.
  if (wave == 0) pend_fetch(a, u, pd, lane);
  int dead = -1;  // the pending eviction's slot: masked
  {
    const int off = wave * 1024 + lane * 16;
    const char *qsrc = static_cast<const char *>(a.q) + (size_t)(b * a.Hq + j * G) * D * EL;
    if (off < QB) dma16(qsrc + off, qs + wave * 1024);
  }

  const float cs = a.scale_log2, tau = 8.f / cs;
  const int grp = wave & 1, half = wave >> 1;  // token group, channel half of P.V
  const int hl = lane & 15, qd = lane >> 4;    // MFMA lane coordinates
  // Per-lane LDS addresses (relative to the sub-chunk's K or V buffer).
  uint32_t ad[12];
  {
    const uint32_t base = lds_addr(smem);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) ad[ks] = base + swz_off(grp * 16 + hl, 16 * ks + 4 * qd);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      ad[8 + t] = base + swz_off(grp * 16 + 4 * qd + (hl >> 2), half * 64 + 16 * t + 4 * (hl & 3));
  }
  f32x4_t O[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) O[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;  // head hl: running maximum (raw q.k) and this lane's partial sum
  bf16x4_t qb[8];
  // The tile streams through a ring of NSUB sub-chunk buffers: the first NSUB
  // are issued up front, and each buffer is refilled as soon as every wave is
  // done with it, so that loads stay in flight while earlier sub-chunks are
  // computed.  Waves 2 and 3 issue every K/V load and waves 0 and 1 every
  // logit store: loads and stores share one completion counter, so a wave
  // that waited for its loads with stores in flight would wait for the
  // stores too, and the ring would stall on every store's round trip.
  const bool loader = wave >= 2;
  const int nsc = (t1 - t0 + TS - 1) / TS;
  if (loader) {
#pragma unroll
    for (int sc = 0; sc < NSUB; ++sc) {
      if (sc < nsc) {
        const int c0 = t0 + sc * TS;
        stage_sub_by<2>(smem + sc * 2 * SUBB, smem + sc * 2 * SUBB + SUBB, kc, vc, kn, vn, c0,
                        min(TS, t1 - c0), t0, Lold, wave - 2, lane);
      }
    }
  }
  float *lgw = lgs + (wave & 1) * 16 * G;  // the wave's logit rows (token-group waves of half 0)
  const uint32_t lgw_a = lds_addr(lgw);
  for (int i = 0; i < nsc; ++i) {
    const int c0 = t0 + i * TS, bsel = i % NSUB;
    // Sub-chunk i has landed once at most the loads issued after it are
    // outstanding (loads complete in order; stores in between can only make
    // the wait longer).  Issued before this wait: the first min(nsc, NSUB),
    // and one refill per earlier iteration but the first.
    if (loader) {
      const int ahead = min(nsc, NSUB + max(0, i - 1)) - (i + 1);
      vm_wait_ahead<4 * NI, NSUB - 1>(ahead);
    } else if (i == 0) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // q and the candidates (no store issued yet)
      if (wave == 0) pend_resolve(a, u, pd, lane, t0 == 0);
    }
    dma_barrier();  // every wave's rows of sub-chunk i are in; every wave is done with i - 1
    if (i == 0) dead = pend_read(pd);
    if (loader && i >= 1 && i + NSUB - 1 < nsc) {
      const int cr = t0 + (i + NSUB - 1) * TS, br = (i - 1) % NSUB;
      stage_sub_by<2>(smem + br * 2 * SUBB, smem + br * 2 * SUBB + SUBB, kc, vc, kn, vn, cr,
                      min(TS, t1 - cr), t0, Lold, wave - 2, lane);
    }
    if (i == 0) {
      // the group's queries as the B operand (head hl in column hl); read by
      // asm so that the compiler does not wait for the ring's loads here
      uint64_t w[8];
      lds_read8_b64(w, lds_addr(qs + ((hl < G ? hl : 0) * D + 4 * qd) * EL));
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qb[ks] = __builtin_bit_cast(bf16x4_t, hl < G ? w[ks] : 0ull);
    }
    uint64_t rd[12];
    if constexpr (NSUB <= 3) {
      if (bsel == 0) mfma_operands<0, SUBB>(rd, ad);
      else if (bsel == 1) mfma_operands<2 * SUBB, 3 * SUBB>(rd, ad);
      else mfma_operands<4 * SUBB, 5 * SUBB>(rd, ad);
    } else {
      uint32_t adb[12];
      const uint32_t boff = (uint32_t)(bsel * 2 * SUBB);
#pragma unroll
      for (int k = 0; k < 12; ++k) adb[k] = ad[k] + boff;
      mfma_operands<0, SUBB>(rd, adb);
    }
    // q.k: lane (qd, hl) gets the raw scores of tokens 4 qd + i of its group for head hl.
    const f32x4_t S = qk16(rd, qb);
    const int nrows = min(TS, t1 - c0);
    float sv[4];
    if (nrows == TS && (unsigned)(dead - c0) >= (unsigned)TS) {  // every row live: nothing to mask
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) sv[r4] = S[r4];
    } else {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int row = grp * 16 + 4 * qd + r4;
        sv[r4] = (row < nrows && c0 + row != dead) ? S[r4] : -INFINITY;
      }
    }
    // The sub-chunk's logits: each half-0 wave gathers its 16 rows x G heads
    // in its own LDS rows and stores them with coalesced write-through stores
    // (little is left for the write-back at the end of the launch, which the
    // second launch waits for).
    if (half == 0) {
      if (hl < G) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) lgw[(4 * qd + r4) * G + hl] = sv[r4];
      }
      float* lgd = lg + (size_t)(c0 + grp * 16) * G;
      const int vrows = nrows - grp * 16;  // rows of this token group in the tile
#pragma unroll
      for (int q0 = 0; q0 < 16 * G; q0 += kWave) {
        const int q = q0 + lane;
        float x;
        asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                     : "=v"(x) : "v"(lgw_a + 4 * min(q, 16 * G - 1)) : "memory");
        if (q < 16 * G && q / G < vrows) store_agent_f(lgd + q, x);
      }
    }
    // Softmax of head hl: one running maximum per wave, moved (with a
    // rescale of l and of the head's output rows) only when the scores pass
    // it by more than 8 / cs.
    float mx = fmaxf(fmaxf(m, fmaxf(sv[0], sv[1])), fmaxf(sv[2], sv[3]));
    {
      float w2 = mx;
      permlane16_swap(mx, w2);
      mx = fmaxf(mx, w2);
      w2 = mx;
      permlane32_swap(mx, w2);
      mx = fmaxf(mx, w2);
    }
    if (__ballot(mx > m + tau) != 0ull) {
      const float corr = (mx == -INFINITY) ? 1.f : fast_exp2((m - mx) * cs);
      l *= corr;
      m = mx;
      // Output row r4 of this lane is head 4 qd + r4; its factor lives in lane (head).
      float fi[4];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float fa = lane_value(corr, r4 < G ? r4 : G - 1);
        if constexpr (G > 4) {
          const float fb = lane_value(corr, 4 + r4);
          fi[r4] = qd == 0 ? fa : fb;
        } else {
          fi[r4] = fa;
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) O[t][r4] *= fi[r4];
    }
    const float mc = (m == -INFINITY) ? 0.f : m * cs;
    float pv[4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      pv[r4] = fast_exp2(fmaf(sv[r4], cs, -mc));
      l += pv[r4];
    }
    bf16x4_t phi, plo;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      phi[r4] = (__bf16)pv[r4];
      plo[r4] = (__bf16)(pv[r4] - (float)phi[r4]);
    }
    // P.V for the wave's 64 channels: O[head][ch] += P[head][tok] V[tok][ch].
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16x4_t vb4 = __builtin_bit_cast(bf16x4_t, rd[8 + t]);
      O[t] = mfma32_2(phi, plo, vb4, vb4, O[t]);  // P = hi + lo, both against the same V
    }
    asm volatile("" : "+v"(m), "+v"(l));
    sched_fence();
  }
  // Tile partial: l summed over the lane rows of each head; the two token
  // groups (waves 2 h and 2 h + 1 for channel half h) combined through LDS.
  {
    float w2 = l;
    permlane16_swap(l, w2);
    l += w2;
    w2 = l;
    permlane32_swap(l, w2);
    l += w2;
  }
  lds_barrier();  // every wave is done with the staging buffers: they become merge scratch
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = 4 * qd + i;
      if (head < G) sm_acc[wave][head][16 * t + hl] = O[t][i];
    }
  if (qd == 0 && hl < G) {
    sm_ml[wave][hl][0] = m;
    sm_ml[wave][hl][1] = l;
  }
  lds_barrier();
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int h = idx / D, ch = idx - h * D, w0 = 2 * (ch >> 6), w1 = w0 + 1;
    const float m0 = sm_ml[w0][h][0], m1 = sm_ml[w1][h][0];
    const float M = fmaxf(m0, m1);
    const float Ms = (M == -INFINITY) ? 0.f : M;
    const float e0 = fast_exp2((m0 - Ms) * cs), e1 = fast_exp2((m1 - Ms) * cs);
    store_agent_f(a.ws.part_acc + ((size_t)tile * G + h) * D + ch, sm_acc[w0][h][ch & 63] * e0 + sm_acc[w1][h][ch & 63] * e1);
    if (ch == 0)
    {
      store_agent_f(a.ws.part_ml + ((size_t)tile * G + h) * 2, M);
      store_agent_f(a.ws.part_ml + ((size_t)tile * G + h) * 2 + 1, sm_ml[w0][h][1] * e0 + sm_ml[w1][h][1] * e1);
    }
  }
  if (a.bulk_split) bulk_hist_clear(a);  // (on every way out: the grid covers it)
  if (blockIdx.x == 0 && !a.hp.n) error_sweep<G, D>(a);
}

// ---------------------------------------------------------------------------
// Stage II's first launch (bf16 K, D = 128; "HiKV", Sec. III-C): per tile,
// the exact logits q.k and the reduced logits over each q-head's r channels
// of largest |q_d| (ties: lower channel) of every live token, from one matrix
// product: the B operand carries the group's queries in columns [0, G) and
// the same queries masked to their channels in columns [G, 2G).  Only K is
// read (the output is formed over the selected tokens in the second launch).
//
// The tile streams 64-token sub-chunks of K (16 KB) through a ring of NSUB
// buffers; wave w takes rows [16 w, 16 w + 16) of each.  Waves 2 and 3 issue
// the loads, waves 0 and 1 the stores (as in k_attend_mfma): every wave puts
// its scores into an LDS buffer of the sub-chunk, which waves 0 and 1 store
// one iteration later (exact logits to ws.logits2, reduced ones to
// ws.logits, token-major like Stage I's).  The softmax statistics of the
// reduced logits (running maximum and sum per column) give the tile's
// (max, sum) pair per head in ws.part_ml, the form the importance blocks of
// the second launch read.  At the first sub-chunk the waves pick the
// channels (each head's mask, one bit per channel, from a bitwise search for
// the r-th largest |q_d| with ballot counts).
// ---------------------------------------------------------------------------
template <int G, int NSUB>
__global__ __launch_bounds__(kThreads) void k_attend_s2(StepArgs a) {
  constexpr int EL = 2, D = 128, RB = D * EL, TS = 64, SUBB = TS * RB, QB = G * D * EL, NC = 2 * G;
  static_assert(NC <= 16 && NSUB <= 3, "exact and reduced columns fit one 16-column tile; ring offsets fit");
  __shared__ __attribute__((aligned(16))) char smem[NSUB * SUBB];
  __shared__ __attribute__((aligned(16))) char qs[QB];
  __shared__ __attribute__((aligned(16))) float lgs[2][TS][NC];  // a sub-chunk's scores, two buffers
  __shared__ __attribute__((aligned(16))) uint64_t s_mask[G][2];
  __shared__ float sm_ml[4][G][2];
  __shared__ __attribute__((aligned(16))) PendLds pd;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int U = a.n_units;
  const int hp_bend = a.hp.base[lane + 1], hp_len = a.hp.L[lane];
  kernarg_warm(0);  // (after the plan's vector loads are issued)
  Plan pl;
  if (a.hp.n) {
    pl = host_plan(a, blockIdx.x, hp_bend, hp_len);
  } else {
    pl = wave_plan(a, blockIdx.x, (int)gridDim.x - U, blockIdx.x == 0 && wave == 0);
    asm volatile("" ::"v"(hp_bend), "v"(hp_len));
  }
  if (!pl.valid) {
    if (a.bulk_split) bulk_hist_clear(a);  // (on every way out: the grid covers it)
    if (blockIdx.x == 0 && !a.hp.n) error_sweep<G, D>(a);
    return;
  }
  const int u = pl.u, b = u / a.Hkv, j = u - b * a.Hkv;
  const int Lold = pl.L - 1, t0 = pl.t0, t1 = pl.t1;
  const int tile = blockIdx.x;
  const char *kc = static_cast<const char *>(a.k_cache) + (size_t)u * a.cap * RB;
  const char *kn = static_cast<const char *>(a.k_new) + (size_t)u * RB;
  float *lgr = a.ws.logits + (size_t)u * a.cap * G;   // reduced
  float *lge = a.ws.logits2 + (size_t)u * a.cap * G;  // exact
  __builtin_amdgcn_s_waitcnt(0x0F70);  // (see k_attend_mfma)
  if (wave == 0) pend_fetch(a, u, pd, lane);
  int dead = -1;
  {
    const int off = wave * 1024 + lane * 16;
    const char *qsrc = static_cast<const char *>(a.q) + (size_t)(b * a.Hq + j * G) * D * EL;
    if (off < QB) dma16(qsrc + off, qs + wave * 1024);
  }
  const float cs = a.scale_log2, tau = 8.f / cs;
  const int hl = lane & 15, qd = lane >> 4;
  uint32_t ad[8];
  {
    const uint32_t base = lds_addr(smem);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) ad[ks] = base + swz_off(wave * 16 + hl, 16 * ks + 4 * qd);
  }
  const uint32_t lgs_a = lds_addr(&lgs[0][0][0]);
  float m = -INFINITY, l = 0.f;  // column hl: running maximum (raw) and this lane's partial sum
  bf16x4_t qb[8];
  const bool loader = wave >= 2;
  const int nsc = (t1 - t0 + TS - 1) / TS;
  if (loader) {
#pragma unroll
    for (int sc = 0; sc < NSUB; ++sc) {
      if (sc < nsc) {
        const int c0 = t0 + sc * TS;
        stage_k_by<2>(smem + sc * SUBB, kc, kn, c0, min(TS, t1 - c0), t0, Lold, wave - 2, lane);
      }
    }
  }
  // Waves 0 and 1: the scores of sub-chunk ip (rows [32 w, 32 w + 32)) to
  // both logit arrays, coalesced write-through stores.
  auto store_logits = [&](int ip) {
    const int c0p = t0 + ip * TS, nr = min(TS, t1 - c0p);
    const uint32_t src = lgs_a + (uint32_t)((ip & 1) * TS * NC) * 4u;
#pragma unroll
    for (int q0 = 0; q0 < 32 * G; q0 += kWave) {
      const int qq = q0 + lane, row = 32 * wave + qq / G, g = qq % G;
      const int rc = min(row, TS - 1);  // (lanes past the 32 G values read a valid row, unused)
      const float xe = lds_read_f32(src + (uint32_t)(rc * NC + g) * 4u);
      const float xr = lds_read_f32(src + (uint32_t)(rc * NC + G + g) * 4u);
      if (qq < 32 * G && row < nr) {
        store_agent_f(lge + (size_t)(c0p + row) * G + g, xe);
        store_agent_f(lgr + (size_t)(c0p + row) * G + g, xr);
      }
    }
  };
  for (int i = 0; i < nsc; ++i) {
    const int c0 = t0 + i * TS, bsel = i % NSUB;
    if (loader) {
      const int ahead = min(nsc, NSUB + max(0, i - 1)) - (i + 1);
      vm_wait_ahead<16 / 2, NSUB - 1>(ahead);
    } else if (i == 0) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // q and the candidates (no store issued yet)
      if (wave == 0) pend_resolve(a, u, pd, lane, t0 == 0);
    }
    // Every wave's rows of sub-chunk i are in, every wave is done with
    // i - 1, and the scores of i - 1 are in LDS.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (i == 0) {
      dead = pend_read(pd);
      // (q is in LDS: waves 0 and 1, which issued its loads, waited for them
      // before the barrier)
      {
        // The channels of heads g = wave, wave + 4: r largest |q_d|, ties to
        // the lower channel; lane l holds channels l and l + 64.  |q| of a
        // bf16 q has its low 16 fp32 bits zero: bits 30 .. 16 are searched.
        for (int g = wave; g < G; g += 4) {
          uint32_t x0, x1;
          lds_read_u16x2(x0, x1, lds_addr(qs + (g * D + lane) * EL), lds_addr(qs + (g * D + lane + 64) * EL));
          const uint32_t a0 = (x0 << 16) & 0x7FFFFFFFu, a1 = (x1 << 16) & 0x7FFFFFFFu;  // |q| as fp32 bits
          uint32_t thr = 0;
          for (int bit = 30; bit >= 16; --bit) {
            const uint32_t c = thr | (1u << bit);
            if (__popcll(__ballot(a0 >= c)) + __popcll(__ballot(a1 >= c)) >= a.r) thr = c;
          }
          const bool g0 = a0 > thr, g1 = a1 > thr;
          const int need = a.r - __popcll(__ballot(g0)) - __popcll(__ballot(g1));
          const uint64_t e0 = __ballot(a0 == thr), e1 = __ballot(a1 == thr);
          const uint64_t below = (1ull << lane) - 1ull;
          const bool s0 = g0 || (a0 == thr && __popcll(e0 & below) < need);
          const bool s1 = g1 || (a1 == thr && __popcll(e0) + __popcll(e1 & below) < need);
          const uint64_t m0 = __ballot(s0), m1 = __ballot(s1);
          if (lane == 0) {  // (asm: a compiler-visible LDS store would wait for the ring)
            asm volatile("ds_write_b64 %0, %1" ::"v"(lds_addr(&s_mask[g][0])), "v"(m0) : "memory");
            asm volatile("ds_write_b64 %0, %1" ::"v"(lds_addr(&s_mask[g][1])), "v"(m1) : "memory");
          }
          if (a.dbg_channels && t0 == 0) {  // the chosen channels, ascending
            int32_t *dc = a.dbg_channels + ((size_t)b * a.Hq + j * G + g) * a.r;
            if (s0) dc[__popcll(m0 & below)] = lane;
            if (s1) dc[__popcll(m0) + __popcll(m1 & below)] = lane + 64;
          }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // the masks
      // B operands: column hl < G the query of head hl; G <= hl < 2G the
      // query of head hl - G with the unchosen channels zeroed; others zero.
      const int gh = hl < G ? hl : (hl < NC ? hl - G : 0);
      uint64_t w[8];
      lds_read8_b64(w, lds_addr(qs + (gh * D + 4 * qd) * EL));
      const uint64_t mlo = lds_read_u64(lds_addr(&s_mask[gh][0])), mhi = lds_read_u64(lds_addr(&s_mask[gh][1]));
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int c = 16 * ks + 4 * qd;  // the lane's four channels c .. c + 3
        const uint32_t nib = (uint32_t)(((c < 64 ? mlo : mhi) >> (c & 63)) & 0xFull);
        uint64_t keep = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((nib >> e) & 1u) keep |= 0xFFFFull << (16 * e);
        if (hl < G) keep = ~0ull;
        else if (hl >= NC) keep = 0;
        qb[ks] = __builtin_bit_cast(bf16x4_t, w[ks] & keep);
      }
    }
    if (loader && i >= 1 && i + NSUB - 1 < nsc) {
      const int cr = t0 + (i + NSUB - 1) * TS, br = (i - 1) % NSUB;
      stage_k_by<2>(smem + br * SUBB, kc, kn, cr, min(TS, t1 - cr), t0, Lold, wave - 2, lane);
    }
    if (!loader && i >= 1) store_logits(i - 1);
    uint64_t rd[8];
    if (bsel == 0) mfma_k_operands<0>(rd, ad);
    else if (bsel == 1) mfma_k_operands<SUBB>(rd, ad);
    else mfma_k_operands<2 * SUBB>(rd, ad);
    // lane (qd, hl): column hl of tokens 4 qd + 0..3 of the wave's rows
    const f32x4_t S = qk16(rd, qb);
    const int nrows = min(TS, t1 - c0);
    float sv[4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int row = wave * 16 + 4 * qd + r4;
      sv[r4] = (row < nrows && c0 + row != dead) ? S[r4] : -INFINITY;
    }
    if (hl < NC) {
      const uint32_t dst = lgs_a + (uint32_t)(((i & 1) * TS + wave * 16 + 4 * qd) * NC + hl) * 4u;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) lds_write_b32(dst + (uint32_t)(r4 * NC) * 4u, sv[r4]);
    }
    // Softmax statistics per column (the reduced columns are kept): one
    // running maximum per wave, moved when the scores pass it by 8 / cs.
    float mx = fmaxf(fmaxf(m, fmaxf(sv[0], sv[1])), fmaxf(sv[2], sv[3]));
    {
      float w2 = mx;
      permlane16_swap(mx, w2);
      mx = fmaxf(mx, w2);
      w2 = mx;
      permlane32_swap(mx, w2);
      mx = fmaxf(mx, w2);
    }
    if (__ballot(mx > m + tau) != 0ull) {
      const float corr = (mx == -INFINITY) ? 1.f : fast_exp2((m - mx) * cs);
      l *= corr;
      m = mx;
    }
    const float mc = (m == -INFINITY) ? 0.f : m * cs;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) l += fast_exp2(fmaf(sv[r4], cs, -mc));
    asm volatile("" : "+v"(m), "+v"(l));
    sched_fence();
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (!loader && nsc > 0) store_logits(nsc - 1);
  // Tile partial of the reduced columns: l over the column's lanes, then the
  // four waves (token groups) combined.
  {
    float w2 = l;
    permlane16_swap(l, w2);
    l += w2;
    w2 = l;
    permlane32_swap(l, w2);
    l += w2;
  }
  if (qd == 0 && hl >= G && hl < NC) {
    sm_ml[wave][hl - G][0] = m;
    sm_ml[wave][hl - G][1] = l;
  }
  lds_barrier();
  if (tid < G) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_ml[w][tid][0]);
    const float Ms = (M == -INFINITY) ? 0.f : M;
    float Ls = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) Ls += sm_ml[w][tid][1] * fast_exp2((sm_ml[w][tid][0] - Ms) * cs);
    store_agent_f(a.ws.part_ml + ((size_t)tile * G + tid) * 2, M);
    store_agent_f(a.ws.part_ml + ((size_t)tile * G + tid) * 2 + 1, Ls);
  }
  if (a.bulk_split) bulk_hist_clear(a);  // (on every way out: the grid covers it)
  if (blockIdx.x == 0 && !a.hp.n) error_sweep<G, D>(a);
}

// ---------------------------------------------------------------------------
// K2: per unit, importance blocks (softmax statistics, importance, eviction,
// placement of the new token) and output blocks (one 64-output chunk each).
// ---------------------------------------------------------------------------
constexpr int kT2 = 1024;            // threads of a second-launch workgroup
constexpr int kNW2 = kT2 / kWave;    // its waves

template <int G, int NT>
struct K2Lay {
  static constexpr int CHUNK = kImpChunk;    // tokens per importance block
  static constexpr int NB = CHUNK / NT;      // tokens per thread per batch
  static_assert(NB * NT == CHUNK, "an importance block takes whole batches");
};

template <int EL, int D, int G>
__host__ __device__ constexpr int k2_noc() { return G * D / 64; }

// Softmax statistics of a unit per head from its tiles' (max, sum) pairs:
// M = max over tiles, L = sum over tiles of sum * 2^(max - M).  Pair i =
// tile * G + g; thread t of NT owns pairs t, t + NT, ... (all of head t % G); v0 is
// its first pair, already loaded.  Every wave finishes the reduction itself,
// so lane l leaves with M and L of head l % G (no broadcast barrier).  When
// sm_m is given, the maxima of head gm are also left there per tile.
template <int G, int NT = kT2>
__device__ __forceinline__ void unit_stats(const float2 *pml, int npair, float2 v0, float cs, float (*red)[G],
                                           float (*red2)[G], float &Mlane, float &Llane, float *sm_m, int gm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NV = NT / kWave * G, KV = (NV + kWave - 1) / kWave;
  float mx = tid < npair ? v0.x : -INFINITY;
  for (int i = tid + NT; i < npair; i += NT) mx = fmaxf(mx, pml[i].x);
  if (sm_m) {
    if (tid < npair && tid % G == gm) sm_m[tid / G] = v0.x;
    for (int i = tid + NT; i < npair; i += NT)
      if (i % G == gm) sm_m[i / G] = pml[i].x;
  }
  mx = lanes_max<G>(mx);
  if (lane < G) red[wave][lane] = mx;
  lds_barrier();
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < KV; ++k) {
    const int idx = lane + kWave * k;  // idx % G == lane % G
    if (idx < NV) M = fmaxf(M, red[idx / G][idx % G]);
  }
  M = lanes_max<G>(M);
  const float Ms = (M == -INFINITY) ? 0.f : M;
  float ls = tid < npair ? v0.y * fast_exp2((v0.x - Ms) * cs) : 0.f;
  for (int i = tid + NT; i < npair; i += NT) {
    const float2 v = pml[i];
    ls += v.y * fast_exp2((v.x - Ms) * cs);
  }
  ls = lanes_sum<G>(ls);
  if (lane < G) red2[wave][lane] = ls;
  lds_barrier();
  float L = 0.f;
#pragma unroll
  for (int k = 0; k < KV; ++k) {
    const int idx = lane + kWave * k;
    if (idx < NV) L += red2[idx / G][idx % G];
  }
  Mlane = M;
  Llane = lanes_sum<G>(L);
}

// ---------------------------------------------------------------------------
// Stage II's output for head g of unit u (an output block of the second
// launch, bf16 V, D = 128): of the live tokens (the dead slot of a pending
// eviction is not one), the k_T with the largest reduced logit, ties to the
// lower position (key: the logit's order bits, then the complemented
// position); then their exact softmax and P.V.  The new token (slot L - 1)
// has position new_pos[b] and its V row in v_new (the importance blocks of
// the same launch write it into the cache).
//
// Selection.  Units of up to KR * kT2 tokens (the steady state), every key
// in registers: a histogram of the keys' top 11 bits gives the bin holding
// the k_T-th largest; the bin's keys are gathered in LDS (narrowed by a
// histogram of the next 11 bits when over 128) and ranked.  Longer units, or
// a crowded sub-bin: radix passes of 8 bits from the top over the workgroup,
// the keys beyond the registers' recomputed from the logits each pass.
// KR = 2, or 4 when some unit of the step is longer than 2048 tokens (more
// registers and a larger key buffer, which cost the short units' steps
// time).
// ---------------------------------------------------------------------------
constexpr int kS2List = kS2TwoMaxTokens;  // selected tokens listed in LDS
static_assert(kS2List * 8 <= 2 * kT2 * 8, "the list fits the key buffer");

template <int G, int KR>
__device__ __forceinline__ void s2_out_block(const StepArgs &a, int u, int g, int L, int dead, int newest,
                                             bool skip) {
  constexpr int D = 128, RB = 256, NW = kNW2;
  __shared__ uint32_t h[256];
  __shared__ __attribute__((aligned(16))) float s2red[NW][D + 8];  // P.V partials; the selection's histogram before
  constexpr int kS2Kr = KR, kS2Wave = KR * kT2;  // units up to kS2Wave tokens: the histogram selection
  __shared__ __attribute__((aligned(16))) char s_buf[kS2Wave * 8];  // the keys, then the list of selected tokens
  __shared__ float s_pm[NW], s_ps[NW];
  __shared__ uint64_t s_T;
  __shared__ int s_d, s_need, s_cnt, s_fall;
  __shared__ uint64_t s_bm[kS2Kr * NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = u / a.Hkv, j = u - b * a.Hkv, hq = j * G + g;
  float *outp = a.out + ((size_t)b * a.Hq + hq) * D;
  if (skip) {  // a unit the step leaves alone
    if (tid < D) outp[tid] = 0.f;
    if (a.dbg_count && tid == 0) a.dbg_count[(size_t)b * a.Hq + hq] = 0;
    return;
  }
  const float *lgr = a.ws.logits + (size_t)u * a.cap * G + g;
  const float *lge = a.ws.logits2 + (size_t)u * a.cap * G + g;
  const int32_t *posw = a.pos + (size_t)u * a.cap;
  const int Lold = L - 1;
  // (loads from clamped addresses, then selects: a load under a condition
  // makes the compiler wait for it where the paths meet)
  auto key_of = [&](int n) -> uint64_t {
    const int nc = min(n, Lold);
    const float lv = lgr[(size_t)nc * G];
    const int pv = posw[nc];
    const int p = n == Lold ? newest : pv;
    const bool live_n = n < L && n != dead;
    return live_n ? (((uint64_t)ord_f32(lv) << 32) | (uint64_t)(~(uint32_t)p)) : 0ull;
  };
  uint64_t kr[kS2Kr];
  float er[kS2Kr];
#pragma unroll
  for (int i = 0; i < kS2Kr; ++i) {
    const int n = tid + i * kT2;
    kr[i] = key_of(n);
    er[i] = lge[(size_t)min(n, Lold) * G];
  }
  const int live = L - (dead >= 0 && dead < L ? 1 : 0);
  const int kT = min(a.kT, live);
  const bool all = kT >= live;  // every live token
  uint64_t T = 1ull;            // selected: key >= T (keys are distinct)
  bool radix = !all && L > kS2Wave;
  if (!all && L <= kS2Wave) {
    // Keys in registers cover the unit (L <= kS2Kr * kT2).  A histogram of
    // their top 11 bits (padded: bin b at word b + b / 32, so that a lane's
    // 32 consecutive bins sit in distinct banks), the bin holding the kT-th
    // largest (wave 0), that bin's keys gathered -- narrowed by a second
    // histogram of the next 11 bits when over 128 -- and ranked (each counts
    // the larger ones).
    static_assert(kS2Wave <= kS2Kr * kT2, "the keys of a unit fit the registers");
    static_assert(kS2Wave * 8 <= (int)sizeof(s_buf), "a bin's keys fit the gather buffer");
    uint32_t *h2 = reinterpret_cast<uint32_t *>(&s2red[0][0]);          // 2112 words
    uint64_t *cand = reinterpret_cast<uint64_t *>(s_buf);                 // a bin's keys
    auto pidx = [](int bin) { return bin + (bin >> 5); };
    // The bin of the 2048-bin histogram in h2 holding the need-th largest
    // counted key (wave 0; lane l takes bins 2047 - 32 l down to 2016 - 32 l,
    // then the lane whose range holds it takes that range one bin per lane):
    // s_d (-1: none), the need within it, its count.
    auto pick = [&](int need) {
      if (wave == 0) {
        uint32_t c = 0;
#pragma unroll 8
        for (int q = 0; q < 32; ++q) c += h2[pidx(2047 - 32 * lane - q)];
        const uint32_t incl = wave_incl_scan_dpp(c), excl = incl - c;
        const uint64_t lm = __ballot(excl < (uint32_t)need && incl >= (uint32_t)need);
        const int lt = lm ? __builtin_ctzll(lm) : 0;
        const uint32_t ex_t = __shfl(excl, lt);
        const uint32_t hb = lane < 32 ? h2[pidx(2047 - 32 * lt - lane)] : 0u;
        const uint32_t in2 = wave_incl_scan_dpp(hb) + ex_t, ex2 = in2 - hb;
        const uint64_t qm = __ballot(lane < 32 && ex2 < (uint32_t)need && in2 >= (uint32_t)need);
        const int qq = qm ? __builtin_ctzll(qm) : 0;
        const int cntb = (int)__shfl(hb, qq), exq = (int)__shfl(ex2, qq);  // (every lane of the wave)
        if (lane == 0) {
          const bool ok = lm && qm;
          s_d = ok ? 2047 - 32 * lt - qq : -1;
          s_need = need - exq;
          s_fall = cntb;
        }
      }
      __syncthreads();
    };
    // Wave-aggregated count of digit d (2048: none) into h2.
    auto count_digit = [&](int d) {
      const int d0 = __builtin_amdgcn_readfirstlane(d);
      const uint64_t same = __ballot(d == d0);
      if (d == d0) {
        if (d0 < 2048 && lane == __builtin_ctzll(same)) atomicAdd(&h2[pidx(d0)], (uint32_t)__popcll(same));
      } else if (d < 2048) {
        atomicAdd(&h2[pidx(d)], 1u);
      }
    };
    for (int i = tid; i < 2112; i += kT2) h2[i] = 0u;
    if (tid == 0) s_cnt = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kS2Kr; ++i) count_digit(kr[i] ? (int)(kr[i] >> 53) : 2048);
    __syncthreads();
    pick(kT);
    const int bin = s_d;
    int needb = s_need;
    radix = bin < 0;
    if (!radix) {
      // The bin's keys, gathered (one atomic per wave; at most kS2Wave).
#pragma unroll
      for (int i = 0; i < kS2Kr; ++i) {
        const uint64_t key = kr[i];
        const bool in = key && (int)(key >> 53) == bin;
        const uint64_t mk = __ballot(in);
        int base = 0;
        if (lane == 0 && mk) base = atomicAdd(&s_cnt, __popcll(mk));
        base = __builtin_amdgcn_readfirstlane(base);
        if (in) cand[base + __popcll(mk & ((1ull << lane) - 1ull))] = key;
      }
      __syncthreads();
      int nc = s_cnt;
      uint64_t floor_key = (uint64_t)bin << 53;  // the lowest key of the bin
      const uint64_t *kc = cand;
      uint64_t *cand2 = reinterpret_cast<uint64_t *>(&s2red[0][0]) + 512;  // past the rank counts
      if (needb < nc && nc > 128) {
        // More than 128: the next 11 bits (52 .. 42) of the bin's keys,
        // histogrammed, narrow it to a sub-bin, whose keys are gathered.
        for (int i = tid; i < 2112; i += kT2) h2[i] = 0u;
        __syncthreads();
        for (int i0 = 0; i0 < nc; i0 += kT2) {
          const int i = i0 + tid;
          count_digit(i < nc ? (int)((cand[i] >> 42) & 2047ull) : 2048);
        }
        __syncthreads();
        pick(needb);
        const int sub = s_d;
        if (sub < 0 || s_fall > 128) {
          radix = true;  // a sub-bin still over 128 keys: radix passes over the unit
        } else {
          needb = s_need;
          floor_key |= (uint64_t)sub << 42;
          if (tid == 0) s_cnt = 0;
          __syncthreads();  // (h2 is done with: cand2 and the rank counts reuse s2red)
          for (int i0 = 0; i0 < nc; i0 += kT2) {
            const int i = i0 + tid;
            const uint64_t key = i < nc ? cand[i] : 0ull;
            const bool in = i < nc && (int)((key >> 42) & 2047ull) == sub;
            const uint64_t mk = __ballot(in);
            int base = 0;
            if (lane == 0 && mk) base = atomicAdd(&s_cnt, __popcll(mk));
            base = __builtin_amdgcn_readfirstlane(base);
            if (in) cand2[base + __popcll(mk & ((1ull << lane) - 1ull))] = key;
          }
          __syncthreads();
          nc = s_cnt;
          kc = cand2;
        }
      }
      if (!radix) {
        // the needb-th largest of the gathered keys: the one with needb - 1
        // larger (keys are distinct).  Thread t counts, for key t % 128, the
        // larger ones among keys 16 (t / 128) .. 16 (t / 128) + 15; the eight
        // counts of each key are then summed.  needb = nc: the whole (sub)bin.
        static_assert(kT2 == 8 * 128, "eight slices of at most 128 gathered keys");
        if (tid == 0) s_T = floor_key;
        if (needb < nc) {
          int *pr = reinterpret_cast<int *>(&s2red[0][0]);  // [8][128] (the histogram is done with)
          const int c = tid & 127, sl = tid >> 7;
          // (the slice's sixteen keys read together: a loop of dependent LDS
          // reads took most of a microsecond; reads past nc stay inside the
          // gather buffer and are not counted)
          const uint64_t key = kc[c];
          uint64_t kv[16];
#pragma unroll
          for (int q = 0; q < 16; ++q) kv[q] = kc[16 * sl + q];
          int part = 0;
#pragma unroll
          for (int q = 0; q < 16; ++q) part += (16 * sl + q < nc && kv[q] > key) ? 1 : 0;
          if (c >= nc) part = 0;
          pr[128 * sl + c] = part;
          __syncthreads();
          if (tid < nc) {
            int rank = 0;
#pragma unroll
            for (int q = 0; q < 8; ++q) rank += pr[128 * q + tid];
            if (rank == needb - 1) s_T = kc[tid];
          }
        }
        __syncthreads();
        T = s_T;
      }
    }
  }
  if (radix) {
    // The kT-th largest key by 8-bit radix passes from the top over the
    // whole workgroup; need = how many of the keys under the current prefix
    // are still to take.
    uint64_t prefix = 0;
    int rem = 64, need = kT;
    while (rem > 0) {
      const int sh = rem - 8;
      if (tid < 256) h[tid] = 0u;
      __syncthreads();
      auto count = [&](uint64_t key) {
        const bool in = key != 0ull && (rem == 64 || (key >> rem) == (prefix >> rem));
        const int d = in ? (int)((key >> sh) & 255ull) : 256;
        const int d0 = __builtin_amdgcn_readfirstlane(d);
        const uint64_t same = __ballot(d == d0);
        if (d == d0) {
          if (d0 < 256 && lane == __builtin_ctzll(same)) atomicAdd(&h[d0], (uint32_t)__popcll(same));
        } else if (d < 256) {
          atomicAdd(&h[d], 1u);
        }
      };
#pragma unroll
      for (int i = 0; i < kS2Kr; ++i) count(kr[i]);
      for (int n = tid + kS2Kr * kT2; n < L; n += kT2) count(key_of(n));
      __syncthreads();
      if (wave == 0) {
        // lane l: digits 255 - 4 l ... 252 - 4 l (descending); the digit at
        // which the count from the top reaches need
        const uint32_t c0 = h[255 - 4 * lane], c1 = h[254 - 4 * lane], c2 = h[253 - 4 * lane],
                       c3 = h[252 - 4 * lane];
        const uint32_t s4 = c0 + c1 + c2 + c3;
        const uint32_t incl = wave_incl_scan_u32(s4), excl = incl - s4, want = (uint32_t)need;
        if (excl < want && incl >= want) {
          const uint32_t a1 = excl + c0, a2 = a1 + c1, a3 = a2 + c2;
          const int q = a1 >= want ? 0 : (a2 >= want ? 1 : (a3 >= want ? 2 : 3));
          const uint32_t above = q == 0 ? excl : (q == 1 ? a1 : (q == 2 ? a2 : a3));
          s_d = 255 - 4 * lane - q;
          s_need = need - (int)above;
          s_cnt = (int)(q == 0 ? c0 : (q == 1 ? c1 : (q == 2 ? c2 : c3)));
        }
      }
      __syncthreads();
      prefix |= (uint64_t)s_d << sh;
      rem = sh;
      need = s_need;
      if (need == s_cnt) break;  // the whole digit is taken: prefix, lower bits 0, is the threshold
      __syncthreads();
    }
    T = prefix;
  }
  auto sel = [&](uint64_t key) { return key != 0ull && key >= T; };

  // Exact softmax over the selected tokens: the maximum over the wave, each
  // thread's sum relative to it and the wave's, then the waves' pairs merged.
  const float cs = a.scale_log2;
  float tm = -INFINITY;
#pragma unroll
  for (int i = 0; i < kS2Kr; ++i)
    if (sel(kr[i])) tm = fmaxf(tm, er[i]);
  for (int n = tid + kS2Kr * kT2; n < L; n += kT2)
    if (sel(key_of(n))) tm = fmaxf(tm, lge[(size_t)n * G]);
  const float wm = wave_max_dpp(tm);
  const float wms = (wm == -INFINITY) ? 0.f : wm * cs;
  float ts_ = 0.f;
#pragma unroll
  for (int i = 0; i < kS2Kr; ++i)
    if (sel(kr[i])) ts_ += fast_exp2(fmaf(er[i], cs, -wms));
  for (int n = tid + kS2Kr * kT2; n < L; n += kT2)
    if (sel(key_of(n))) ts_ += fast_exp2(fmaf(lge[(size_t)n * G], cs, -wms));
  const float wsum = wave_sum_dpp(ts_);
  if (lane == 0) s_pm[wave] = wm, s_ps[wave] = wsum;  // (published by the list's barriers)

  // The selected tokens and their exact logits into an LDS list, in token
  // order (the P.V sums then repeat bit for bit): per chunk of kS2Kr * kT2
  // tokens, a bitmap of the selected ones (one ballot per 64 tokens), then
  // each token's place from the bits before it.  The two-launch path is
  // taken for k_T <= kS2List only.
  int *s_list = reinterpret_cast<int *>(s_buf);
  float *s_e = reinterpret_cast<float *>(s_buf + kS2List * 4);
  constexpr int CW = kS2Kr * NW;  // bitmap words per chunk
  int done = 0;
  for (int c0 = 0; c0 < L; c0 += kS2Kr * kT2) {
    bool tk[kS2Kr];
    float ek[kS2Kr];
#pragma unroll
    for (int i = 0; i < kS2Kr; ++i) {
      const int n = c0 + tid + i * kT2;
      const uint64_t key = c0 == 0 ? kr[i] : key_of(n);
      tk[i] = n < L && sel(key);
      ek[i] = c0 == 0 ? er[i] : lge[(size_t)min(n, Lold) * G];
      const uint64_t m = __ballot(tk[i]);
      if (lane == 0) s_bm[i * NW + wave] = m;
    }
    __syncthreads();
    // exclusive prefix of the words' counts: lane l < CW holds word l
    const uint32_t wc = lane < CW ? (uint32_t)__popcll(s_bm[lane]) : 0u;
    const uint32_t wi = wave_incl_scan_dpp(wc), we = wi - wc;
#pragma unroll
    for (int i = 0; i < kS2Kr; ++i) {
      const int w = i * NW + wave;
      const uint64_t m = s_bm[w];
      const int pos = done + (int)__builtin_amdgcn_readlane(we, w) + __popcll(m & ((1ull << lane) - 1ull));
      if (tk[i] && pos < kS2List) {
        s_list[pos] = c0 + tid + i * kT2;
        s_e[pos] = ek[i];
      }
    }
    done += (int)__builtin_amdgcn_readlane(wi, CW - 1);
    __syncthreads();  // the list so far (and s_bm is free again)
  }
  float pm = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) pm = fmaxf(pm, s_pm[w]);
  const float Ms = (pm == -INFINITY) ? 0.f : pm * cs;
  float ps = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) ps += s_ps[w] * fast_exp2(fmaf(s_pm[w], cs, -Ms));
  const float inv = 1.f / ps;
  const int nsel = min(done, kS2List);

  // P.V: 16 lanes per V row (8 channels each), 64 rows at a time; group q
  // takes list entries q, q + 64, ... (four rows in flight).
  const int grp = tid >> 4, cl = tid & 15;
  const char *vc = static_cast<const char *>(a.v_cache) + (size_t)u * a.cap * RB + cl * 16;
  const char *vn = static_cast<const char *>(a.v_new) + (size_t)u * RB + cl * 16;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add_row = [&](const uint4 &v4, float p) {
    const uint32_t w4[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = fmaf(p, __uint_as_float(w4[e] << 16), acc[2 * e]);
      acc[2 * e + 1] = fmaf(p, __uint_as_float(w4[e] & 0xFFFF0000u), acc[2 * e + 1]);
    }
  };
  constexpr int GS = kT2 / 16;  // row groups
  for (int i0 = grp; i0 < nsel; i0 += 4 * GS) {
    int nn[4];
    float pp[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + r * GS;
      nn[r] = i < nsel ? s_list[i] : -1;
      pp[r] = i < nsel ? fast_exp2(fmaf(s_e[i], cs, -Ms)) * inv : 0.f;
    }
    const uint4 v0 = *reinterpret_cast<const uint4 *>(nn[0] == Lold ? vn : vc + (size_t)max(nn[0], 0) * RB);
    const uint4 v1 = *reinterpret_cast<const uint4 *>(nn[1] == Lold ? vn : vc + (size_t)max(nn[1], 0) * RB);
    const uint4 v2 = *reinterpret_cast<const uint4 *>(nn[2] == Lold ? vn : vc + (size_t)max(nn[2], 0) * RB);
    const uint4 v3 = *reinterpret_cast<const uint4 *>(nn[3] == Lold ? vn : vc + (size_t)max(nn[3], 0) * RB);
    add_row(v0, pp[0]);
    add_row(v1, pp[1]);
    add_row(v2, pp[2]);
    add_row(v3, pp[3]);
  }
  // the four groups of a wave (lanes 16 apart: permlane swaps), then the waves
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float w2 = acc[e];
    permlane16_swap(acc[e], w2);
    acc[e] += w2;
    w2 = acc[e];
    permlane32_swap(acc[e], w2);
    acc[e] += w2;
  }
  if (lane < 16) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s2red[wave][cl * 8 + e] = acc[e];
  }
  __syncthreads();
  if (tid < D) {
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) o += s2red[w][tid];
    outp[tid] = o;
  }
  if (a.dbg_count && tid == 0) a.dbg_count[(size_t)b * a.Hq + hq] = kT;
  if (a.dbg_tokens) {
    // the selected positions, ascending, -1 padded (debug only: each
    // selected token is ranked by counting)
    int32_t *dt = a.dbg_tokens + ((size_t)b * a.Hq + hq) * a.kT;
    for (int i = tid; i < a.kT; i += kT2) dt[i] = -1;
    __syncthreads();
    for (int n = tid; n < L; n += kT2) {
      const uint64_t kn_ = key_of(n);
      if (!sel(kn_)) continue;
      const uint32_t pn = ~(uint32_t)kn_;
      int rank = 0;
      for (int m2 = 0; m2 < L; ++m2) {
        const uint64_t km = key_of(m2);
        rank += sel(km) && (~(uint32_t)km) < pn;
      }
      if (rank < a.kT) dt[rank] = (int32_t)pn;
    }
  }
}

// A bulk cut of a whole unit in one importance block, out of line.  With the
// caller's lengths and budgets the host splits every bulk cut it can foresee
// over launches of their own; the one it cannot (a unit one token over budget
// that holds no pending eviction) takes this call.  Inlined, its registers would push the
// steady path's values into scratch, and reloading them waits for every store
// the block has issued.  The LDS buffers keep their address space across the
// call.
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) int lds_int;
typedef __attribute__((address_space(3))) RadixState lds_radix;
template <int NT, int RB>
__device__ __attribute__((noinline)) void bulk_cut_unit(const uint64_t *keys, int L, int beta, char *kw, char *vw,
                                                        int32_t *posw, float *impw, int32_t *holes, int32_t *movers,
                                                        int32_t *len_u, int32_t *status, lds_u32 *hist,
                                                        lds_u32 *whist, lds_int *sc, lds_radix *rs) {
  bulk_compact<NT, RB>(keys, L, beta, L - beta, kw, vw, posw, impw, holes, movers, len_u, status,
                       (uint32_t *)hist, (uint32_t *)whist, (int *)sc, (RadixState *)rs, nullptr);
}

// IB: the in-block bulk cut inlined (when the host cannot foresee bulk cuts,
// any unit may be cut in bulk in this block), or called out of line.
template <int EL, int D, int G, bool S2 = false, bool IB = false, int KR = 2>
__global__ __launch_bounds__(S2 ? kT2 : kT2 / 2) __attribute__((amdgpu_waves_per_eu(S2 ? 8 : 6))) void k_finalize(StepArgs a) {
  // Workgroup size: Stage II's output blocks select among up to 2 kT2 keys
  // held two per thread; Stage I's blocks take half as many threads (two
  // workgroups' waves per launch round fit where one did).
  constexpr int NTF = S2 ? kT2 : kT2 / 2, NWF = NTF / kWave;
  constexpr int RB = D * EL, NR = RB / 16, GD = G * D;
  constexpr int NB = K2Lay<G, NTF>::NB, CHUNK = K2Lay<G, NTF>::CHUNK;
  // output blocks per unit: Stage I one per 64 outputs, Stage II one per head
  constexpr int NOC = S2 ? G : k2_noc<EL, D, G>();
  constexpr int NTW = 8 * kNW2 / NWF;  // tiles per wave loaded in one batch by an output block
  __shared__ float red[NWF][G], red2[NWF][G];
  __shared__ float sm_m[kMaxGrid];           // output blocks: tile maxima of their head
  __shared__ float red_o[NWF][kWave];       // output blocks: per-wave partial sums
  __shared__ uint64_t sk[NWF];
  __shared__ int ss[NWF];
  __shared__ float s_newimp;
  __shared__ int s_last;
  __shared__ __attribute__((aligned(16))) uint4 s_nrow[kWave];  // the new token's K and V rows
  // bulk cut: radix-select scratch (one block per unit), or the block's key
  // histogram (kBulkBins words of whist) when the cut is spread over blocks
  __shared__ uint32_t hist[256];
  __shared__ __attribute__((aligned(16))) uint32_t whist[NWF * 256];
  __shared__ int sc[NTF];
  __shared__ RadixState rs;
  static_assert(kBulkBins <= NWF * 256, "the key histogram fits the radix scratch");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int vz = vzero();
  // Grid: x = the unit, y = the unit's workgroup, so that the unit is known
  // without a load.  r: nib importance blocks, then NOC output blocks.  The
  // blocks that end the step are dispatched first: every unit's importance
  // blocks in Stage I, its output blocks (the selection, the exact softmax and
  // the gathered V rows) in Stage II.
  const int nib = (int)gridDim.y - NOC;  // importance blocks per unit
  const int u = blockIdx.x,
            r = S2 ? ((int)blockIdx.y < NOC ? (int)blockIdx.y + nib : (int)blockIdx.y - NOC) : (int)blockIdx.y;
  // The host plan's words (kernel arguments, clamped to its table) are loaded
  // with the flag that says whether there is one, so that the host plan costs
  // one round trip; the device plan's path uses them too, after its own load,
  // so that the compiler issues them ahead of the branch.
  const int uh = min(u, kHostPlanUnits - 1);
  kernarg_warm(uh);
  const int hb0 = a.hp.base[uh], hb1 = a.hp.base[uh + 1], hlen = a.hp.L[uh];
  const int bsplit = a.bulk_split;
  asm volatile("" ::"s"(hb0), "s"(hb1), "s"(hlen), "s"(bsplit));  // one wait for all four
  int tb, nt, L;
  if (a.hp.n) {
    tb = hb0, nt = hb1 - hb0, L = hlen;
  } else {
    const int4 rec = reinterpret_cast<const int4 *>(a.ws.urec)[u];
    tb = rec.x, nt = rec.y, L = rec.z;
  }
  // The move launch that may follow reads every unit's count: none unless a
  // bulk cut below says otherwise (the same thread writes both).  (After the
  // plan's loads, so that its flag is loaded with them.)
  if (bsplit && r == 0 && tid == 0) {
    a.ws.nmoves[u] = 0;
    a.ws.bsel[4 * u + 3] = 0;
  }
  if (nt <= 0) return;  // a unit the first launch excluded
  const bool imp_blk = r < nib;
  const int nb0 = imp_blk ? r * CHUNK : 0;
  if (imp_blk && nb0 >= L && r > 0) return;  // no tokens here (nor the whole unit's eviction)
  const int b = u / a.Hkv, j = u - b * a.Hkv;
  const int Lold = L - 1;
  const int npair = nt * G;
  const float2 *pml = reinterpret_cast<const float2 *>(a.ws.part_ml) + (size_t)tb * G;
  float *impw = a.imp + (size_t)u * a.cap;
  int32_t *posw = a.pos + (size_t)u * a.cap;
  const int S = a.n_sink;

  // ---- One batch of independent loads: unconditional, from clamped (valid)
  // addresses, validity applied where a value is used.  A load under a
  // condition makes the compiler wait for it on the spot to merge it with a
  // default value.
  // (Issued inside each path: loads in flight where the two paths part would
  // be waited for at the start of the second path.)

  // The importance path comes first in the code so that its loads are not
  // held back by waits the compiler places where the two paths meet.
  if (imp_blk) {
    [&]() __attribute__((always_inline)) {
      // ---------------- importance block ----------------
      const int newest = ld_vec(a.new_pos + b, vz);
      // (the Stage II instance loads it plainly: there the pointer is not kept
      // in scalar registers, which the opaque load's constraint requires)
      const int *bp = a.budget ? a.budget + u : a.new_pos + b;
      const int beta_ld = S2 ? ld_vec(bp, vz) : ld_opaque(bp, vz);
      const float2 v0 = pml[min(tid, npair - 1)];
      const char *kn = static_cast<const char *>(a.k_new) + (size_t)u * RB;
      const char *vn = static_cast<const char *>(a.v_new) + (size_t)u * RB;
      char *kw = static_cast<char *>(a.k_w) + (size_t)u * a.cap * RB;
      char *vw = static_cast<char *>(a.v_w) + (size_t)u * a.cap * RB;
      const float *lg = a.ws.logits + (size_t)u * a.cap * G;
      const int len_dev = ld_vec(a.len + u, vz);
      const int dead_ld = ld_vec(unit_state(a, u) + 1, vz);
      // The new token's K and V rows (2 NR pieces of 16 bytes) go to LDS by
      // DMA from wave 0, ahead of the batch, to be written out at the end:
      // held in registers they would take VGPRs the batch needs.
      if (wave == 0) {
        const int rt = min(lane, 2 * NR - 1);
        dma16(rt < NR ? kn + rt * 16 : vn + (rt - NR) * 16, s_nrow);
      }
      float tl[NB][G], ti[NB];
      int tp[NB];
      auto load_batch = [&](int base) {
    #pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int n = min(base + tid + i * NTF, Lold);
          if constexpr (G % 4 == 0) {
    #pragma unroll
            for (int g = 0; g < G; g += 4) {
              const float4 v4 = *reinterpret_cast<const float4 *>(lg + (size_t)n * G + g);
              tl[i][g] = v4.x, tl[i][g + 1] = v4.y, tl[i][g + 2] = v4.z, tl[i][g + 3] = v4.w;
            }
          } else if constexpr (G == 2) {
            const float2 v2 = *reinterpret_cast<const float2 *>(lg + (size_t)n * 2);
            tl[i][0] = v2.x, tl[i][1] = v2.y;
          } else {
            tl[i][0] = lg[n];
          }
          ti[i] = impw[n];  // slot Lold holds no token yet: replaced below
          tp[i] = posw[n];
        }
      };
      load_batch(nb0);
      const int beta = a.budget ? beta_ld : a.budget_all;
      float Mlane, Llane;
      unit_stats<G, NTF>(pml, npair, v0, a.scale_log2, red, red2, Mlane, Llane, nullptr, 0);
      if (a.hp.n) {  // a host plan covers every unit: check it against the device
        const int err = (L > a.cap) ? HIKV_ECAPACITY : ((beta < S || beta > a.cap) ? HIKV_EBUDGET : 0);
        if (r == 0 && tid == 0) {
          if (err) set_status(a.ws.status, err);
          else if (len_dev != Lold) set_status(a.ws.status, HIKV_EINVAL);
        }
        if (err) return;
      }
      // The pending eviction of the previous step (found by the attention
      // launch): a dead slot, not live and not attended, that the new token
      // takes over unless the unit is cut in bulk.
      const int dead = dead_ld;
      const int live = L - (dead >= 0 ? 1 : 0);
      const bool over = live > beta;
      const int n_evict = over ? live - beta : 0;
      // One eviction (the steady state) is spread over the unit's blocks like
      // the importance, and its victim is left pending for the next call;
      // more than one (a bulk cut) needs every token in one block.  Evicting
      // whole blocks of positions is always a bulk cut.
      const bool bulk = a.block ? n_evict > 0 : n_evict > 1;
      // With the caller's lengths a bulk cut is spread over the unit's blocks
      // (each leaves its keys and a histogram of them; k_bulk_select finishes
      // the cut); without them one block takes every token.  Stage II always
      // spreads it: its output blocks read V rows, which must not move during
      // this launch.  So does block-granular eviction, whose keys are made by
      // a launch of their own (k_block_keys).
      const bool split = bulk && (a.bulk_split || S2 || a.block);
      if (bulk && !split && r > 0) return;
      const int nb1 = (bulk && !split) ? L : min(L, nb0 + CHUNK);
      const int nact = (L + CHUNK - 1) / CHUNK;  // blocks holding tokens of the unit
      const int Wp = min(a.n_recent, beta - S);
      // The new token's slot: the dead slot of a pending eviction, except in
      // a bulk cut of single tokens (which keys the dead slot to go first).
      const int fs = (dead >= 0 && (!bulk || a.block)) ? dead : Lold;
      const bool tkeys = bulk && !a.block;  // this launch keys the tokens
      const bool thist = split && !a.block;  // ... and histograms the keys
      // Kelle's pre-softmax score: the logit scale * q.k (raw q.k times scale)
      const float scale_nat = a.scale_log2 * 0.69314718055994531f;
      float Mg[G], ILg[G];
    #pragma unroll
      for (int g = 0; g < G; ++g) {
        const float Mr = lane_value(Mlane, g);  // raw q.k units
        Mg[g] = (Mr == -INFINITY) ? 0.f : Mr * a.scale_log2;
        ILg[g] = 1.f / lane_value(Llane, g);
      }
      uint64_t *bkeys = a.ws.bkeys + (size_t)u * a.cap;  // bulk: every slot's key
      uint64_t best = ~0ull;
      int best_slot = -1;
      if (thist) {
        for (int i = tid; i < kBulkBins; i += NTF) whist[i] = 0u;
        __syncthreads();
      }
      // One batch of the block's tokens: probabilities, importance, the
      // block's lowest eviction key and, in a bulk cut, every key.
      auto batch = [&](int base) __attribute__((always_inline)) {
        // Every loaded value is used before the first store: a load still
        // outstanding on some path would make the compiler wait for the
        // stores issued after it as well.
        float ivs[NB];
        int pns[NB];
    #pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int n = base + tid + i * NTF;
          float p = 0.f;
    #pragma unroll
          for (int g = 0; g < G; ++g)
            p += a.acc_logit ? tl[i][g] * scale_nat : fast_exp2(fmaf(tl[i][g], a.scale_log2, -Mg[g])) * ILg[g];
          const bool is_new = n == Lold;
          const int pn = is_new ? newest : tp[i];
          // HiKV's dual bank: only the recent window accumulates; the scores
          // of older tokens are frozen (and not rewritten).
          const bool acc = !a.acc_recent || pn > newest - Wp;
          ivs[i] = (is_new ? 0.f : ti[i]) + (acc ? p : 0.f);
          pns[i] = pn;
          asm volatile("" : "+v"(ivs[i]), "+v"(pns[i]));
        }
        // (and the new rows' DMA, issued before the batch, has landed)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    #pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int n = base + tid + i * NTF;
          int hbin = kBulkBins;  // the key's histogram bin (a spread bulk cut), or none
          if (n < nb1 && n != dead) {
            const bool is_new = n == Lold;
            const int pn = pns[i];
            const bool recent = pn > newest - Wp;
            const bool acc = !a.acc_recent || recent;
            const float iv = ivs[i];
            if (is_new) s_newimp = iv;
            else if (acc) impw[n] = iv;
            const bool cand = !((pn < S) || recent);
            if (over && cand) {
              const uint64_t k = evict_key(iv, pn);
              if (k < best) {
                best = k;
                best_slot = is_new ? fs : n;
              }
            }
            if (tkeys) {
              const uint64_t kk = cand ? evict_key(iv, pn) : ~0ull;
              bkeys[n] = kk;
              if (cand) hbin = (int)(kk >> kBulkShift);
            }
          } else if (tkeys && n < nb1) {
            bkeys[n] = 0;  // the dead slot: the first to go
            hbin = 0;
          }
          if (thist) {
            // Nearby importances share bins: the lanes with the first lane's
            // bin are counted with one atomic.
            const int h0 = __builtin_amdgcn_readfirstlane(hbin);
            const uint64_t same = __ballot(hbin == h0);
            if (hbin == h0) {
              if (h0 < kBulkBins && lane == __builtin_ctzll(same)) atomicAdd(&whist[h0], (uint32_t)__popcll(same));
            } else if (hbin < kBulkBins) {
              atomicAdd(&whist[hbin], 1u);
            }
          }
        }
      };
      if (bulk && !split) {
        // Bulk in one block: the new token goes to slot Lold, then the unit's L
        // slots (the dead one included, keyed to go first) are cut to the
        // budget: select the L - beta lowest keys among the unprotected tokens
        // and move survivors from above the budget into the evicted slots
        // below it.  (A path of its own: the steady path after it then waits
        // for no load of the later batches.)
        for (int base = nb0; base < nb1; base += CHUNK) {
          if (base != nb0) load_batch(base);
          batch(base);
        }
        lds_barrier();  // s_newimp
        const float newimp = s_newimp;
        if (tid < 2 * NR) reinterpret_cast<uint4 *>((tid < NR ? kw : vw) + (size_t)Lold * RB)[tid % NR] =
              lds_read_u128(lds_addr(&s_nrow[tid]));
        if (tid == 0) {
          impw[Lold] = newimp;
          posw[Lold] = newest;
          unit_state(a, u)[0] = 0;
        }
        __syncthreads();  // every key is stored
        if constexpr (IB)
          bulk_compact<NTF, RB>(bkeys, L, beta, L - beta, kw, vw, posw, impw, a.ws.holes + (size_t)u * a.cap,
                                a.ws.movers + (size_t)u * a.cap, a.len + u, a.ws.status, hist, whist, sc, &rs,
                                nullptr);
        else
          bulk_cut_unit<NTF, RB>(bkeys, L, beta, kw, vw, posw, impw, a.ws.holes + (size_t)u * a.cap,
                            a.ws.movers + (size_t)u * a.cap, a.len + u, a.ws.status, (lds_u32 *)hist,
                            (lds_u32 *)whist, (lds_int *)sc, (lds_radix *)&rs);
        return;
      }
      batch(nb0);  // the block's tokens: one batch
      if (split) {
        __syncthreads();  // the histogram, s_newimp
        if (thist) {  // the block's counts join the unit's histogram
          uint32_t *dst = a.ws.uhist + (size_t)u * kBulkHistWords;
          for (int i = tid; i < kBulkBins; i += NTF) {
            const uint32_t c = whist[i];
            if (c) atomicAdd(&dst[i], c);
          }
        }
        if (nb1 == L) {  // the block holding slot Lold places the new token
          if (tid < 2 * NR) reinterpret_cast<uint4 *>((tid < NR ? kw : vw) + (size_t)fs * RB)[tid % NR] =
              lds_read_u128(lds_addr(&s_nrow[tid]));
          if (tid == 0) {
            impw[fs] = s_newimp;
            posw[fs] = newest;
          }
        }
        if (r == 0 && tid == 0) {
          unit_state(a, u)[0] = 0;
          // the slots the cut considers: a dead slot now holds the new token
          reinterpret_cast<int4 *>(a.ws.bsel)[u] = make_int4(n_evict, beta, fs == Lold ? L : Lold, 1);
        }
        return;
      }
      {
        wave_min_key(best, best_slot);
        if (lane == 0) {
          sk[wave] = best;
          ss[wave] = best_slot;
        }
        lds_barrier();  // s_newimp, the waves' lowest keys
        if (nb1 == L) {
          // The block holding slot Lold places the new token: into the dead
          // slot, or appended at Lold.
          if (tid < 2 * NR) reinterpret_cast<uint4 *>((tid < NR ? kw : vw) + (size_t)fs * RB)[tid % NR] =
              lds_read_u128(lds_addr(&s_nrow[tid]));
          if (tid == 0) {
            impw[fs] = s_newimp;
            posw[fs] = newest;
            if (dead < 0) a.len[u] = L;
          }
        }
        int32_t *cand = unit_state(a, u) + 4;
        if (n_evict == 1) {
          // The eviction stays pending: each block leaves its lowest key.
          if (wave == 0) {
            uint64_t kk = lane < NWF ? sk[lane] : ~0ull;
            int vs = lane < NWF ? ss[lane] : -1;
            wave_min_key(kk, vs);
            if (lane == 0) {
              cand[4 * r] = (int32_t)(uint32_t)kk;
              cand[4 * r + 1] = (int32_t)(uint32_t)(kk >> 32);
              cand[4 * r + 2] = vs;
              if (r == 0) unit_state(a, u)[0] = nact;
            }
          }
        } else if (r == 0 && tid == 0) {
          unit_state(a, u)[0] = 0;
        }
      }
    }();
    end_wave();
  }
  if constexpr (S2) {
    // ---------------- Stage II output block: head r - nib ----------------
    const int beta = a.budget ? ld_vec(a.budget + u, vz) : a.budget_all;
    const int dead = ld_vec(unit_state(a, u) + 1, vz);
    const int newest = ld_vec(a.new_pos + b, vz);
    s2_out_block<G, KR>(a, u, r - nib, L, dead, newest, a.hp.n && (L > a.cap || beta < S || beta > a.cap));
  } else {
  // ---------------- output block: chunk c of the unit's G*D outputs ----
  const int beta_ld = ld_opaque(a.budget ? a.budget + u : a.new_pos + b, vz);
  const float2 v0 = pml[min(tid, npair - 1)];
  const int c = r - nib;
  const int o = c * 64 + lane, g = (c * 64) / D;
  const float *pacc = a.ws.part_acc + (size_t)tb * GD + o;
  float pa[NTW];
#pragma unroll
  for (int i = 0; i < NTW; ++i) pa[i] = pacc[(size_t)min(wave + NWF * i, nt - 1) * GD];
  const int beta = a.budget ? beta_ld : a.budget_all;
  float Mlane, Llane;
  unit_stats<G, NTF>(pml, npair, v0, a.scale_log2, red, red2, Mlane, Llane, sm_m, g);
  const float Mo = lane_value(Mlane, g), Lo = lane_value(Llane, g);
  float *outu = a.out + (size_t)(b * a.Hq + j * G) * D;
  if (a.hp.n && (L > a.cap || beta < S || beta > a.cap)) {  // unit left alone
    if (wave == 0) outu[o] = 0.f;
    end_wave();
  }
  const float Ms = (Mo == -INFINITY) ? 0.f : Mo;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < NTW; ++i) {
    const int t = wave + NWF * i;
    if (t < nt) acc += pa[i] * fast_exp2((sm_m[t] - Ms) * a.scale_log2);
  }
  for (int t = wave + NWF * NTW; t < nt; t += NWF)
    acc += pacc[(size_t)t * GD] * fast_exp2((sm_m[t] - Ms) * a.scale_log2);
  red_o[wave][lane] = acc;
  lds_barrier();
  if (wave == 0) {
    float sum = 0.f;
    for (int w = 0; w < NWF; ++w) sum += red_o[w][lane];
    outu[o] = sum / Lo;
  }
  }

  end_wave();
}

// ---------------------------------------------------------------------------
// Block-granular eviction ("KV Cache Compression and Dynamic Pruning in
// Production Serving", Sec. 5, PagedAttention block fragmentation): the keys
// of a unit cut in bulk when whole blocks of P positions go (block id =
// pos / P).  k_pos_rank has listed the unit's slots in position order
// (ws.order); workgroup r takes the ranks [r kImpChunk, (r + 1) kImpChunk)
// and loads them, with the P - 1 after them and the one before, into LDS.  A
// rank that starts a block (the rank before it lies in another block) sums the
// block's importance in position order -- fp32, the same order every call --
// notes whether any of its tokens is protected, and gives every token of the
// block the block's key: evict_key with the block sum and the block id, so
// that equal sums send the higher block first, or no key (~0) when protected.
// The workgroup leaves the histogram of its keys' top bits as the importance
// blocks do for single tokens; k_bulk_select then takes every key up to the
// need-th smallest, which is whole blocks since a block's tokens share one key.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int floor_div(int x, int p) { return x >= 0 ? x / p : -((-x + p - 1) / p); }

__global__ __launch_bounds__(kT2) void k_block_keys(StepArgs a) {
  constexpr int NL = kImpChunk + HIKV_MAX_BLOCK_TOKENS;  // ranks an LDS copy holds
  __shared__ int s_slot[NL];
  __shared__ int s_pos[NL];
  __shared__ float s_imp[NL];
  __shared__ uint32_t whist[kBulkBins];
  const int u = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const int4 bs = reinterpret_cast<const int4 *>(a.ws.bsel)[u];
  if (bs.w != 1) return;  // not cut this step
  const int beta = bs.y, L = bs.z, P = a.block;
  const int i0 = r * kImpChunk;
  if (i0 >= L) return;
  const int iend = min(L, i0 + kImpChunk);  // ranks whose blocks may start here
  const int lo = max(i0 - 1, 0), hi = min(L, i0 + kImpChunk + P - 1);  // ranks loaded
  const int32_t *order = a.ws.order + (size_t)u * a.cap;
  const int32_t *posw = a.pos + (size_t)u * a.cap;
  const float *impw = a.imp + (size_t)u * a.cap;
  uint64_t *bkeys = a.ws.bkeys + (size_t)u * a.cap;
  for (int k = tid; k < hi - lo; k += kT2) {
    const int sl = min(max(order[lo + k], 0), a.cap - 1);
    s_slot[k] = sl;
    s_pos[k] = posw[sl];
    s_imp[k] = impw[sl];
  }
  for (int i = tid; i < kBulkBins; i += kT2) whist[i] = 0u;
  __syncthreads();
  const int b = u / a.Hkv;
  const int S = a.n_sink, newest = a.new_pos[b], Wp = min(a.n_recent, beta - S);
  for (int i = i0 + tid; i < iend; i += kT2) {
    const int k = i - lo;
    const int blk = floor_div(s_pos[k], P);
    if (i > 0 && floor_div(s_pos[k - 1], P) == blk) continue;  // not the first rank of its block
    float sum = 0.f;
    bool prot = false;
    int m = 0;
    for (int j = k; j < hi - lo && floor_div(s_pos[j], P) == blk; ++j, ++m) {
      sum += s_imp[j];
      prot = prot || s_pos[j] < S || s_pos[j] > newest - Wp;
    }
    const uint64_t key = prot ? ~0ull : evict_key(sum, blk);
    for (int j = k; j < k + m; ++j) bkeys[s_slot[j]] = key;
    if (!prot) atomicAdd(&whist[(int)(key >> kBulkShift)], (uint32_t)m);
  }
  __syncthreads();
  uint32_t *dst = a.ws.uhist + (size_t)u * kBulkHistWords;
  for (int i = tid; i < kBulkBins; i += kT2) {
    const uint32_t c = whist[i];
    if (c) atomicAdd(&dst[i], c);
  }
}

// ---------------------------------------------------------------------------
// A bulk cut (when the host can tell, and always for whole blocks) ends in
// launches of its own.  The importance blocks (or k_block_keys) leave every
// slot's eviction key (~0: protected) and add a histogram of the keys' top
// kBulkBits bits to the unit's, which the attention launch cleared.  The
// n_evict smallest keys go:
//  - k_bulk_mark, one workgroup per kMarkSlots slots of a unit: the histogram's
//    prefix gives the bin holding the n_evict-th smallest key (need: how many
//    of the bin's keys go; cnt: how many it holds).  Each workgroup marks its
//    slots whose key lies below the bin in a bitmap (one word per 64 slots)
//    and appends the bin's keys and slots to the unit's candidate list; the
//    first leaves the bin in the unit's record.  A bin of more than kBulkCand
//    keys, or a unit longer than the select's LDS bitmap, is left to the select
//    (kCutSlow).
//  - k_bulk_select, a few workgroups per unit: the need-th smallest candidate
//    (radix passes in LDS) is the threshold; the candidates up to it join the
//    bitmap, and the holes (marked slots below the new length) and movers
//    (unmarked live slots at or above it) are listed in ascending slot order
//    for k_bulk_moves, each workgroup listing its share of the bitmap's words.
//    With kCutSlow one workgroup finds the bin itself, narrowing it by
//    passes over the keys until it holds at most kBulkCand keys, and gathers it.
// Whole blocks: a block's tokens share one key, so the keys up to the threshold
// are whole blocks and the new length is L less those; when protected blocks
// leave fewer candidates than the need every candidate goes, and with none the
// unit stays as it is (kCutKeep).
// ---------------------------------------------------------------------------
constexpr int kBulkMapSlots = 1 << 18;  // slots the select's LDS bitmap covers (32 KB)
constexpr int kMarkKpt = 8, kMarkSlots = kMarkKpt * kT2;  // k_bulk_mark: keys per thread, per workgroup
constexpr int kBulkKpt = 16;            // keys per thread per pass in flight (kCutSlow)
// The record, words kBulkRec.. of a unit's uhist row: candidates appended, bin,
// need, cnt, mode.
enum : int { kCutNone = 0, kCutFast = 1, kCutSlow = 2, kCutKeep = 3, kCutError = 4 };

struct BinPick {
  int bin, need, cnt, tot;
};

// The bin of a 2 NT-bin histogram (bins 2 tid, 2 tid + 1 in c0, c1) holding
// the need-th smallest counted key (bin -1: fewer keys), and the count of every
// key; every thread sees the same *bp on return.
template <int NT>
__device__ void pick_bin(uint32_t c0, uint32_t c1, int need, int *sc, BinPick *bp) {
  const int tid = threadIdx.x;
  if (tid == 0) bp->bin = -1;
  int tot;
  const int ex = block_excl_scan<NT>((int)(c0 + c1), sc, &tot);  // (its barriers order the writes)
  if (tid == 0) bp->tot = tot;
  if (ex < need && ex + (int)(c0 + c1) >= need) {
    const bool first = ex + (int)c0 >= need;
    bp->bin = first ? 2 * tid : 2 * tid + 1;
    bp->need = first ? need - ex : need - ex - (int)c0;
    bp->cnt = first ? (int)c0 : (int)c1;
  }
  __syncthreads();
}

// The cut's bin from the unit's histogram, k keys to go.  Whole blocks: fewer
// candidates than k all go (none: kCutKeep).  Returns kCutFast or the mode
// that ends the cut.
template <int NT>
__device__ int cut_bin(uint32_t c0, uint32_t c1, int k, bool blocks, int *sc, BinPick *bp) {
  pick_bin<NT>(c0, c1, k, sc, bp);
  if (bp->bin < 0 && blocks) {
    const int tot = bp->tot;
    __syncthreads();  // every thread has read *bp
    if (tot == 0) return kCutKeep;
    pick_bin<NT>(c0, c1, tot, sc, bp);
  }
  return bp->bin < 0 ? kCutError : kCutFast;
}

__global__ __launch_bounds__(kT2) void k_bulk_mark(StepArgs a) {
  static_assert(kBulkBins == 2 * kT2, "two histogram bins per thread");
  constexpr int KPT = kMarkKpt;
  __shared__ int sc[kNW2];
  __shared__ BinPick bp;
  __shared__ uint64_t lk[kBulkCand];
  __shared__ int ls[kBulkCand];
  __shared__ int s_nc, s_base;
  const int u = blockIdx.x, r = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t *uh = a.ws.uhist + (size_t)u * kBulkHistWords;
  const uint64_t *keys = a.ws.bkeys + (size_t)u * a.cap;
  const int i0 = r * kMarkSlots;
  // Issued together: the cut's parameters, the histogram's two bins, the keys.
  const int4 bs = reinterpret_cast<const int4 *>(a.ws.bsel)[u];
  const uint2 hv = reinterpret_cast<const uint2 *>(uh)[tid];
  uint64_t kk[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) kk[j] = keys[min(i0 + j * kT2 + tid, a.cap - 1)];
  kernarg_warm(0);
  if (bs.w != 1) return;  // not cut in bulk
  const int k = bs.x, L = bs.z;
  if (i0 >= L) return;
  if (tid == 0) s_nc = 0;
  int mode = cut_bin<kT2>(hv.x, hv.y, k, a.block != 0, sc, &bp);
  const int bin = bp.bin, need = bp.need, cnt = bp.cnt;
  if (mode == kCutFast && (cnt > kBulkCand || L > kBulkMapSlots)) mode = kCutSlow;
  if (r == 0 && tid == 0) {
    uh[kBulkRec + 1] = (uint32_t)bin;
    uh[kBulkRec + 2] = (uint32_t)need;
    uh[kBulkRec + 3] = (uint32_t)cnt;
    uh[kBulkRec + 4] = (uint32_t)mode;
  }
  if (mode != kCutFast) return;
  const bool all = need == cnt;  // the whole bin goes
  uint64_t *ebits = a.ws.ebits + (size_t)u * ((a.cap + 63) / 64);
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int n = i0 + j * kT2 + tid;
    const bool valid = n < L && kk[j] != ~0ull;
    const int top = (int)(kk[j] >> kBulkShift);
    const uint64_t m = __ballot(valid && (top < bin || (all && top == bin)));
    const int s0 = i0 + j * kT2 + wave * 64;  // the wave's first slot
    if (lane == 0 && s0 < L) ebits[s0 / 64] = m;
    const bool c = valid && !all && top == bin;
    const uint64_t mc = __ballot(c);
    if (mc) {  // one LDS atomic per wave
      int b0 = 0;
      if (lane == 0) b0 = atomicAdd(&s_nc, __popcll(mc));
      b0 = __shfl(b0, 0);
      const int i = b0 + __popcll(mc & ((1ull << lane) - 1ull));
      if (c && i < kBulkCand) {
        lk[i] = kk[j];
        ls[i] = n;
      }
    }
  }
  __syncthreads();
  const int nc = min(s_nc, kBulkCand);
  if (nc == 0) return;
  if (tid == 0) s_base = (int)atomicAdd(&uh[kBulkRec], (uint32_t)s_nc);
  __syncthreads();
  const int base = s_base;
  uint64_t *cand = a.ws.cand + (size_t)u * kBulkCand;
  int32_t *cslot = a.ws.cslot + (size_t)u * kBulkCand;
  for (int i = tid; i < nc && base + i < kBulkCand; i += kT2) {
    cand[base + i] = lk[i];
    cslot[base + i] = ls[i];
  }
}

// Exclusive prefix sums of two values over the block, in one exchange; sc
// holds 2 NT / 64 words.
template <int NT>
__device__ void block_excl_scan2(int va, int vb, int *sc, int *ea, int *eb, int *ta, int *tb) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int ia = va, ib = vb;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int ya = __shfl_up(ia, off), yb = __shfl_up(ib, off);
    if (lane >= off) ia += ya, ib += yb;
  }
  if (lane == 63) sc[wave] = ia, sc[NW + wave] = ib;
  __syncthreads();
  int ba = 0, bb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int xa = sc[w], xb = sc[NW + w];
    if (w < wave) ba += xa, bb += xb;
    sa += xa;
    sb += xb;
  }
  *ta = sa;
  *tb = sb;
  *ea = ba + ia - va;
  *eb = bb + ib - vb;
  __syncthreads();  // sc is free for the next call
}

template <int RB>
__global__ __launch_bounds__(kT2) void k_bulk_select(StepArgs a) {
  static_assert(kBulkBins == 2 * kT2, "two histogram bins per thread");
  constexpr int NT = kT2, KPT = kBulkKpt, NMW = kBulkMapSlots / 64;
  static_assert(NMW == 4 * NT && kBulkCand == 4 * NT, "four bitmap words and four candidates per thread");
  __shared__ uint32_t h[kBulkBins];
  __shared__ uint64_t ck[kBulkCand];
  __shared__ int cs[kBulkCand];
  __shared__ uint64_t eb[NMW];
  __shared__ int sc[2 * kNW2];
  __shared__ BinPick bp;
  __shared__ int s_bin, s_need, s_cnt, s_nc;
  // Workgroup y of a unit lists its share of the bitmap's words (kCutFast; the
  // rest of the select, which every workgroup of the unit repeats, gives each
  // the same bitmap and prefixes); kCutSlow is workgroup 0's alone.
  const int u = blockIdx.x, sl = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t *uh = a.ws.uhist + (size_t)u * kBulkHistWords;
  // Issued together (one round trip): the cut's parameters, the record
  // k_bulk_mark left, and what it gathered -- the bitmap words and the
  // candidates, from clamped addresses, used only in kCutFast.
  const int4 bs = reinterpret_cast<const int4 *>(a.ws.bsel)[u];
  const int4 rec = reinterpret_cast<const int4 *>(uh + kBulkRec)[0];  // candidates, bin, need, cnt
  const int mode = (int)uh[kBulkRec + 4];
  const int nwc = (a.cap + 63) / 64;
  uint64_t ev[4], cv[4];
  int sv[4];
  {
    const uint64_t *cand = a.ws.cand + (size_t)u * kBulkCand;
    const int32_t *cslot = a.ws.cslot + (size_t)u * kBulkCand;
    const uint64_t *ebits = a.ws.ebits + (size_t)u * nwc;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = tid + q * NT;
      ev[q] = ebits[min(i, nwc - 1)];
      cv[q] = cand[i];
      sv[q] = cslot[i];
    }
  }
  kernarg_warm(0);
  if (bs.w != 1) return;  // not cut in bulk
  const int beta = bs.y, L = bs.z;
  const uint64_t *keys = a.ws.bkeys + (size_t)u * a.cap;
  // The unit's length after the cut: the budget, or, when whole blocks go
  // (every key of a block is the same), L less every key up to the threshold.
  int newlen = beta;
  if (mode == kCutKeep) {
    if (tid == 0 && sl == 0) a.len[u] = L;
    return;
  }
  if (mode != kCutFast && mode != kCutSlow) {  // fewer candidates than tokens to evict: cannot happen
    if (tid == 0) set_status(a.ws.status, HIKV_EINVAL);
    return;
  }
  if (mode == kCutSlow && sl != 0) return;
  uint64_t prefix;  // the bin: the keys' top pbits bits
  int pbits = kBulkBits, need, cnt;
  const bool use_map = L <= kBulkMapSlots;
  if (mode == kCutFast) {
    // The bin, its candidates and the bitmap below it, as k_bulk_mark left
    // them.
    prefix = (uint64_t)rec.y;
    need = rec.z;
    cnt = rec.w;
    const int nw = (L + 63) / 64;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = tid + q * NT;
      if (i < nw) eb[i] = ev[q];
      if (i < rec.x) {
        ck[i] = cv[q];
        cs[i] = min(max(sv[q], 0), L - 1);
      }
    }
    if (rec.x != (need == cnt ? 0 : cnt)) {  // the histogram and the keys disagree: cannot happen
      if (tid == 0) set_status(a.ws.status, HIKV_EINVAL);
      return;
    }
    __syncthreads();
  } else {
    // The bin from the histogram, narrowed while it holds more than kBulkCand
    // keys by one pass over the keys per kBulkBits bits; then one pass marks
    // the slots below it (LDS bitmap) and gathers its keys and slots.
    const uint2 hv = reinterpret_cast<const uint2 *>(uh)[tid];
    if (cut_bin<NT>(hv.x, hv.y, bs.x, a.block != 0, sc, &bp) != kCutFast) {  // cannot happen
      if (tid == 0) set_status(a.ws.status, HIKV_EINVAL);
      return;
    }
    prefix = (uint64_t)bp.bin;
    need = bp.need;
    cnt = bp.cnt;
    while (cnt > kBulkCand && pbits < 64) {
      const int nb = min(kBulkBits, 64 - pbits), sh = 64 - pbits - nb;
      for (int i = tid; i < kBulkBins; i += NT) h[i] = 0u;
      __syncthreads();
      for (int n0 = 0; n0 < L; n0 += KPT * NT) {
        uint64_t kk[KPT];
#pragma unroll
        for (int j = 0; j < KPT; ++j) kk[j] = keys[min(n0 + j * NT + tid, L - 1)];
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
          const bool in = n0 + j * NT + tid < L && kk[j] != ~0ull && (kk[j] >> (64 - pbits)) == prefix;
          const int d = in ? (int)((kk[j] >> sh) & ((1ull << nb) - 1ull)) : kBulkBins;
          const int d0 = __builtin_amdgcn_readfirstlane(d);
          const uint64_t same = __ballot(d == d0);
          if (d == d0) {
            if (d0 < kBulkBins && lane == __builtin_ctzll(same)) atomicAdd(&h[d0], (uint32_t)__popcll(same));
          } else if (d < kBulkBins) {
            atomicAdd(&h[d], 1u);
          }
        }
      }
      __syncthreads();
      pick_bin<NT>(h[2 * tid], h[2 * tid + 1], need, sc, &bp);
      if (bp.bin < 0) {
        if (tid == 0) set_status(a.ws.status, HIKV_EINVAL);
        return;
      }
      prefix = (prefix << nb) | (uint64_t)bp.bin;
      pbits += nb;
      need = bp.need;
      cnt = bp.cnt;
      __syncthreads();  // every thread has read bp and h
    }
    const int tsh = 64 - pbits;
    const bool all = need == cnt;
    if (tid == 0) s_nc = 0;
    __syncthreads();
    for (int n0 = 0; n0 < L; n0 += KPT * NT) {
      uint64_t kk[KPT];
#pragma unroll
      for (int j = 0; j < KPT; ++j) kk[j] = keys[min(n0 + j * NT + tid, L - 1)];
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int n = n0 + j * NT + tid;
        const bool valid = n < L && kk[j] != ~0ull;
        const uint64_t top = tsh >= 64 ? 0ull : (kk[j] >> tsh);
        const bool ev = valid && (top < prefix || (all && top == prefix));
        const bool c = valid && !all && top == prefix;
        if (use_map) {
          const uint64_t m = __ballot(ev);
          if (lane == 0 && n0 + j * NT < L) eb[(n0 + j * NT) / 64 + wave] = m;
        }
        const uint64_t mc = __ballot(c);  // one atomic per wave
        int b0 = 0;
        if (lane == 0 && mc) b0 = atomicAdd(&s_nc, __popcll(mc));
        b0 = __shfl(b0, 0);
        const int i = b0 + __popcll(mc & ((1ull << lane) - 1ull));
        if (c && i < kBulkCand) ck[i] = kk[j], cs[i] = n;
      }
    }
    __syncthreads();
    if (!all && s_nc != cnt) {  // the histogram and the keys disagree: cannot happen
      if (tid == 0) set_status(a.ws.status, HIKV_EINVAL);
      return;
    }
  }
  const int tsh = 64 - pbits;    // bits below the bin's
  const bool all = need == cnt;  // the whole bin goes

  // 3. The need-th smallest key of the bin: radix passes of 8 bits over the
  // gathered keys, below the bits the bin fixes.  T: the largest key that goes.
  uint64_t T;
  if (all) {
    T = (prefix << tsh) | (tsh == 0 ? 0ull : ((1ull << tsh) - 1ull));
  } else {
    uint64_t pre = prefix << tsh;  // the bits fixed so far
    int rem = tsh, nd = need, nc = cnt;
    while (rem > 0 && nd < nc) {
      const int nb = min(8, rem), sh = rem - nb;
      if (tid < 256) h[tid] = 0u;
      __syncthreads();
      for (int i = tid; i < cnt; i += NT) {
        const uint64_t key = ck[i];
        const bool in = (key >> rem) == (pre >> rem);
        const int d = in ? (int)((key >> sh) & ((1ull << nb) - 1ull)) : 256;
        const int d0 = __builtin_amdgcn_readfirstlane(d);
        const uint64_t same = __ballot(d == d0);
        if (d == d0) {
          if (d0 < 256 && lane == __builtin_ctzll(same)) atomicAdd(&h[d0], (uint32_t)__popcll(same));
        } else if (d < 256) {
          atomicAdd(&h[d], 1u);
        }
      }
      __syncthreads();
      if (wave == 0) {
        const uint32_t h0 = h[4 * lane], h1 = h[4 * lane + 1], h2 = h[4 * lane + 2], h3 = h[4 * lane + 3];
        const uint32_t s4 = h0 + h1 + h2 + h3;
        const uint32_t incl = wave_incl_scan_u32(s4), excl = incl - s4;
        if (excl < (uint32_t)nd && incl >= (uint32_t)nd) {
          // (named values: a small array indexed at run time goes to scratch)
          const uint32_t c1 = excl + h0, c2 = c1 + h1, c3 = c2 + h2, want = (uint32_t)nd;
          const int d = c1 >= want ? 0 : (c2 >= want ? 1 : (c3 >= want ? 2 : 3));
          const uint32_t cum = d == 0 ? excl : (d == 1 ? c1 : (d == 2 ? c2 : c3));
          s_bin = 4 * lane + d;
          s_need = nd - (int)cum;
          s_cnt = (int)(d == 0 ? h0 : (d == 1 ? h1 : (d == 2 ? h2 : h3)));
        }
      }
      __syncthreads();
      pre |= (uint64_t)s_bin << sh;
      nd = s_need;
      nc = s_cnt;
      rem = sh;
      __syncthreads();  // h is cleared for the next pass
    }
    T = pre | (rem == 0 ? 0ull : ((1ull << rem) - 1ull));
    if (use_map)
      for (int i = tid; i < cnt; i += NT)
        if (ck[i] <= T) atomicOr(reinterpret_cast<unsigned long long *>(&eb[cs[i] >> 6]), 1ull << (cs[i] & 63));
  }
  char *kw = static_cast<char *>(a.k_w) + (size_t)u * a.cap * RB;
  char *vw = static_cast<char *>(a.v_w) + (size_t)u * a.cap * RB;
  int32_t *holes = a.ws.holes + (size_t)u * a.cap, *movers = a.ws.movers + (size_t)u * a.cap;
  if (!use_map) {  // a key goes exactly when it is at most T
    if (a.block) {
      int c = 0;
      for (int n = tid; n < L; n += NT) c += (keys[n] != ~0ull && keys[n] <= T) ? 1 : 0;
      int tot;
      block_excl_scan<NT>(c, sc, &tot);
      newlen = L - tot;
    }
    bulk_list<NT, RB>(keys, L, newlen, T, 0, kw, vw, a.pos + (size_t)u * a.cap, a.imp + (size_t)u * a.cap,
                      holes, movers, a.len + u, a.ws.status, reinterpret_cast<uint64_t *>(ck), sc,
                      a.ws.nmoves + u);
    return;
  }
  __syncthreads();  // the bitmap is complete

  // 4. Holes and movers from the bitmap.  Each thread counts a run of words;
  // the runs' prefix gives every word the list positions of its first hole and
  // mover (ph, pm: LDS over ck, which is free now), and then each wave lists
  // whole words, one slot per lane, so that a word's entries go out together.
  const int nw = (L + 63) / 64, wpt = (nw + NT - 1) / NT;
  const int w0 = min(tid * wpt, nw), w1 = min(w0 + wpt, nw);
  auto below = [](int c) -> uint64_t { return c <= 0 ? 0ull : (c >= 64 ? ~0ull : ((1ull << c) - 1ull)); };
  if (a.block) {
    int c = 0;
    for (int w = w0; w < w1; ++w) c += __popcll(eb[w] & below(L - 64 * w));
    int tot;
    block_excl_scan<NT>(c, sc, &tot);
    newlen = L - tot;
  }
  int nh = 0, nm = 0;
  for (int w = w0; w < w1; ++w) {
    const uint64_t e = eb[w], valid = below(L - 64 * w), low = below(newlen - 64 * w);
    nh += __popcll(e & valid & low);
    nm += __popcll(~e & valid & ~low);
  }
  int th, tm, ih, im;
  block_excl_scan2<NT>(nh, nm, sc, &ih, &im, &th, &tm);
  int *ph = reinterpret_cast<int *>(ck), *pm = ph + NMW;
  for (int w = w0; w < w1; ++w) {
    const uint64_t e = eb[w], valid = below(L - 64 * w), low = below(newlen - 64 * w);
    ph[w] = ih;
    pm[w] = im;
    ih += __popcll(e & valid & low);
    im += __popcll(~e & valid & ~low);
  }
  __syncthreads();
  // Four words per wave at a time, their LDS reads issued together; the word
  // index is the wave's, so the masks are scalar work.  A lane's rank among
  // a word's listed slots is the count of listed bits below it (mbcnt).
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int per = mode == kCutFast ? (nw + (int)gridDim.y - 1) / (int)gridDim.y : nw;
  const int lw0 = mode == kCutFast ? sl * per : 0, lw1 = min(lw0 + per, nw);  // this workgroup's words
  auto put = [&](uint64_t m, int first, int slot, int32_t *list) __attribute__((always_inline)) {
    const uint32_t lo = (uint32_t)m, hi = (uint32_t)(m >> 32);
    const uint32_t mine = (lane < 32 ? lo >> lane : hi >> (lane - 32)) & 1u;
    if (mine) list[first + (int)__builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u))] = slot;
  };
  for (int wb = lw0 + wv; wb < lw1; wb += 4 * kNW2) {
    uint64_t e[4];
    int h0[4], m0[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int w = min(wb + q * kNW2, lw1 - 1);
      e[q] = eb[w];
      h0[q] = ph[w];
      m0[q] = pm[w];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int w = wb + q * kNW2;
      if (w >= lw1) break;
      const int slot = 64 * w + lane;
      if (64 * w + 64 <= newlen) {  // every slot below the new length: holes only
        put(e[q], h0[q], slot, holes);
      } else if (64 * w >= newlen && 64 * w + 64 <= L) {  // every slot live, at or above it: movers only
        put(~e[q], m0[q], slot, movers);
      } else {
        const uint64_t valid = below(L - 64 * w), low = below(newlen - 64 * w);
        put(e[q] & valid & low, h0[q], slot, holes);
        put(~e[q] & valid & ~low, m0[q], slot, movers);
      }
    }
  }
  if (tid == 0 && sl == 0) {
    if (th != tm) {  // cannot happen for distinct positions; fail safe
      set_status(a.ws.status, HIKV_EINVAL);
    } else {
      a.ws.nmoves[u] = tm;
      a.len[u] = newlen;
    }
  }
}

// ---------------------------------------------------------------------------
// Fourth launch of a step that cuts units in bulk (when the host can tell): the
// rows k_bulk_select listed move from above the budget into the evicted
// slots below it (K and V rows, position, importance): workgroup y of a unit
// takes moves [64 y, 64 y + 64) (bf16 rows of 128; fewer for wider rows),
// the host sizing the grid from its bound on any unit's moves.  Hole and
// mover lists pair up in order; every source and destination is distinct, so
// the moves are independent.
// ---------------------------------------------------------------------------
template <int RB>
__global__ __launch_bounds__(256) void k_bulk_moves(StepArgs a) {
  constexpr int CPR = RB / 16, RPP = 256 / CPR;  // threads per row, rows per pass (4 passes)
  static_assert(RPP * 4 == bulk_moves_per_wg(RB), "moves per workgroup");
  const int tid = threadIdx.x, lane = tid & 63;
  int u = blockIdx.x, y0 = blockIdx.y;
  // The chunk table's words (kernel arguments, always readable) are loaded
  // before the flag that says whether there is one is known.
  const int mvend = a.hp.mvb[min(lane, kHostPlanUnits - 1) + 1];
  kernarg_warm(0);
  if (a.moves_flat) {
    // One chunk of one unit's moves: the unit is the number of units whose
    // chunks end at or before this workgroup's.
    const int end = lane < a.n_units ? mvend : 0x7fffffff;
    u = (int)__builtin_amdgcn_readfirstlane(__popcll(__ballot(end <= (int)blockIdx.x)));
    y0 = (int)blockIdx.x - (u > 0 ? __builtin_amdgcn_readlane(end, u - 1) : 0);
  }
  const int ci = tid % CPR, rr = tid / CPR;
  const int32_t *holes = a.ws.holes + (size_t)u * a.cap, *movers = a.ws.movers + (size_t)u * a.cap;
  char *kw = static_cast<char *>(a.k_w) + (size_t)u * a.cap * RB;
  char *vw = static_cast<char *>(a.v_w) + (size_t)u * a.cap * RB;
  int32_t *posw = a.pos + (size_t)u * a.cap;
  float *impw = a.imp + (size_t)u * a.cap;
  // The count and the group's list entries are loaded together (the entries
  // from clamped addresses; an entry past the count is a stale slot number,
  // clamped, read and not used), so the rows follow one round trip later.
  // Four moves per thread group in named registers (arrays of 16-byte
  // vectors are not kept in registers by the compiler).
  const int nm = a.ws.nmoves[u];
  auto ent = [&](const int32_t *l, int i) { return min(max(l[min(i, a.cap - 1)], 0), a.cap - 1); };
  auto row = [&](const char *base, int slot) { return reinterpret_cast<const uint4 *>(base + (size_t)slot * RB)[ci]; };
  auto put = [&](int i, int dst, const uint4 &k, const uint4 &v, int p, float x) {
    if (i < nm) {
      reinterpret_cast<uint4 *>(kw + (size_t)dst * RB)[ci] = k;
      reinterpret_cast<uint4 *>(vw + (size_t)dst * RB)[ci] = v;
      if (ci == 0) posw[dst] = p, impw[dst] = x;
    }
  };
  // Moves [RPP 4 y, RPP 4 (y + 1)) for y = y0, y0 + gridDim.y, ... (one y
  // when the host sized the grid to the moves).
  for (int y = y0;; y += (int)gridDim.y) {
    const int i0 = y * RPP * 4 + rr;  // this group's moves: i0, i0 + RPP, ...
    const int ia = i0, ib = i0 + RPP, ic = i0 + 2 * RPP, id = i0 + 3 * RPP;
    const int sa = ent(movers, ia), sb = ent(movers, ib), sc = ent(movers, ic), sd = ent(movers, id);
    const int da = ent(holes, ia), db = ent(holes, ib), dc = ent(holes, ic), dd = ent(holes, id);
    if (y * RPP * 4 >= nm) return;  // past this unit's moves
    const uint4 ka = row(kw, sa), kb = row(kw, sb), kc = row(kw, sc), kd = row(kw, sd);
    const uint4 va = row(vw, sa), vb = row(vw, sb), vc = row(vw, sc), vd = row(vw, sd);
    const int pa = posw[sa], pb = posw[sb], pc = posw[sc], pd = posw[sd];
    const float xa = impw[sa], xb = impw[sb], xc = impw[sc], xd = impw[sd];
    put(ia, da, ka, va, pa, xa);
    put(ib, db, kb, vb, pb, xb);
    put(ic, dc, kc, vc, pc, xc);
    put(id, dd, kd, vd, pd, xd);
    if (a.moves_flat) return;  // one chunk per workgroup
  }
}

// The move launch's grid: one workgroup per chunk of the host's per-unit
// bounds (moves_flat), else per unit one workgroup per bulk_moves_per_wg
// moves of the largest bound; a bound that is only the capacity (no caller's
// lengths) takes at most 8 per unit, each looping over its share.
// The select's grid: per unit, one workgroup per 4096 slots of the longest
// unit, each listing its share of the bitmap's words, with at most one
// workgroup per CU in all (the select's LDS).
static dim3 select_grid(const StepArgs &a) {
  int mx = a.cap;
  if (a.hp.n == a.n_units) {
    mx = 1;
    for (int u = 0; u < a.hp.n; ++u) mx = max(mx, a.hp.L[u] + 1);
  }
  const int sl = (min(mx, kBulkMapSlots) + 4095) / 4096;
  return dim3((unsigned)a.n_units, (unsigned)max(1, min(sl, 256 / max(1, a.n_units))));
}

template <int RB>
static dim3 moves_grid(const StepArgs &a) {
  if (a.moves_flat) return dim3((unsigned)a.hp.mvb[a.hp.n]);
  const int per = bulk_moves_per_wg(RB);
  const int gy = max(1, (a.bulk_rows + per - 1) / per);
  return dim3((unsigned)a.n_units, (unsigned)(a.bulk_known ? gy : min(gy, 8)));
}

// ---------------------------------------------------------------------------
// Resolution of the pending eviction, one wave per unit: the dead slot (the
// lowest of the unit's candidate keys), reported in slot_out when given
// (-1: none pending); with apply, the unit's last slot moves into it (K and V
// rows, position, importance) and len drops by one, as if the step had
// evicted in place.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kWave) void k_settle(StepArgs a, int32_t *slot_out, int apply, int rb) {
  const int u = blockIdx.x;
  if (slot_out) {
    const int d = pending_slot_wave(a, u);
    if (threadIdx.x == 0) slot_out[u] = d;
  }
  if (apply) settle_unit(a, u, rb);
}

hipError_t launch_settle(const StepArgs &a, int dtype, int32_t *slot_out, bool apply, hipStream_t s) {
  const int rb = a.D * (dtype == HIKV_BF16 ? 2 : 4);
  hipLaunchKernelGGL(k_settle, dim3((unsigned)a.n_units), dim3(kWave), 0, s, a, slot_out, apply ? 1 : 0, rb);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
// The attention kernel of a configuration: matrix cores for bf16 with
// D = 128, vector ALUs otherwise.
template <int EL, int D, int G>
static constexpr bool use_mfma() { return EL == 2 && D == 128; }
template <int EL, int D, int G, bool S2 = false>
static void (*attend_kernel())(StepArgs) {
  if constexpr (S2) return k_attend_s2<G, 2>;
  else if constexpr (use_mfma<EL, D, G>()) return k_attend_mfma<G, 2>;
  else return k_attend<EL, D, G>;
}

template <int EL, int D, int G, bool S2 = false>
static int attend_grid(int n_units) {
  static int per_cu_cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int &pc = per_cu_cache[dev];
  if (pc == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attend_kernel<EL, D, G, S2>(), kThreads, 0) !=
        hipSuccess)
      return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    pc = per_cu * cus;
  }
  // One resident round of tiles, and at least 64 tiles beyond one per unit.
  return min(max(pc, n_units + 64), kMaxGrid);
}

template <int EL, int D, int G>
static hipError_t step_go(const StepArgs &a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const int g = attend_grid<EL, D, G>(a.n_units);
  if (g <= 0) return hipErrorInvalidValue;
  const dim3 grid(g), block(kThreads);
  hipError_t e;
  void (*kern)(StepArgs) = attend_kernel<EL, D, G>();
  if (ev0 && ev1) {
    // The events are recorded by the dispatch itself: they time the kernel's
    // execution, not the command processor's way to it.
    hipExtLaunchKernelGGL(kern, grid, block, 0, s, ev0, ev1, 0, a);
  } else {
    hipLaunchKernelGGL(kern, grid, block, 0, s, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // Second launch: per unit, importance blocks to cover the capacity, then
  // one output block per 64 outputs.
  // With a host plan the longest unit is known: no importance blocks beyond
  // its length are launched (they would only start and exit).
  int nib = imp_blocks(a.cap);
  if (a.hp.n) {
    int mx = 1;
    for (int u = 0; u < a.hp.n; ++u) mx = max(mx, a.hp.L[u]);
    nib = min(nib, (mx + kImpChunk - 1) / kImpChunk);
  }
  const dim3 g2((unsigned)a.n_units, (unsigned)(nib + k2_noc<EL, D, G>()));
  if (a.bulk_known) hipLaunchKernelGGL((k_finalize<EL, D, G>), g2, dim3(kT2 / 2), 0, s, a);
  else hipLaunchKernelGGL((k_finalize<EL, D, G, false, true>), g2, dim3(kT2 / 2), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.bulk_split) {
    if (a.block) {  // whole blocks: the position order, then the blocks' keys
      if ((e = launch_pos_rank(a, s)) != hipSuccess) return e;
      hipLaunchKernelGGL(k_block_keys, dim3((unsigned)a.n_units, (unsigned)nib), dim3(kT2), 0, s, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_bulk_mark, dim3((unsigned)a.n_units, (unsigned)((nib * kImpChunk + kMarkSlots - 1) / kMarkSlots)),
                       dim3(kT2), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((k_bulk_select<D * EL>), select_grid(a), dim3(kT2), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((k_bulk_moves<D * EL>), moves_grid<D * EL>(a), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

// Stage II in two launches (bf16, D = 128): the attention launch over K, the
// second launch (importance blocks and one output block per head), and the
// bulk cut's select and moves when some unit is cut in bulk.
template <int G>
static hipError_t step_go_s2(const StepArgs &a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  constexpr int EL = 2, D = 128;
  const int g = attend_grid<EL, D, G, true>(a.n_units);
  if (g <= 0) return hipErrorInvalidValue;
  hipError_t e;
  void (*kern)(StepArgs) = attend_kernel<EL, D, G, true>();
  if (ev0 && ev1) hipExtLaunchKernelGGL(kern, dim3(g), dim3(kThreads), 0, s, ev0, ev1, 0, a);
  else hipLaunchKernelGGL(kern, dim3(g), dim3(kThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  int nib = imp_blocks(a.cap);
  if (a.hp.n) {
    int mx = 1;
    for (int u = 0; u < a.hp.n; ++u) mx = max(mx, a.hp.L[u]);
    nib = min(nib, (mx + kImpChunk - 1) / kImpChunk);
  }
  // Four keys per thread in the output blocks when some unit is longer than
  // two (the new token included).
  int mxl = a.cap + 1;
  if (a.hp.n == a.n_units) {
    mxl = 1;
    for (int u = 0; u < a.hp.n; ++u) mxl = max(mxl, a.hp.L[u]);
  }
  if (mxl > 2 * kT2)
    hipLaunchKernelGGL((k_finalize<EL, D, G, true, false, 4>), dim3((unsigned)a.n_units, (unsigned)(nib + G)),
                       dim3(kT2), 0, s, a);
  else
    hipLaunchKernelGGL((k_finalize<EL, D, G, true>), dim3((unsigned)a.n_units, (unsigned)(nib + G)), dim3(kT2), 0, s,
                       a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.bulk_split) {
    hipLaunchKernelGGL(k_bulk_mark, dim3((unsigned)a.n_units, (unsigned)((nib * kImpChunk + kMarkSlots - 1) / kMarkSlots)),
                       dim3(kT2), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((k_bulk_select<D * EL>), select_grid(a), dim3(kT2), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((k_bulk_moves<D * EL>), moves_grid<D * EL>(a), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int EL, int D>
static hipError_t step_g(const StepArgs &a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  if constexpr (EL == 2 && D == 128) {
    if (a.s2_two) {
      switch (a.G) {
        case 1: return step_go_s2<1>(a, s, ev0, ev1);
        case 2: return step_go_s2<2>(a, s, ev0, ev1);
        case 4: return step_go_s2<4>(a, s, ev0, ev1);
        case 8: return step_go_s2<8>(a, s, ev0, ev1);
        default: return hipErrorInvalidValue;
      }
    }
  }
  switch (a.G) {
    case 1: return step_go<EL, D, 1>(a, s, ev0, ev1);
    case 2: return step_go<EL, D, 2>(a, s, ev0, ev1);
    case 4: return step_go<EL, D, 4>(a, s, ev0, ev1);
    case 8: return step_go<EL, D, 8>(a, s, ev0, ev1);
    default: return hipErrorInvalidValue;
  }
}

// Fill a.hp from a host copy of len[] exactly as the kernels would derive the
// plan from the device copy.  Returns false when no host plan applies.
template <int EL, int D, int G>
static bool host_plan_fill(StepArgs &a, const int32_t *len_hint) {
  const int U = a.n_units;
  if (U > kHostPlanUnits) return false;
  int g = 0;
  if constexpr (EL == 2 && D == 128) g = a.s2_two ? attend_grid<EL, D, G, true>(U) : attend_grid<EL, D, G>(U);
  else g = attend_grid<EL, D, G>(U);
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

hipError_t launch_step(const StepArgs &a, int dtype, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  if (dtype == HIKV_BF16) {
    if (a.D == 128) return step_g<2, 128>(a, s, ev0, ev1);
    if (a.D == 64) return step_g<2, 64>(a, s, ev0, ev1);
  } else {
    if (a.D == 128) return step_g<4, 128>(a, s, ev0, ev1);
    if (a.D == 64) return step_g<4, 64>(a, s, ev0, ev1);
  }
  return hipErrorInvalidValue;
}


}  // namespace hikv
