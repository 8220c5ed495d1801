// stage2.hip -- HiKV-style Stage II: reduced-channel logits and an exact
// softmax over the best tokens.
//
// "HiKV: Hierarchical Importance-Aware KV Cache", Sec. III-C and Algorithm 1:
// the B_II = d_h / r_II channels of the query with the largest magnitude
// select which K elements are loaded for QK^T.  Here, per q-head:
//   E    = the r channels of largest |q_d| (ties: lower channel)    [kernel S1]
//   s~   = scale * sum_{d in E} q_d k_d over every live token        [attention
//          kernel with the query masked to E, K-only]
//   p~   = softmax(s~) feeds the importance (accumulation kernel)
//   T    = the k_T tokens of largest s~ (ties: lower position)       [kernel S2]
//   out  = exact full-D softmax over T only, times V                 [kernel S3]
// That is the V side with HIKV_S2V_TOPK.  HIKV_S2V_CHUNK is the page's own V
// side: rows selected per chunk of P, with no renormalisation (kernel k_chunk_pv).

#include "hikv_block.h"
#include "hikv_launch.h"
#include "hikv_stats.h"

namespace hikv {

__device__ __forceinline__ float load_abs(const void *q, size_t idx, int el) {
  if (el == 2) {
    const uint32_t w = (uint32_t) static_cast<const uint16_t *>(q)[idx] << 16;
    return fabsf(__uint_as_float(w));
  }
  return fabsf(static_cast<const float *>(q)[idx]);
}

__device__ __forceinline__ bool unit_has_tiles(const StepArgs &a, int u) {
  const int U = a.n_units;
  const int nt = ((u + 1 < U) ? a.ws.plan[u + 1] : a.ws.plan[U]) - a.ws.plan[u];
  return nt > 0;
}

// S1: one wave per (b, q-head): the r channels of largest |q| (ties: lower
// channel).  Lane l holds channels l and l + 64.  |q| as its IEEE bits orders
// like the value (non-negative floats); the r-th largest bit pattern is found
// one bit at a time from the top (count of lanes at or above a trial
// threshold by ballot), then the channels above it are taken, and of those
// equal to it the lowest-numbered ones that complete r.
__global__ __launch_bounds__(64) void k_stage2_channels(StepArgs a, int el) {
  const int bh = blockIdx.x, lane = threadIdx.x;
  const int D = a.D;
  // This path evicts in place: the first q-head of each KV group resolves an
  // eviction a two-launch step left pending on the unit, before any launch
  // that reads the cache.
  {
    const int b = bh / a.Hq, h = bh - b * a.Hq;
    if (h % a.G == 0) settle_unit(a, b * a.Hkv + h / a.G, D * el);
  }
  const uint32_t v0 = __float_as_uint(load_abs(a.q, (size_t)bh * D + lane, el));
  const uint32_t v1 = D > 64 ? __float_as_uint(load_abs(a.q, (size_t)bh * D + 64 + lane, el)) : 0u;
  const bool has1 = D > 64;
  auto count_ge = [&](uint32_t t) {
    return __popcll(__ballot(v0 >= t)) + (has1 ? __popcll(__ballot(v1 >= t)) : 0);
  };
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    if (count_ge(cand) >= a.r) thr = cand;
  }
  const uint64_t gt0 = __ballot(v0 > thr), gt1 = has1 ? __ballot(v1 > thr) : 0ull;
  const uint64_t eq0 = __ballot(v0 == thr), eq1 = has1 ? __ballot(v1 == thr) : 0ull;
  const int need = a.r - __popcll(gt0) - __popcll(gt1);  // equal channels still to take
  const uint64_t below = (1ull << lane) - 1ull;
  bool sel[2];
  sel[0] = v0 > thr || (v0 == thr && __popcll(eq0 & below) < need);
  sel[1] = has1 && (v1 > thr || (v1 == thr && __popcll(eq0) + __popcll(eq1 & below) < need));
  const uint64_t b0 = __ballot(sel[0]);
  const uint64_t b1 = __ballot(sel[1]);
  if (lane == 0) {
    uint32_t *mw = a.ws.chmask + (size_t)bh * (D / 32);
    mw[0] = (uint32_t)b0;
    mw[1] = (uint32_t)(b0 >> 32);
    if (D > 64) {
      mw[2] = (uint32_t)b1;
      mw[3] = (uint32_t)(b1 >> 32);
    }
  }
  if (a.dbg_channels) {
    const int n0 = __popcll(b0);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int d = lane + 64 * t;
      if (d < D && sel[t]) {
        const uint64_t below = (lane == 0) ? 0ull : ((t == 0 ? b0 : b1) & ((1ull << lane) - 1ull));
        const int idx = (t == 0 ? 0 : n0) + __popcll(below);
        a.dbg_channels[(size_t)bh * a.r + idx] = d;
      }
    }
  }
}

// S2: per (b, q-head), the k_T live tokens with the largest reduced logit
// (ties: lower position), gathered in slot order.
constexpr int kSelThreads = 256;

__device__ __forceinline__ void stage2_tokens(const StepArgs &a) {
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int b = bh / a.Hq, h = bh - b * a.Hq, j = h / a.G, g = h - j * a.G;
  const int u = b * a.Hkv + j;
  int32_t *tsel = a.ws.tsel + (size_t)bh * a.kT;
  if (!unit_has_tiles(a, u)) {
    if (tid == 0) a.ws.tcount[bh] = 0;
    if (a.dbg_count && tid == 0) a.dbg_count[bh] = 0;
    if (a.dbg_tokens)
      for (int i = tid; i < a.kT; i += kSelThreads) a.dbg_tokens[(size_t)bh * a.kT + i] = -1;
    return;
  }
  const int L = a.len[u] + 1;
  const int k = min(a.kT, L);
  const float *lg = a.ws.logits + (size_t)u * a.cap * a.G;
  const int32_t *pos = a.pos + (size_t)u * a.cap;
  __shared__ uint32_t hist[256];
  __shared__ int sc[kSelThreads];
  __shared__ RadixState rs;
  // Smaller key = better token: larger logit, then lower position.
  auto key_of = [&](int n, uint64_t &key) -> bool {
    key = ((uint64_t)(~ord_f32(lg[(size_t)n * a.G + g])) << 32) | (uint32_t)pos[n];
    return true;
  };
  radix_select_smallest<kSelThreads>(L, k, key_of, hist, &rs);
  const uint64_t prefix = rs.prefix;
  const int shift = rs.shift;
  const int per = (L + kSelThreads - 1) / kSelThreads;
  const int n0 = min(tid * per, L), n1 = min(n0 + per, L);
  int cnt = 0;
  for (int n = n0; n < n1; ++n) {
    uint64_t key;
    key_of(n, key);
    cnt += (key >> shift) <= (prefix >> shift);
  }
  int total;
  int o = block_excl_scan<kSelThreads>(cnt, sc, &total);
  for (int n = n0; n < n1; ++n) {
    uint64_t key;
    key_of(n, key);
    if ((key >> shift) <= (prefix >> shift)) {
      if (o < a.kT) tsel[o] = n;  // exactly k with distinct positions; bound anyway
      ++o;
    }
  }
  if (total > a.kT) total = a.kT;
  if (tid == 0) a.ws.tcount[bh] = total;
  __syncthreads();
  if (a.dbg_count && tid == 0) a.dbg_count[bh] = total;
  if (a.dbg_tokens) {
    int32_t *dt = a.dbg_tokens + (size_t)bh * a.kT;
    for (int i = tid; i < a.kT; i += kSelThreads) {
      if (i >= total) {
        dt[i] = -1;
        continue;
      }
      const int p = pos[tsel[i]];
      int rank = 0;
      for (int e = 0; e < total; ++e) rank += pos[tsel[e]] < p;
      if (rank < a.kT) dt[rank] = p;
    }
  }
}

// S3: per (b, q-head), exact logits over the selected tokens, softmax over
// them only, P.V.  Same lane layout as the attention kernel: LPR lanes per
// row, one online softmax per row, rows and waves merged at the end.
template <int EL, int D>
__device__ __forceinline__ void stage2_exact(const StepArgs &a) {
  constexpr int CH = 16 / EL, LPR = D / CH, TPW = kWave / LPR;
  constexpr int U = (16 / TPW) > 0 ? 16 / TPW : 1;
  constexpr int RB = D * EL;
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = bh / a.Hq, h = bh - b * a.Hq, j = h / a.G;
  const int u = b * a.Hkv + j;
  const int r = lane / LPR, c = lane - r * LPR;
  float *outp = a.out + (size_t)bh * D;
  const int nt = a.ws.tcount[bh];
  if (nt == 0) {
    for (int d = tid; d < D; d += 256) outp[d] = 0.f;
    return;
  }
  const int32_t *tsel = a.ws.tsel + (size_t)bh * a.kT;
  const char *kc = static_cast<const char *>(a.k_cache) + (size_t)u * a.cap * RB;
  const char *vc = static_cast<const char *>(a.v_cache) + (size_t)u * a.cap * RB;
  const uint4 qf = *reinterpret_cast<const uint4 *>(static_cast<const char *>(a.q) +
                                                    ((size_t)bh * D + c * CH) * EL);
  float m = -INFINITY, l = 0.f, acc[CH];
#pragma unroll
  for (int e = 0; e < CH; ++e) acc[e] = 0.f;
  // The selected slots go to LDS a chunk at a time, so that the K/V row loads
  // do not wait for an index load; the row loads run one step ahead of the
  // arithmetic (two register buffers).
  constexpr int CHK = 1024, STEP = 4 * TPW * U;
  __shared__ int s_n[CHK];
  auto load_rows = [&](int cn, int base, uint4 (&kf)[U], uint4 (&vf)[U]) {
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int t = base + i * TPW + r;
      const bool ok = t < cn;
      const int n = ok ? s_n[t] : 0;
      kf[i] = ok ? *reinterpret_cast<const uint4 *>(kc + (size_t)n * RB + c * 16) : make_uint4(0, 0, 0, 0);
      vf[i] = ok ? *reinterpret_cast<const uint4 *>(vc + (size_t)n * RB + c * 16) : make_uint4(0, 0, 0, 0);
    }
  };
  auto consume = [&](int cn, int base, const uint4 (&kf)[U], const uint4 (&vf)[U]) {
    float s[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      float d;
      if constexpr (EL == 2) {
        d = dot2_bf16(qf.x, kf[i].x, 0.f);
        d = dot2_bf16(qf.y, kf[i].y, d);
        d = dot2_bf16(qf.z, kf[i].z, d);
        d = dot2_bf16(qf.w, kf[i].w, d);
      } else {
        d = __uint_as_float(qf.x) * __uint_as_float(kf[i].x);
        d = fmaf(__uint_as_float(qf.y), __uint_as_float(kf[i].y), d);
        d = fmaf(__uint_as_float(qf.z), __uint_as_float(kf[i].z), d);
        d = fmaf(__uint_as_float(qf.w), __uint_as_float(kf[i].w), d);
      }
      d = row_sum<LPR>(d) * a.scale_log2;
      s[i] = (base + i * TPW + r < cn) ? d : -INFINITY;
    }
    float mx = m;
#pragma unroll
    for (int i = 0; i < U; ++i) mx = fmaxf(mx, s[i]);
    const float mxs = (mx == -INFINITY) ? 0.f : mx;
    const float corr = fast_exp2(m - mxs);
    l *= corr;
#pragma unroll
    for (int e = 0; e < CH; ++e) acc[e] *= corr;
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const float p = fast_exp2(s[i] - mxs);
      l += p;
      if constexpr (EL == 2) {
        const uint32_t *vw = reinterpret_cast<const uint32_t *>(&vf[i]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] = fmaf(p, bf_lo(vw[e]), acc[2 * e]);
          acc[2 * e + 1] = fmaf(p, bf_hi(vw[e]), acc[2 * e + 1]);
        }
      } else {
        const float *vv = reinterpret_cast<const float *>(&vf[i]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(p, vv[e], acc[e]);
      }
    }
    m = mx;
  };
  for (int cb = 0; cb < nt; cb += CHK) {
    const int cn = min(CHK, nt - cb);
    __syncthreads();  // the previous chunk's indices are no longer read
    for (int i = tid; i < cn; i += 256) s_n[i] = tsel[cb + i];
    __syncthreads();
    uint4 ka[U], va[U], kb[U], vb[U];
    int base = wave * TPW * U;
    load_rows(cn, base, ka, va);
    for (; base < cn; base += 2 * STEP) {
      load_rows(cn, base + STEP, kb, vb);
      consume(cn, base, ka, va);
      if (base + STEP >= cn) break;
      load_rows(cn, base + 2 * STEP, ka, va);
      consume(cn, base + STEP, kb, vb);
    }
  }
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
    const float mo = __shfl_xor(m, off), lo = __shfl_xor(l, off);
    const float mx = fmaxf(m, mo);
    const float mxs = (mx == -INFINITY) ? 0.f : mx;
    const float ea = fast_exp2(m - mxs), eb = fast_exp2(mo - mxs);
    l = l * ea + lo * eb;
#pragma unroll
    for (int e = 0; e < CH; ++e) acc[e] = acc[e] * ea + __shfl_xor(acc[e], off) * eb;
    m = mx;
  }
  __shared__ float sm_ml[4][2];
  __shared__ float sm_acc[4][D];
  if (r == 0) {
#pragma unroll
    for (int e = 0; e < CH; ++e) sm_acc[wave][c * CH + e] = acc[e];
    if (c == 0) {
      sm_ml[wave][0] = m;
      sm_ml[wave][1] = l;
    }
  }
  __syncthreads();
  for (int d = tid; d < D; d += 256) {
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_ml[w][0]);
    const float Ms = (M == -INFINITY) ? 0.f : M;
    float av = 0.f, lv = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float e = fast_exp2(sm_ml[w][0] - Ms);
      av += sm_acc[w][d] * e;
      lv += sm_ml[w][1] * e;
    }
    outp[d] = av / lv;
  }
}

// ---------------------------------------------------------------------------
// Stage II V side as HiKV states it (Sec. III-C, Algorithm 1): the reduced-
// logit probabilities P over the live tokens, taken in position order, are
// cut into chunks of D tokens; each chunk keeps its r largest entries (ties:
// lower position), and the output sums those entries times their V rows with
// no renormalisation.
//
// Two launches:
//  k_pos_rank, one workgroup per unit: the position order.  Positions are
//  distinct, so a token's rank is the number of live positions below its
//  own: the positions are set as bits of an LDS bitmap over a window of
//  kRankBits positions, the per-word popcounts are scanned, and rank =
//  tokens in earlier windows + prefix of its word + popcount of the word's
//  lower bits; the slot is written at its rank.  A span of positions wider
//  than one window takes one pass over the unit's positions per window, so
//  the cost is len * ceil(span / kRankBits) (one pass for spans up to 262144
//  positions).  With repeated positions ranks collide: results are then
//  undefined, and every slot read back is clamped, so memory stays in bounds.
//  k_chunk_pv, one workgroup per (chunk, unit):
//  1. the chunk's D slots are read from the order, with their logits;
//  2. wave w selects for q-heads w, w + 4: lane l holds the chunk's entries l
//     and l + 64; the r-th largest probability is found one bit at a time by
//     ballot counts (the IEEE bits of a non-negative float order like its
//     value), and of the entries equal to it the lowest-ranked complete r.
//  3. the rows any q-head kept are read once, 16 bytes per lane, and each
//     lane sums p * v for every q-head.
//  4. the partials go out; the accumulation launch that follows adds each
//     unit's chunks up in chunk order (results repeat bit for bit).
// ---------------------------------------------------------------------------
constexpr int kRankBits = 1 << 18;  // positions one bitmap window covers (32 KB)
constexpr int kRankThreads = 1024;

__global__ __launch_bounds__(kRankThreads) void k_pos_rank(StepArgs a) {
  constexpr int NW = kRankBits / 32, WPT = NW / kRankThreads, KR = 8, NWV = kRankThreads / kWave;
  __shared__ uint32_t bits[NW];
  __shared__ int wpre[NW];
  __shared__ int s_lo[NWV], s_hi[NWV], s_wsum[NWV];
  const int u = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Block-granular eviction orders only the units its second launch marked
  // as cut this step, over the slots the cut considers; the chunked V side
  // orders every unit with tiles, over its L slots (the new token sits in
  // slot L - 1).
  int L;
  if (a.block) {
    const int4 bs = reinterpret_cast<const int4 *>(a.ws.bsel)[u];
    if (bs.w != 1) return;
    L = bs.z;
  } else {
    if (!unit_has_tiles(a, u)) return;
    L = a.len[u] + 1;
  }
  const int32_t *pos = a.pos + (size_t)u * a.cap;
  int32_t *order = a.ws.order + (size_t)u * a.cap;
  // The first KR * kRankThreads positions stay in registers.
  int ps[KR];
  int lo = INT_MAX, hi = INT_MIN;
#pragma unroll
  for (int i = 0; i < KR; ++i) {
    const int n = tid + kRankThreads * i;
    ps[i] = pos[min(n, L - 1)];
    if (n < L) lo = min(lo, ps[i]), hi = max(hi, ps[i]);
  }
  for (int n = tid + kRankThreads * KR; n < L; n += kRankThreads) {
    const int p = pos[n];
    lo = min(lo, p), hi = max(hi, p);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lo = min(lo, __shfl_xor(lo, off));
    hi = max(hi, __shfl_xor(hi, off));
  }
  if (lane == 0) s_lo[wave] = lo, s_hi[wave] = hi;
  __syncthreads();
  lo = s_lo[0], hi = s_hi[0];
  for (int w = 1; w < NWV; ++w) lo = min(lo, s_lo[w]), hi = max(hi, s_hi[w]);
  int done = 0;  // tokens in the windows before this one
  for (int64_t w0 = lo; w0 <= (int64_t)hi; w0 += kRankBits) {
    const int64_t nw64 = ((int64_t)hi - w0 + 32) / 32;
    const int nw = (int)(nw64 < NW ? nw64 : NW);
    for (int w = tid; w < nw; w += kRankThreads) bits[w] = 0u;
    __syncthreads();
    auto in_win = [&](int p) { return (int64_t)p >= w0 && (int64_t)p < w0 + kRankBits; };
#pragma unroll
    for (int i = 0; i < KR; ++i)
      if (tid + kRankThreads * i < L && in_win(ps[i])) {
        const int d = (int)(ps[i] - w0);
        atomicOr(&bits[d >> 5], 1u << (d & 31));
      }
    for (int n = tid + kRankThreads * KR; n < L; n += kRankThreads) {
      const int p = pos[n];
      if (in_win(p)) {
        const int d = (int)(p - w0);
        atomicOr(&bits[d >> 5], 1u << (d & 31));
      }
    }
    __syncthreads();
    // exclusive prefix of the popcounts per word: WPT words per thread, a
    // wave scan of the thread sums, then the waves
    int cnt[WPT], ts = 0;
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      const int w = tid * WPT + k;
      cnt[k] = w < nw ? __popc(bits[w]) : 0;
      ts += cnt[k];
    }
    int incl = ts;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int base = done + incl - ts, total = 0;
    for (int w = 0; w < NWV; ++w) {
      if (w < wave) base += s_wsum[w];
      total += s_wsum[w];
    }
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      const int w = tid * WPT + k;
      if (w < nw) wpre[w] = base;
      base += cnt[k];
    }
    __syncthreads();
    auto rank_of = [&](int p) -> int {  // clamped: repeated positions stay in bounds
      const int d = (int)(p - w0);
      const int rk = wpre[d >> 5] + __popc(bits[d >> 5] & ((1u << (d & 31)) - 1u));
      return rk < L - 1 ? rk : L - 1;
    };
#pragma unroll
    for (int i = 0; i < KR; ++i) {
      const int n = tid + kRankThreads * i;
      if (n < L && in_win(ps[i])) order[rank_of(ps[i])] = n;
    }
    for (int n = tid + kRankThreads * KR; n < L; n += kRankThreads) {
      const int p = pos[n];
      if (in_win(p)) order[rank_of(p)] = n;
    }
    done += total;
    __syncthreads();  // the bitmap is rebuilt for the next window
  }
}

template <int EL, int D, int G>
__global__ __launch_bounds__(256) void k_chunk_pv(StepArgs a) {
  constexpr int CH = 16 / EL;      // V elements per 16-byte load
  constexpr int LPR = D / CH;      // lanes per V row
  constexpr int RG = 256 / LPR;    // rows read at once by the workgroup
  constexpr int MAXIT = D / RG;    // rows per lane group, at most
  constexpr int RB = D * EL;
  constexpr int NPL = D / 64;      // chunk entries per lane in the selection
  const int c = blockIdx.x, u = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = u / a.Hkv, j = u - b * a.Hkv;
  float *outp = a.out + ((size_t)b * a.Hq + (size_t)j * G) * D;  // the group's rows are adjacent
  if (!unit_has_tiles(a, u)) {  // a unit the step skipped (an error): zero output
    if (c == 0) {
      for (int i = tid; i < G * D; i += 256) outp[i] = 0.f;
      if (a.dbg_count && tid < G) a.dbg_count[(size_t)b * a.Hq + (size_t)j * G + tid] = 0;
    }
    return;
  }
  const int L = a.len[u] + 1;  // the new token sits in slot L - 1
  const int c0 = c * D;
  if (c0 >= L) return;
  const int m = min(D, L - c0);
  const int keep = min(a.r, m);
  const size_t NC = (size_t)((a.cap + D - 1) / D);
  __shared__ int s_slot[D];
  __shared__ float s_p[G][D];  // the chunk's logits, then the kept probabilities
  __shared__ int s_list[D];
  __shared__ int s_nlist;
  __shared__ float s_red[4][G * D];
  const float *lg = a.ws.logits + (size_t)u * a.cap * G;
  // The unit statistics of this wave's q-heads (w, w + 4), loaded now so
  // that they arrive with the positions.
  float Mw[2] = {0.f, 0.f}, ILw[2] = {0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int g = wave + 4 * k;
    if (g < G) {
      float Sg;
      unit_softmax_stats(a, u, g, Mw[k], Sg);
      ILw[k] = 1.f / Sg;
    }
  }

  // 1. The chunk's slots in position order, and their logits.
  const int32_t *order = a.ws.order + (size_t)u * a.cap + c0;
  for (int t = tid; t < m; t += 256) {
    const int n = min(max(order[t], 0), L - 1);
    s_slot[t] = n;
#pragma unroll
    for (int g = 0; g < G; ++g) s_p[g][t] = lg[(size_t)n * G + g];
  }
  __syncthreads();

  // 2. Selection.
  for (int g = wave; g < G; g += 4) {
    const float M = Mw[g >> 2], IL = ILw[g >> 2];
    float pv[NPL];
    uint32_t kv[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int t = lane + 64 * i;
      const bool ok = t < m;
      pv[i] = ok ? fast_exp2(s_p[g][t] - M) * IL : 0.f;
      kv[i] = ok ? __float_as_uint(pv[i]) + 1u : 0u;  // 0: no token of the chunk
    }
    auto count_ge = [&](uint32_t thr) {
      int k = 0;
#pragma unroll
      for (int i = 0; i < NPL; ++i) k += __popcll(__ballot(kv[i] >= thr));
      return k;
    };
    uint32_t thr = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = thr | (1u << bit);
      if (count_ge(cand) >= keep) thr = cand;
    }
    int need = keep;
#pragma unroll
    for (int i = 0; i < NPL; ++i) need -= __popcll(__ballot(kv[i] > thr));
    const uint64_t below = (1ull << lane) - 1ull;
    int eq_before = 0, kept = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const uint64_t eq = __ballot(kv[i] == thr);
      const bool sel = kv[i] > thr || (kv[i] == thr && eq_before + __popcll(eq & below) < need);
      eq_before += __popcll(eq);
      kept += __popcll(__ballot(sel));
      s_p[g][lane + 64 * i] = sel ? pv[i] : 0.f;
    }
    if (lane == 0) a.ws.chunk_cnt[((size_t)u * NC + c) * G + g] = kept;
  }
  __syncthreads();
  if (wave == 0) {  // the rows some q-head kept, in chunk order
    int nbase = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int t = lane + 64 * i;
      bool any = false;
#pragma unroll
      for (int g = 0; g < G; ++g) any |= s_p[g][t] > 0.f;
      const uint64_t bm = __ballot(any);
      if (any) s_list[nbase + __popcll(bm & ((1ull << lane) - 1ull))] = t;
      nbase += __popcll(bm);
    }
    if (lane == 0) s_nlist = nbase;
  }
  __syncthreads();

  // 3. P.V over the kept rows.
  const int nl = s_nlist;
  const int rg = tid / LPR, cl = tid - rg * LPR;
  const char *vc = static_cast<const char *>(a.v_cache) + (size_t)u * a.cap * RB;
  uint4 vf[MAXIT];
  int tt[MAXIT];
#pragma unroll
  for (int i = 0; i < MAXIT; ++i) {  // every row load first, from clamped addresses
    const int li = rg + i * RG;
    tt[i] = nl > 0 ? s_list[min(li, nl - 1)] : 0;
    const int sl = min(max(s_slot[tt[i]], 0), L - 1);
    vf[i] = *reinterpret_cast<const uint4 *>(vc + (size_t)sl * RB + cl * 16);
  }
  float acc[G][CH];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < CH; ++e) acc[g][e] = 0.f;
#pragma unroll
  for (int i = 0; i < MAXIT; ++i) {
    const bool live = rg + i * RG < nl;
    float vv[CH];
    if constexpr (EL == 2) {
      const uint32_t *w = reinterpret_cast<const uint32_t *>(&vf[i]);
#pragma unroll
      for (int e = 0; e < 4; ++e) vv[2 * e] = bf_lo(w[e]), vv[2 * e + 1] = bf_hi(w[e]);
    } else {
      const float *f = reinterpret_cast<const float *>(&vf[i]);
#pragma unroll
      for (int e = 0; e < 4; ++e) vv[e] = f[e];
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float p = live ? s_p[g][tt[i]] : 0.f;
#pragma unroll
      for (int e = 0; e < CH; ++e) acc[g][e] = fmaf(p, vv[e], acc[g][e]);
    }
  }
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1)
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < CH; ++e) acc[g][e] += __shfl_xor(acc[g][e], off);
  if (lane < LPR) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < CH; ++e) s_red[wave][g * D + cl * CH + e] = acc[g][e];
  }
  __syncthreads();

  // 4. Partials out; k_accumulate adds them up.
  float *dst = a.ws.chunk_acc + ((size_t)u * NC + c) * G * D;
  for (int i = tid; i < G * D; i += 256) dst[i] = s_red[0][i] + s_red[1][i] + s_red[2][i] + s_red[3][i];
}

template <int EL, int D>
static void chunk_pv_g(const StepArgs &a, dim3 grid, hipStream_t s) {
  switch (a.G) {
    case 1: hipLaunchKernelGGL((k_chunk_pv<EL, D, 1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_chunk_pv<EL, D, 2>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_chunk_pv<EL, D, 4>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((k_chunk_pv<EL, D, 8>), grid, dim3(256), 0, s, a); break;
  }
}

hipError_t launch_pos_rank(const StepArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_pos_rank, dim3((unsigned)a.n_units), dim3(kRankThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_chunk_pv(const StepArgs &a, int dtype, hipStream_t s) {
  hipLaunchKernelGGL(k_pos_rank, dim3((unsigned)a.n_units), dim3(kRankThreads), 0, s, a);
  const dim3 grid((a.cap + a.D - 1) / a.D, a.n_units);
  if (dtype == HIKV_BF16) {
    if (a.D == 128) chunk_pv_g<2, 128>(a, grid, s);
    else chunk_pv_g<2, 64>(a, grid, s);
  } else {
    if (a.D == 128) chunk_pv_g<4, 128>(a, grid, s);
    else chunk_pv_g<4, 64>(a, grid, s);
  }
  return hipGetLastError();
}

hipError_t launch_stage2_channels(const StepArgs &a, int dtype, hipStream_t s) {
  hipLaunchKernelGGL(k_stage2_channels, dim3(a.B * a.Hq), dim3(64), 0, s, a,
                     dtype == HIKV_BF16 ? 2 : 4);
  return hipGetLastError();
}


// S2 + S3 in one launch per (b, q-head): the selected slots go to global
// memory and are read back by the same workgroup after a barrier (all of
// its waves share one CU's cache, so the barrier's fences make them
// visible), which saves a launch and its drain.
template <int EL, int D>
__global__ __launch_bounds__(256) void k_stage2_select_exact(StepArgs a) {
  stage2_tokens(a);
  __syncthreads();
  stage2_exact<EL, D>(a);
}

hipError_t launch_stage2_exact(const StepArgs &a, int dtype, hipStream_t s) {
  const dim3 grid(a.B * a.Hq), block(256);
  if (dtype == HIKV_BF16) {
    if (a.D == 128) hipLaunchKernelGGL((k_stage2_select_exact<2, 128>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_stage2_select_exact<2, 64>), grid, block, 0, s, a);
  } else {
    if (a.D == 128) hipLaunchKernelGGL((k_stage2_select_exact<4, 128>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_stage2_select_exact<4, 64>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace hikv
