// prefill.hip -- prompt-side importance.
//
// "Kelle" summary, Sec. 4.1 (prefill): a token's importance is the sum over
// the prompt's queries of the attention it receives (a column sum of the
// causal attention matrix).  "HiKV", Sec. III-B / III-D: the localized score
// counts only the queries within B_I/2 steps of the token; a softmax row is
// still taken over everything the query sees.
//
// Two passes, deterministic (no float atomics):
//   P1  one workgroup per (unit, q-head, observation query): softmax max and
//       sum over the tokens the query sees (pos <= q_pos), log2 domain;
//   P2  one workgroup per (unit, 64-token tile): each token row sums, over
//       every (q-head, query) pair whose window admits it, exp2(s - m) / l,
//       and adds that to its importance once.
// This plain VALU form serves fp32 caches; bf16 caches take the matrix-core
// form below.

#include "hikv_block.h"
#include "hikv_launch.h"

namespace hikv {

template <int EL, int D>
__device__ __forceinline__ float row_logit(const char *krow, const char *qrow, int c) {
  constexpr int CH = 16 / EL, LPR = D / CH;
  const uint4 kf = *reinterpret_cast<const uint4 *>(krow + c * 16);
  const uint4 qf = *reinterpret_cast<const uint4 *>(qrow + c * 16);
  float d;
  if constexpr (EL == 2) {
    d = dot2_bf16(qf.x, kf.x, 0.f);
    d = dot2_bf16(qf.y, kf.y, d);
    d = dot2_bf16(qf.z, kf.z, d);
    d = dot2_bf16(qf.w, kf.w, d);
  } else {
    d = __uint_as_float(qf.x) * __uint_as_float(kf.x);
    d = fmaf(__uint_as_float(qf.y), __uint_as_float(kf.y), d);
    d = fmaf(__uint_as_float(qf.z), __uint_as_float(kf.z), d);
    d = fmaf(__uint_as_float(qf.w), __uint_as_float(kf.w), d);
  }
  return row_sum<LPR>(d);
}

template <int EL, int D>
__global__ __launch_bounds__(256) void k_prefill_stats(PrefillArgs p) {
  constexpr int CH = 16 / EL, LPR = D / CH, TPW = kWave / LPR, RB = D * EL;
  const int id = blockIdx.x;  // ((u * G) + g) * n_obs + i
  const int i = id % p.n_obs, ug = id / p.n_obs, g = ug % p.G, u = ug / p.G;
  const int b = u / p.Hkv, j = u - b * p.Hkv, h = j * p.G + g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane / LPR, c = lane - r * LPR;
  const int L = min(p.len[u], p.cap);
  const int qp = p.q_pos[(size_t)b * p.n_obs + i];
  const char *kc = static_cast<const char *>(p.k_cache) + (size_t)u * p.cap * RB;
  const int32_t *pos = p.pos + (size_t)u * p.cap;
  const char *qrow = static_cast<const char *>(p.q_obs) + (((size_t)(b * p.Hq + h)) * p.n_obs + i) * RB;
  float m = -INFINITY, l = 0.f;
  for (int n = wave * TPW + r; n < L; n += 4 * TPW) {
    const float s = row_logit<EL, D>(kc + (size_t)n * RB, qrow, c) * p.scale_log2;
    if (pos[n] > qp) continue;
    const float mx = fmaxf(m, s);
    l = l * fast_exp2(m - mx) + fast_exp2(s - mx);
    m = mx;
  }
  // Rows of a wave, then waves.
  for (int off = LPR; off < kWave; off <<= 1) {
    const float mo = __shfl_xor(m, off), lo = __shfl_xor(l, off);
    const float mx = fmaxf(m, mo);
    const float mxs = (mx == -INFINITY) ? 0.f : mx;
    l = l * fast_exp2(m - mxs) + lo * fast_exp2(mo - mxs);
    m = mx;
  }
  __shared__ float sm[4][2];
  if (lane == 0) {
    sm[wave][0] = m;
    sm[wave][1] = l;
  }
  __syncthreads();
  if (tid == 0) {
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm[w][0]);
    const float Ms = (M == -INFINITY) ? 0.f : M;
    float lv = 0.f;
    for (int w = 0; w < 4; ++w) lv += sm[w][1] * fast_exp2(sm[w][0] - Ms);
    p.stats[(size_t)id * 2] = M;
    p.stats[(size_t)id * 2 + 1] = lv;
  }
}

template <int EL, int D>
__global__ __launch_bounds__(256) void k_prefill_accum(PrefillArgs p) {
  constexpr int CH = 16 / EL, LPR = D / CH, TPW = kWave / LPR, RB = D * EL;
  constexpr int TILE = 64;
  const int u = blockIdx.y, tile = blockIdx.x;
  const int b = u / p.Hkv, j = u - b * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane / LPR, c = lane - r * LPR;
  const int L = min(p.len[u], p.cap);
  const int t0 = tile * TILE, t1 = min(t0 + TILE, L);
  if (t0 >= t1) return;
  const char *kc = static_cast<const char *>(p.k_cache) + (size_t)u * p.cap * RB;
  const int32_t *pos = p.pos + (size_t)u * p.cap;
  // All LPR lanes of a token row share n, so each row's reductions run with
  // the whole row active.
  for (int n = t0 + wave * TPW + r; n < t1; n += 4 * TPW) {
    const int pn = pos[n];
    float sum = 0.f;
    for (int g = 0; g < p.G; ++g) {
      const int h = j * p.G + g;
      for (int i = 0; i < p.n_obs; ++i) {
        const char *qrow = static_cast<const char *>(p.q_obs) + (((size_t)(b * p.Hq + h)) * p.n_obs + i) * RB;
        const float s = row_logit<EL, D>(kc + (size_t)n * RB, qrow, c) * p.scale_log2;
        const int qp = p.q_pos[(size_t)b * p.n_obs + i];
        const long long dist = (long long)qp - pn;
        if (dist < 0) continue;
        if (p.window > 0 && dist >= p.window) continue;
        const size_t sid = (((size_t)u * p.G + g) * p.n_obs + i) * 2;
        sum += fast_exp2(s - p.stats[sid]) / p.stats[sid + 1];
      }
    }
    if (c == 0) {
      if (p.pool > 1) p.padd[(size_t)u * p.cap + n] = sum;  // pooled below
      else p.imp[(size_t)u * p.cap + n] += sum;
    }
  }
}

// ---------------------------------------------------------------------------
// The same two passes on the matrix cores (bf16), for prompts of thousands of
// tokens: S = q.k tiles of 64 queries x 64 keys from v_mfma_f32_16x16x32_bf16
// with K rows as the A operand (16 keys) and q rows as the B operand (16
// queries), so a lane holds four keys of one query.  A lane feeds both
// operands the same eight of the 32 contracted elements (the sum over them
// does not depend on which eight).  Each wave keeps all four blocks of its
// stationary operand in registers, so one LDS read of the streaming operand
// feeds four products.
//   R   per 64-slot key tile of each unit, the lowest and highest position of
//       its live slots; per 64-query tile of each batch row, the lowest and
//       highest query position.  Tiles that cannot meet are skipped below.
//   S1  one workgroup per (64-query tile, unit, q-head): the queries stay in
//       registers, the unit's key tiles pass through LDS, wave w taking keys
//       16w..16w+15 of each; every lane keeps an online max and sum per
//       query block, merged over lanes and waves at the end.
//   S2  one workgroup per (64-slot key tile, unit): the keys stay in
//       registers, the query tiles of every q-head of the group pass through
//       LDS with their statistics, wave w taking queries 16w..16w+15 of
//       each; every lane sums its keys' probabilities over its queries, and
//       the sums meet over lanes and waves at the end and are added to the
//       tile's importance.  No float atomics: repeatable.
// ---------------------------------------------------------------------------
constexpr int kPT = 64;  // rows of a key or query tile

typedef __bf16 pbf16x8_t __attribute__((ext_vector_type(8)));
typedef float pf32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ pf32x4_t pmfma(pbf16x8_t a, pbf16x8_t b, pf32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(64) void k_prefill_ranges(PrefillArgs p) {
  const int t = blockIdx.x, y = blockIdx.y, lane = threadIdx.x;
  int lo = INT_MAX, hi = INT_MIN;
  if (y < p.n_units) {
    const int nkt = (p.cap + kPT - 1) / kPT;
    if (t >= nkt) return;
    const int L = min(p.len[y], p.cap);
    const int n = t * kPT + lane;
    if (n < L) lo = hi = p.pos[(size_t)y * p.cap + n];
  } else {
    const int b = y - p.n_units, nqt = (p.n_obs + kPT - 1) / kPT;
    if (t >= nqt) return;
    const int i = t * kPT + lane;
    if (i < p.n_obs) lo = hi = p.q_pos[(size_t)b * p.n_obs + i];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lo = min(lo, __shfl_xor(lo, off));
    hi = max(hi, __shfl_xor(hi, off));
  }
  if (lane == 0) {
    int32_t *r = y < p.n_units ? p.krange + ((size_t)y * ((p.cap + kPT - 1) / kPT) + t) * 2
                               : p.qrange + ((size_t)(y - p.n_units) * ((p.n_obs + kPT - 1) / kPT) + t) * 2;
    r[0] = lo;
    r[1] = hi;
  }
}

// A tile of 64 rows of D bf16 moves global memory -> registers (issued one
// tile ahead of its use) -> LDS rows of D * 2 + 16 bytes (the pad spreads
// the 16 rows an operand read touches over the banks).  Row r of the tile
// is global row row0 + r, clamped to last.
typedef unsigned int pu32x4_t __attribute__((ext_vector_type(4)));

template <int D>
struct TileShape {
  static constexpr int RB = D * 2, LRB = RB + 16, CPR = RB / 16, RPP = 256 / CPR, REPS = kPT / RPP;
};

template <int D>
__device__ __forceinline__ void tile_fetch(pu32x4_t (&v)[TileShape<D>::REPS], const char *src, int row0, int last,
                                           int tid) {
  using T = TileShape<D>;
#pragma unroll
  for (int rep = 0; rep < T::REPS; ++rep) {
    const int r = rep * T::RPP + tid / T::CPR, c = tid % T::CPR;
    v[rep] = *reinterpret_cast<const pu32x4_t *>(src + (size_t)min(row0 + r, last) * T::RB + c * 16);
  }
}

template <int D>
__device__ __forceinline__ void tile_put(const pu32x4_t (&v)[TileShape<D>::REPS], char *lds, int tid) {
  using T = TileShape<D>;
#pragma unroll
  for (int rep = 0; rep < T::REPS; ++rep) {
    const int r = rep * T::RPP + tid / T::CPR, c = tid % T::CPR;
    *reinterpret_cast<pu32x4_t *>(lds + r * T::LRB + c * 16) = v[rep];
  }
}

// Which tiles of a loop are worth visiting, as a bitmask in LDS (one bit per
// tile, at most kMaxTiles), built by the whole workgroup; next() finds the
// next set bit after t (or n when none is left).
constexpr int kMaxTiles = 32768;
struct TileMask {
  uint32_t *w;
  int n;
  __device__ __forceinline__ int next(int t) const {
    int i = t + 1;
    while (i < n) {
      const uint32_t m = w[i >> 5] >> (i & 31);
      if (m) return min(i + __builtin_ctz(m), n);
      i = (i | 31) + 1;
    }
    return n;
  }
};

template <int D>
__global__ __launch_bounds__(256) void k_prefill_stats_mfma(PrefillArgs p) {
  constexpr int RB = D * 2, LRB = RB + 16, KS = D / 32;
  const int nkt = (p.cap + kPT - 1) / kPT, nqt = (p.n_obs + kPT - 1) / kPT;
  // last query tiles first: in a causal prompt they see the most keys, so
  // the longest workgroups start first and the short ones fill the tail
  const int qt = nqt - 1 - (int)blockIdx.x, ug = blockIdx.y, g = ug % p.G, u = ug / p.G;
  const int b = u / p.Hkv, j = u - b * p.Hkv, h = j * p.G + g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, quad = lane >> 4, col = lane & 15;
  const int L = min(p.len[u], p.cap);
  const int ntile = (L + kPT - 1) / kPT;
  const int qmax = p.qrange[((size_t)b * nqt + qt) * 2 + 1];
  __shared__ uint32_t sMask[kMaxTiles / 32], sFull[kMaxTiles / 32];
  __shared__ __attribute__((aligned(16))) char sK[kPT * LRB];
  __shared__ int sP[kPT];
  __shared__ float sML[4][kPT][2];
  const int qmin = p.qrange[((size_t)b * nqt + qt) * 2];
  // key tiles with some key at or before the tile's last query; of those,
  // the complete ones wholly at or before its first query need no mask
  for (int w = tid; w < (ntile + 31) / 32; w += 256) sMask[w] = 0u, sFull[w] = 0u;
  __syncthreads();
  for (int t = tid; t < ntile; t += 256) {
    if (p.krange[((size_t)u * nkt + t) * 2] <= qmax) atomicOr(&sMask[t >> 5], 1u << (t & 31));
    if (p.krange[((size_t)u * nkt + t) * 2 + 1] <= qmin && (t + 1) * kPT <= L)
      atomicOr(&sFull[t >> 5], 1u << (t & 31));
  }
  const char *qbase = static_cast<const char *>(p.q_obs) + ((size_t)(b * p.Hq + h)) * p.n_obs * RB;
  pbf16x8_t qb[4][KS];  // B operands: the tile's four query blocks
  int qp[4];
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    const int ic = min(qt * kPT + blk * 16 + col, p.n_obs - 1);
    qp[blk] = p.q_pos[(size_t)b * p.n_obs + ic];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qb[blk][ks] = *reinterpret_cast<const pbf16x8_t *>(qbase + (size_t)ic * RB + ks * 64 + quad * 16);
  }
  const char *kc = static_cast<const char *>(p.k_cache) + (size_t)u * p.cap * RB;
  const int32_t *pos = p.pos + (size_t)u * p.cap;
  __syncthreads();
  const TileMask mask{sMask, ntile};
  float m[4], l[4];
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) m[blk] = -INFINITY, l[blk] = 0.f;
  pu32x4_t pre[TileShape<D>::REPS];
  int ppos = INT_MAX;
  int kt = mask.next(-1);
  {  // unconditional (a clamped tile when none is used), so that pre stays in registers
    const int kf = min(kt, ntile - 1);
    tile_fetch<D>(pre, kc, kf * kPT, L - 1, tid);
    if (tid < kPT && kf * kPT + tid < L) ppos = pos[kf * kPT + tid];
  }
  while (kt < ntile) {
    __syncthreads();  // the previous tile is no longer read
    tile_put<D>(pre, sK, tid);
    if (tid < kPT) sP[tid] = ppos;
    __syncthreads();
    const int kn = mask.next(kt);
    {  // the next tile's loads fly while this one is computed (after the
       // last one: the current tile again, unused)
      const int kf = kn < ntile ? kn : kt;
      tile_fetch<D>(pre, kc, kf * kPT, L - 1, tid);
      ppos = (tid < kPT && kf * kPT + tid < L) ? pos[kf * kPT + tid] : INT_MAX;
    }
    pf32x4_t S[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) S[blk] = (pf32x4_t){0.f, 0.f, 0.f, 0.f};
    const char *arow = sK + (wave * 16 + col) * LRB + quad * 16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const pbf16x8_t a = *reinterpret_cast<const pbf16x8_t *>(arow + ks * 64);
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) S[blk] = pmfma(a, qb[blk][ks], S[blk]);
    }
    if ((sFull[kt >> 5] >> (kt & 31)) & 1u) {  // every key visible to every query
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const float r = fmaxf(fmaxf(S[blk][0], S[blk][1]), fmaxf(S[blk][2], S[blk][3])) * p.scale_log2;
        const float mx = fmaxf(m[blk], r);
        float lv = l[blk] * fast_exp2(m[blk] - mx);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) lv += fast_exp2(fmaf(S[blk][ii], p.scale_log2, -mx));
        l[blk] = lv;
        m[blk] = mx;
      }
      kt = kn;
      continue;
    }
    int kp[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) kp[ii] = sP[wave * 16 + quad * 4 + ii];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      float sv[4], mx = m[blk];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        sv[ii] = kp[ii] <= qp[blk] ? S[blk][ii] * p.scale_log2 : -INFINITY;
        mx = fmaxf(mx, sv[ii]);
      }
      if (mx != -INFINITY) {
        float lv = l[blk] * fast_exp2(m[blk] - mx);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) lv += fast_exp2(sv[ii] - mx);
        l[blk] = lv;
        m[blk] = mx;
      }
    }
    kt = kn;
  }
  // merge the four lanes of a query (quads), then the four waves
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
#pragma unroll
    for (int off = 16; off < 64; off <<= 1) {
      const float mo = __shfl_xor(m[blk], off), lo = __shfl_xor(l[blk], off);
      const float mx = fmaxf(m[blk], mo);
      const float mxs = (mx == -INFINITY) ? 0.f : mx;
      l[blk] = l[blk] * fast_exp2(m[blk] - mxs) + lo * fast_exp2(mo - mxs);
      m[blk] = mx;
    }
    if (quad == 0) {
      sML[wave][blk * 16 + col][0] = m[blk];
      sML[wave][blk * 16 + col][1] = l[blk];
    }
  }
  __syncthreads();
  if (tid < kPT) {
    const int i = qt * kPT + tid;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sML[w][tid][0]);
    const float Ms = (M == -INFINITY) ? 0.f : M;
    float lv = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) lv += sML[w][tid][1] * fast_exp2(sML[w][tid][0] - Ms);
    if (i < p.n_obs) {
      const size_t sid = (((size_t)u * p.G + g) * p.n_obs + i) * 2;
      p.stats[sid] = M;
      p.stats[sid + 1] = lv;
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void k_prefill_accum_mfma(PrefillArgs p) {
  constexpr int RB = D * 2, LRB = RB + 16, KS = D / 32;
  const int kt = blockIdx.x, u = blockIdx.y;
  const int b = u / p.Hkv, j = u - b * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, quad = lane >> 4, col = lane & 15;
  const int L = min(p.len[u], p.cap);
  if (kt * kPT >= L) return;
  const int nkt = (p.cap + kPT - 1) / kPT, nqt = (p.n_obs + kPT - 1) / kPT;
  const int kmin = p.krange[((size_t)u * nkt + kt) * 2], kmax = p.krange[((size_t)u * nkt + kt) * 2 + 1];
  __shared__ uint32_t sMask[kMaxTiles / 32], sFull[kMaxTiles / 32];
  __shared__ __attribute__((aligned(16))) char sQ[kPT * LRB];
  __shared__ float sM[kPT];
  __shared__ int sQP[kPT];
  __shared__ float sC[4][kPT];
  // query tiles that can meet a key of this tile (causal, within the
  // window); of those, the ones that meet every key with every query
  for (int w = tid; w < (nqt + 31) / 32; w += 256) sMask[w] = 0u, sFull[w] = 0u;
  __syncthreads();
  for (int t = tid; t < nqt; t += 256) {
    const int qlo = p.qrange[((size_t)b * nqt + t) * 2], qhi = p.qrange[((size_t)b * nqt + t) * 2 + 1];
    const bool meet = (int64_t)qhi >= kmin && (p.window == 0 || (int64_t)qlo - kmax < p.window);
    const bool all = (int64_t)qlo >= kmax && (p.window == 0 || (int64_t)qhi - kmin < p.window);
    if (meet) atomicOr(&sMask[t >> 5], 1u << (t & 31));
    if (all) atomicOr(&sFull[t >> 5], 1u << (t & 31));
  }
  const char *kc = static_cast<const char *>(p.k_cache) + (size_t)u * p.cap * RB;
  const int32_t *pos = p.pos + (size_t)u * p.cap;
  pbf16x8_t ka[4][KS];  // A operands: the tile's four key blocks
  int kp[4][4];         // positions of this lane's output keys (INT_MAX: none)
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int kr = min(kt * kPT + kb * 16 + col, L - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      ka[kb][ks] = *reinterpret_cast<const pbf16x8_t *>(kc + (size_t)kr * RB + ks * 64 + quad * 16);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int n = kt * kPT + kb * 16 + quad * 4 + ii;
      kp[kb][ii] = n < L ? pos[n] : INT_MAX;
    }
  }
  __syncthreads();
  const TileMask mask{sMask, nqt};
  float cs[4][4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) cs[kb][ii] = 0.f;
  const char *qhead = static_cast<const char *>(p.q_obs) + ((size_t)(b * p.Hq + j * p.G)) * p.n_obs * RB;
  const size_t hstride = (size_t)p.n_obs * RB;  // q-heads of a group are adjacent
  pu32x4_t pre[TileShape<D>::REPS];
  float pm = 0.f, pl = 0.f;
  int pq = INT_MIN;
  auto fetch = [&](int g, int qt) {
    tile_fetch<D>(pre, qhead + (size_t)g * hstride, qt * kPT, p.n_obs - 1, tid);
    if (tid < kPT) {
      const int i = qt * kPT + tid;
      const bool ok = i < p.n_obs;
      const size_t sid = (((size_t)u * p.G + g) * p.n_obs + (ok ? i : 0)) * 2;
      pm = ok ? p.stats[sid] : 0.f;
      pl = ok ? p.stats[sid + 1] : 0.f;
      pq = ok ? p.q_pos[(size_t)b * p.n_obs + i] : INT_MIN;
    }
  };
  const int q0 = mask.next(-1);
  int g = 0, qt = q0;
  fetch(0, min(q0, nqt - 1));  // unconditional, so that pre stays in registers
  while (q0 < nqt && g < p.G) {
    __syncthreads();  // the previous tile is no longer read
    tile_put<D>(pre, sQ, tid);
    if (tid < kPT) {  // p = exp2(s - m - log2 l); a query that sees nothing gets none
      sM[tid] = pl > 0.f ? pm + __log2f(pl) : INFINITY;
      sQP[tid] = pq;
    }
    __syncthreads();
    int gn = g, qn = mask.next(qt);
    if (qn >= nqt) gn = g + 1, qn = q0;
    // the next tile's loads fly while this one is computed (after the last
    // one: the current tile again, unused)
    if (gn < p.G) fetch(gn, qn);
    else fetch(g, qt);
    pf32x4_t S[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) S[kb] = (pf32x4_t){0.f, 0.f, 0.f, 0.f};
    const char *brow = sQ + (wave * 16 + col) * LRB + quad * 16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const pbf16x8_t bq = *reinterpret_cast<const pbf16x8_t *>(brow + ks * 64);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) S[kb] = pmfma(ka[kb][ks], bq, S[kb]);
    }
    const int qi = wave * 16 + col;
    const float mq = sM[qi];
    if ((sFull[qt >> 5] >> (qt & 31)) & 1u) {  // every pair counts
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) cs[kb][ii] += fast_exp2(fmaf(S[kb][ii], p.scale_log2, -mq));
    } else {
      const int qp = sQP[qi];
      const uint32_t win = p.window > 0 ? (uint32_t)p.window : 0xffffffffu;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          // distance qp - kp without overflow: unsigned once kp <= qp
          const bool ok = kp[kb][ii] <= qp && (uint32_t)qp - (uint32_t)kp[kb][ii] < win;
          cs[kb][ii] += ok ? fast_exp2(fmaf(S[kb][ii], p.scale_log2, -mq)) : 0.f;
        }
    }
    g = gn, qt = qn;
  }
  // the 16 lanes of a quad hold the same keys for different queries; then
  // the four waves (different queries) meet in LDS
#pragma unroll
  for (int off = 1; off < 16; off <<= 1)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) cs[kb][ii] += __shfl_xor(cs[kb][ii], off);
  if (col == 0) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) sC[wave][kb * 16 + quad * 4 + ii] = cs[kb][ii];
  }
  __syncthreads();
  if (tid < kPT) {
    const int n = kt * kPT + tid;
    if (n < L) {
      const float sum = sC[0][tid] + sC[1][tid] + sC[2][tid] + sC[3][tid];
      if (p.pool > 1) p.padd[(size_t)u * p.cap + n] = sum;  // pooled below
      else p.imp[(size_t)u * p.cap + n] += sum;
    }
  }
}

// ---------------------------------------------------------------------------
// SnapKV's pooling ("KV Cache Compression and Dynamic Pruning in Production
// Serving", SnapKV section): a token at position p adds the largest of this
// call's scores over the live positions p .. p+pool-1.
//   P1  one workgroup per unit: the position order.  The live positions are
//       set as bits of an LDS bitmap over [min, max]; popcount prefixes per
//       group of 32 words are scanned; a slot's rank is its group prefix plus
//       the popcounts before it in the group.  Spans beyond the bitmap are
//       ranked by counting.  Writes order[rank] = slot and rank[slot].
//   P2  one thread per slot: walks forward in position order while the
//       positions stay below p + pool and adds the largest score.
// ---------------------------------------------------------------------------
constexpr int kPoolBits = 1 << 19;  // 64 KB of LDS

static hipError_t launch_prefill_scores(const PrefillArgs &p, int dtype, hipStream_t s);

__global__ __launch_bounds__(256) void k_pool_rank(PrefillArgs p) {
  const int u = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = min(p.len[u], p.cap);
  if (L <= 0) return;
  const int32_t *pos = p.pos + (size_t)u * p.cap;
  int32_t *ord = p.pord + (size_t)u * p.cap, *rk = p.prank + (size_t)u * p.cap;
  __shared__ uint32_t bits[kPoolBits / 32];
  __shared__ int gpre[kPoolBits / 1024];
  __shared__ int s_lo[4], s_hi[4], s_ws[4];
  int lo = INT_MAX, hi = INT_MIN;
  for (int n = tid; n < L; n += 256) lo = min(lo, pos[n]), hi = max(hi, pos[n]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lo = min(lo, __shfl_xor(lo, off)), hi = max(hi, __shfl_xor(hi, off));
  if (lane == 0) s_lo[wave] = lo, s_hi[wave] = hi;
  __syncthreads();
  lo = min(min(s_lo[0], s_lo[1]), min(s_lo[2], s_lo[3]));
  hi = max(max(s_hi[0], s_hi[1]), max(s_hi[2], s_hi[3]));
  if ((int64_t)hi - lo + 1 > kPoolBits) {  // counting, positions staged through LDS
    int *sp = reinterpret_cast<int *>(bits);
    constexpr int kTile = kPoolBits / 32;
    for (int nb = 0; nb < L; nb += 256) {
      const int n = nb + tid;
      const int pn = pos[min(n, L - 1)];
      int r = 0;
      for (int t0 = 0; t0 < L; t0 += kTile) {
        const int tn = min(kTile, L - t0);
        __syncthreads();
        for (int i = tid; i < tn; i += 256) sp[i] = pos[t0 + i];
        __syncthreads();
        for (int i = 0; i < tn; ++i) r += sp[i] < pn;
      }
      if (n < L) {
        r = min(r, L - 1);
        ord[r] = n;
        rk[n] = r;
      }
    }
    return;
  }
  const int nw = (int)(((int64_t)hi - lo + 32) / 32), ng = (nw + 31) / 32;
  for (int w = tid; w < nw; w += 256) bits[w] = 0u;
  __syncthreads();
  for (int n = tid; n < L; n += 256) {
    const int d = pos[n] - lo;
    atomicOr(&bits[d >> 5], 1u << (d & 31));
  }
  __syncthreads();
  // groups of 32 words: ng <= 512, two per thread, then a block scan
  int c0 = 0, c1 = 0;
  for (int k = 0; k < 32; ++k) {
    const int w0 = (2 * tid) * 32 + k, w1 = (2 * tid + 1) * 32 + k;
    if (w0 < nw) c0 += __popc(bits[w0]);
    if (w1 < nw) c1 += __popc(bits[w1]);
  }
  const int ts = c0 + c1;
  int incl = ts;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_ws[wave] = incl;
  __syncthreads();
  int base = incl - ts;
  for (int w = 0; w < wave; ++w) base += s_ws[w];
  if (2 * tid < ng) gpre[2 * tid] = base;
  if (2 * tid + 1 < ng) gpre[2 * tid + 1] = base + c0;
  __syncthreads();
  for (int n = tid; n < L; n += 256) {
    const int d = pos[n] - lo, w = d >> 5;
    int r = gpre[w >> 5];
    for (int k = w & ~31; k < w; ++k) r += __popc(bits[k]);
    r = min(r + __popc(bits[w] & ((1u << (d & 31)) - 1u)), L - 1);
    ord[r] = n;
    rk[n] = r;
  }
}

__global__ __launch_bounds__(256) void k_pool_apply(PrefillArgs p) {
  const int u = blockIdx.y, n = blockIdx.x * 256 + threadIdx.x;
  const int L = min(p.len[u], p.cap);
  if (n >= L) return;
  const size_t o = (size_t)u * p.cap;
  const int r = min(max(p.prank[o + n], 0), L - 1);
  const int64_t p0 = p.pos[o + n];
  float best = p.padd[o + n];
  for (int m = r + 1; m < L && m - r < p.pool; ++m) {
    const int sl = min(max(p.pord[o + m], 0), L - 1);
    if ((int64_t)p.pos[o + sl] - p0 >= p.pool) break;
    best = fmaxf(best, p.padd[o + sl]);
  }
  p.imp[o + n] += best;
}

hipError_t launch_prefill(const PrefillArgs &p, int dtype, hipStream_t s) {
  hipError_t e = launch_prefill_scores(p, dtype, s);
  if (e != hipSuccess || p.pool <= 1) return e;
  hipLaunchKernelGGL(k_pool_rank, dim3(p.n_units), dim3(256), 0, s, p);
  hipLaunchKernelGGL(k_pool_apply, dim3((p.cap + 255) / 256, p.n_units), dim3(256), 0, s, p);
  return hipGetLastError();
}

static hipError_t launch_prefill_scores(const PrefillArgs &p, int dtype, hipStream_t s) {
  const dim3 blk(256);
  if (dtype == HIKV_BF16) {  // matrix cores
    const int nkt = (p.cap + kPT - 1) / kPT, nqt = (p.n_obs + kPT - 1) / kPT;
    hipLaunchKernelGGL(k_prefill_ranges, dim3(max(nkt, nqt), p.n_units + p.B), dim3(64), 0, s, p);
    if (p.D == 128) {
      hipLaunchKernelGGL((k_prefill_stats_mfma<128>), dim3(nqt, p.n_units * p.G), blk, 0, s, p);
      hipLaunchKernelGGL((k_prefill_accum_mfma<128>), dim3(nkt, p.n_units), blk, 0, s, p);
    } else {
      hipLaunchKernelGGL((k_prefill_stats_mfma<64>), dim3(nqt, p.n_units * p.G), blk, 0, s, p);
      hipLaunchKernelGGL((k_prefill_accum_mfma<64>), dim3(nkt, p.n_units), blk, 0, s, p);
    }
    return hipGetLastError();
  }
  const dim3 g1(p.n_units * p.G * p.n_obs);
  const dim3 g2((p.cap + 63) / 64, p.n_units);
  if (p.D == 128) {
    hipLaunchKernelGGL((k_prefill_stats<4, 128>), g1, blk, 0, s, p);
    hipLaunchKernelGGL((k_prefill_accum<4, 128>), g2, blk, 0, s, p);
  } else {
    hipLaunchKernelGGL((k_prefill_stats<4, 64>), g1, blk, 0, s, p);
    hipLaunchKernelGGL((k_prefill_accum<4, 64>), g2, blk, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace hikv
