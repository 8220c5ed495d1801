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
    if (c == 0) p.imp[(size_t)u * p.cap + n] += sum;
  }
}

// ---------------------------------------------------------------------------
// The same two passes on the matrix cores (bf16), for prompts of thousands of
// tokens: S = q.k tiles of 64 queries x 64 keys from v_mfma_f32_16x16x16_bf16,
// with K rows as the A operand (16 keys) and q rows as the B operand (16
// queries), so a lane holds four keys of one query.
//   R   per 64-slot key tile of each unit, the lowest and highest position of
//       its live slots; per 64-query tile of each batch row, the lowest and
//       highest query position.  Tiles that cannot meet are skipped below.
//   S1  one workgroup per (64-query tile, unit, q-head): the queries stay in
//       registers, the unit's key tiles pass through LDS; each lane keeps an
//       online max and sum of its four keys per tile, merged at the end.
//   S2  one workgroup per (64-slot key tile, unit): the keys stay in
//       registers, the query tiles of every q-head of the group pass through
//       LDS with their statistics; each lane sums its four keys' probability
//       over its queries, the sums meet across lanes at the end, and the
//       tile adds them to its importance.  No float atomics: repeatable.
// ---------------------------------------------------------------------------
constexpr int kPT = 64;  // rows of a key or query tile

typedef __bf16 pbf16x4_t __attribute__((ext_vector_type(4)));
typedef float pf32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ pf32x4_t pmfma(pbf16x4_t a, pbf16x4_t b, pf32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
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

// 64 rows of D bf16 from global memory (row r of the tile -> global row
// row0 + r, clamped to last) into LDS rows of D * 2 + 16 bytes (the pad
// keeps the 16 rows an MFMA operand read touches in distinct banks).
template <int D>
__device__ __forceinline__ void stage_rows(char *lds, const char *src, size_t stride, int row0, int last,
                                           int tid) {
  constexpr int RB = D * 2, LRB = RB + 16, CPR = RB / 16, RPP = 256 / CPR;
#pragma unroll
  for (int rep = 0; rep < kPT / RPP; ++rep) {
    const int r = rep * RPP + tid / CPR, c = tid % CPR;
    const int gr = min(row0 + r, last);
    const uint4 v = *reinterpret_cast<const uint4 *>(src + (size_t)gr * stride + c * 16);
    *reinterpret_cast<uint4 *>(lds + r * LRB + c * 16) = v;
  }
}

template <int D>
__global__ __launch_bounds__(256) void k_prefill_stats_mfma(PrefillArgs p) {
  constexpr int RB = D * 2, LRB = RB + 16, KS = D / 16;
  const int qt = blockIdx.x, ug = blockIdx.y, g = ug % p.G, u = ug / p.G;
  const int b = u / p.Hkv, j = u - b * p.Hkv, h = j * p.G + g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, quad = lane >> 4, col = lane & 15;
  const int L = min(p.len[u], p.cap);
  const int nkt = (p.cap + kPT - 1) / kPT, nqt = (p.n_obs + kPT - 1) / kPT;
  const int i = qt * kPT + wave * 16 + col;  // this lane's query
  const int ic = min(i, p.n_obs - 1);
  const int qp = p.q_pos[(size_t)b * p.n_obs + ic];
  const char *qrow = static_cast<const char *>(p.q_obs) + (((size_t)(b * p.Hq + h)) * p.n_obs + ic) * RB;
  pbf16x4_t qb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qb[ks] = *reinterpret_cast<const pbf16x4_t *>(qrow + ks * 32 + quad * 8);
  const int qmax = p.qrange[((size_t)b * nqt + qt) * 2 + 1];
  __shared__ __attribute__((aligned(16))) char sK[kPT * LRB];
  __shared__ int sP[kPT];
  const char *kc = static_cast<const char *>(p.k_cache) + (size_t)u * p.cap * RB;
  const int32_t *pos = p.pos + (size_t)u * p.cap;
  float m = -INFINITY, l = 0.f;
  for (int kt = 0; kt * kPT < L; ++kt) {
    if (p.krange[((size_t)u * nkt + kt) * 2] > qmax) continue;  // every key after every query
    __syncthreads();  // the previous tile is no longer read
    stage_rows<D>(sK, kc, RB, kt * kPT, L - 1, tid);
    if (tid < kPT) sP[tid] = kt * kPT + tid < L ? pos[kt * kPT + tid] : INT_MAX;
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < kPT / 16; ++kb) {
      pf32x4_t S = {0.f, 0.f, 0.f, 0.f};
      const char *arow = sK + (kb * 16 + col) * LRB + quad * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) S = pmfma(*reinterpret_cast<const pbf16x4_t *>(arow + ks * 32), qb[ks], S);
      float s[4], mx = m;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int kp = sP[kb * 16 + quad * 4 + ii];
        s[ii] = kp <= qp ? S[ii] * p.scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[ii]);
      }
      if (mx != -INFINITY) {
        l *= fast_exp2(m - mx);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) l += fast_exp2(s[ii] - mx);
        m = mx;
      }
    }
  }
  // the four lanes of a query (quads) merge their running max and sum
#pragma unroll
  for (int off = 16; off < 64; off <<= 1) {
    const float mo = __shfl_xor(m, off), lo = __shfl_xor(l, off);
    const float mx = fmaxf(m, mo);
    const float mxs = (mx == -INFINITY) ? 0.f : mx;
    l = l * fast_exp2(m - mxs) + lo * fast_exp2(mo - mxs);
    m = mx;
  }
  if (quad == 0 && i < p.n_obs) {
    const size_t sid = (((size_t)u * p.G + g) * p.n_obs + i) * 2;
    p.stats[sid] = m;
    p.stats[sid + 1] = l;
  }
}

template <int D>
__global__ __launch_bounds__(256) void k_prefill_accum_mfma(PrefillArgs p) {
  constexpr int RB = D * 2, LRB = RB + 16, KS = D / 16;
  const int kt = blockIdx.x, u = blockIdx.y;
  const int b = u / p.Hkv, j = u - b * p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, quad = lane >> 4, col = lane & 15;
  const int L = min(p.len[u], p.cap);
  if (kt * kPT >= L) return;
  const int nkt = (p.cap + kPT - 1) / kPT, nqt = (p.n_obs + kPT - 1) / kPT;
  const char *kc = static_cast<const char *>(p.k_cache) + (size_t)u * p.cap * RB;
  const int32_t *pos = p.pos + (size_t)u * p.cap;
  // A operand: the wave's 16 keys stay in registers
  const int kr = min(kt * kPT + wave * 16 + col, L - 1);
  pbf16x4_t ka[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    ka[ks] = *reinterpret_cast<const pbf16x4_t *>(kc + (size_t)kr * RB + ks * 32 + quad * 8);
  int kp[4];  // positions of this lane's four output keys (INT_MAX: no key)
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int n = kt * kPT + wave * 16 + quad * 4 + ii;
    kp[ii] = n < L ? pos[n] : INT_MAX;
  }
  const int kmin = p.krange[((size_t)u * nkt + kt) * 2], kmax = p.krange[((size_t)u * nkt + kt) * 2 + 1];
  __shared__ __attribute__((aligned(16))) char sQ[kPT * LRB];
  __shared__ float sM[kPT], sIL[kPT];
  __shared__ int sQP[kPT];
  float cs[4] = {0.f, 0.f, 0.f, 0.f};
  for (int g = 0; g < p.G; ++g) {
    const int h = j * p.G + g;
    const char *qbase = static_cast<const char *>(p.q_obs) + ((size_t)(b * p.Hq + h)) * p.n_obs * RB;
    for (int qt = 0; qt < nqt; ++qt) {
      const int qlo = p.qrange[((size_t)b * nqt + qt) * 2], qhi = p.qrange[((size_t)b * nqt + qt) * 2 + 1];
      if ((int64_t)qhi < kmin) continue;                                   // every query before every key
      if (p.window > 0 && (int64_t)qlo - kmax >= p.window) continue;       // every query past the window
      __syncthreads();
      stage_rows<D>(sQ, qbase, RB, qt * kPT, p.n_obs - 1, tid);
      if (tid < kPT) {
        const int i = qt * kPT + tid;
        const bool ok = i < p.n_obs;
        const size_t sid = (((size_t)u * p.G + g) * p.n_obs + (ok ? i : 0)) * 2;
        const float lv = ok ? p.stats[sid + 1] : 0.f;
        sM[tid] = ok ? p.stats[sid] : 0.f;
        sIL[tid] = lv > 0.f ? 1.f / lv : 0.f;
        sQP[tid] = ok ? p.q_pos[(size_t)b * p.n_obs + i] : INT_MIN;
      }
      __syncthreads();
#pragma unroll
      for (int qb = 0; qb < kPT / 16; ++qb) {
        pf32x4_t S = {0.f, 0.f, 0.f, 0.f};
        const char *brow = sQ + (qb * 16 + col) * LRB + quad * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) S = pmfma(ka[ks], *reinterpret_cast<const pbf16x4_t *>(brow + ks * 32), S);
        const int qi = qb * 16 + col;
        const int qp = sQP[qi];
        const float mq = sM[qi], il = sIL[qi];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int64_t d = (int64_t)qp - kp[ii];
          const bool ok = d >= 0 && (p.window == 0 || d < p.window);
          cs[ii] += ok ? fast_exp2(S[ii] * p.scale_log2 - mq) * il : 0.f;
        }
      }
    }
  }
  // the 16 lanes of a quad hold the same keys for different queries
#pragma unroll
  for (int off = 1; off < 16; off <<= 1)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) cs[ii] += __shfl_xor(cs[ii], off);
  if (col == 0) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int n = kt * kPT + wave * 16 + quad * 4 + ii;
      if (n < L) p.imp[(size_t)u * p.cap + n] += cs[ii];
    }
  }
}

hipError_t launch_prefill(const PrefillArgs &p, int dtype, hipStream_t s) {
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
