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
// This is the plain VALU form for modest prompt sizes.

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

hipError_t launch_prefill(const PrefillArgs &p, int dtype, hipStream_t s) {
  const dim3 g1(p.n_units * p.G * p.n_obs), blk(256);
  const dim3 g2((p.cap + 63) / 64, p.n_units);
  if (dtype == HIKV_BF16) {
    if (p.D == 128) {
      hipLaunchKernelGGL((k_prefill_stats<2, 128>), g1, blk, 0, s, p);
      hipLaunchKernelGGL((k_prefill_accum<2, 128>), g2, blk, 0, s, p);
    } else {
      hipLaunchKernelGGL((k_prefill_stats<2, 64>), g1, blk, 0, s, p);
      hipLaunchKernelGGL((k_prefill_accum<2, 64>), g2, blk, 0, s, p);
    }
  } else {
    if (p.D == 128) {
      hipLaunchKernelGGL((k_prefill_stats<4, 128>), g1, blk, 0, s, p);
      hipLaunchKernelGGL((k_prefill_accum<4, 128>), g2, blk, 0, s, p);
    } else {
      hipLaunchKernelGGL((k_prefill_stats<4, 64>), g1, blk, 0, s, p);
      hipLaunchKernelGGL((k_prefill_accum<4, 64>), g2, blk, 0, s, p);
    }
  }
  return hipGetLastError();
}

}  // namespace hikv
