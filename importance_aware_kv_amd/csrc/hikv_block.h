// hikv_block.h -- workgroup-wide scan / reduction / radix-select helpers.
#pragma once

#include "hikv_common.h"

namespace hikv {

template <int NT>
__device__ int block_excl_scan(int v, int *sc, int *total) {
  const int t = threadIdx.x;
  sc[t] = v;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {
    const int x = (t >= off) ? sc[t - off] : 0;
    __syncthreads();
    sc[t] += x;
    __syncthreads();
  }
  const int incl = sc[t];
  *total = sc[NT - 1];
  __syncthreads();
  return incl - v;
}

template <int NT>
__device__ long long block_sum_ll(long long v, long long *sc) {
  const int t = threadIdx.x;
  sc[t] = v;
  __syncthreads();
  for (int off = NT / 2; off > 0; off >>= 1) {
    if (t < off) sc[t] += sc[t + off];
    __syncthreads();
  }
  const long long r = sc[0];
  __syncthreads();
  return r;
}

__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t x = __shfl_up(v, off);
    if (lane >= off) v += x;
  }
  return v;
}

struct RadixState {
  uint64_t prefix;
  int shift, krem, done;
};

// Radix select over 64-bit keys, 8-bit digits from the most significant one.
// Among the items n in [0, n_items) for which key_of(n, key) is true, finds
// (prefix, shift) such that exactly k of them satisfy
// (key >> shift) <= (prefix >> shift).  Keys must be distinct and
// 1 <= k <= number of participating items.  The search stops at the first
// digit whose bucket is taken whole.  Every thread of the block must call it;
// the result is in *st when it returns.
template <int NT, typename F>
__device__ void radix_select_smallest(int n_items, int k, F key_of, uint32_t *hist,
                                      RadixState *st) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    st->prefix = 0;
    st->shift = 64;
    st->krem = k;
    st->done = 0;
  }
  __syncthreads();
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    const uint64_t prefix = st->prefix;
    for (int i = tid; i < 256; i += NT) hist[i] = 0;
    __syncthreads();
    for (int n = tid; n < n_items; n += NT) {
      uint64_t key;
      if (!key_of(n, key)) continue;
      if (pass > 0 && (key >> (shift + 8)) != (prefix >> (shift + 8))) continue;
      atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // Find the digit whose bucket holds the krem-th smallest key: each lane
      // owns 4 bins, one wave scan gives the crossing lane.
      const uint32_t krem = (uint32_t)st->krem;
      const uint32_t h0 = hist[4 * tid], h1 = hist[4 * tid + 1], h2 = hist[4 * tid + 2],
                     h3 = hist[4 * tid + 3];
      const uint32_t s = h0 + h1 + h2 + h3;
      const uint32_t incl = wave_incl_scan_u32(s);
      const uint32_t excl = incl - s;
      if (excl < krem && incl >= krem) {
        const uint32_t hh[4] = {h0, h1, h2, h3};
        uint32_t cum = excl;
        int d = 3;
        for (int i = 0; i < 4; ++i) {
          if (cum + hh[i] >= krem) {
            d = i;
            break;
          }
          cum += hh[i];
        }
        const uint32_t rem = krem - cum;
        st->prefix = prefix | ((uint64_t)(4 * tid + d) << shift);
        st->shift = shift;
        st->krem = (int)rem;
        st->done = (hh[d] == rem) ? 1 : 0;
      }
    }
    __syncthreads();
    if (st->done) break;
  }
}

// The same selection over a contiguous array of keys, UINT64_MAX marking an
// item that does not take part (a real key equals it only for a NaN
// importance at position 0).  Each pass streams the array with KPT
// independent loads per thread in flight.  Every wave counts into a
// histogram of its own (whist: NT / 64 x 256 words): the digits of one pass
// are often nearly all equal, and a shared histogram would serialise the
// whole block on one or two bins.
template <int NT, int KPT>
__device__ void radix_select_keys(const uint64_t *keys, int n_items, int k, uint32_t *hist,
                                  uint32_t *whist, RadixState *st) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  uint32_t *mine = whist + (tid >> 6) * 256;
  if (tid == 0) {
    st->prefix = 0;
    st->shift = 64;
    st->krem = k;
    st->done = 0;
  }
  __syncthreads();
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    const uint64_t prefix = st->prefix;
    for (int i = tid; i < NW * 256; i += NT) whist[i] = 0;
    __syncthreads();
    for (int base = 0; base < n_items; base += NT * KPT) {
      uint64_t kk[KPT];
#pragma unroll
      for (int j = 0; j < KPT; ++j) kk[j] = keys[min(base + tid + j * NT, n_items - 1)];
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const uint64_t key = kk[j];
        const bool in = base + tid + j * NT < n_items && key != ~0ull &&
                        (pass == 0 || (key >> (shift + 8)) == (prefix >> (shift + 8)));
        const int d = in ? (int)((key >> shift) & 255u) : 256;
        // The lanes that share the first lane's digit are counted at once.
        const int d0 = __builtin_amdgcn_readfirstlane(d);
        const uint64_t same = __ballot(d == d0);
        if (d == d0) {
          if (d0 < 256 && (tid & 63) == __builtin_ctzll(same)) atomicAdd(&mine[d0], (uint32_t)__popcll(same));
        } else if (d < 256) {
          atomicAdd(&mine[d], 1u);
        }
      }
    }
    __syncthreads();
    for (int i = tid; i < 256; i += NT) {
      uint32_t c = 0;
      for (int w = 0; w < NW; ++w) c += whist[w * 256 + i];
      hist[i] = c;
    }
    __syncthreads();
    if (tid < 64) {
      const uint32_t krem = (uint32_t)st->krem;
      const uint32_t h0 = hist[4 * tid], h1 = hist[4 * tid + 1], h2 = hist[4 * tid + 2],
                     h3 = hist[4 * tid + 3];
      const uint32_t s = h0 + h1 + h2 + h3;
      const uint32_t incl = wave_incl_scan_u32(s);
      const uint32_t excl = incl - s;
      if (excl < krem && incl >= krem) {
        const uint32_t hh[4] = {h0, h1, h2, h3};
        uint32_t cum = excl;
        int d = 3;
        for (int i = 0; i < 4; ++i) {
          if (cum + hh[i] >= krem) {
            d = i;
            break;
          }
          cum += hh[i];
        }
        const uint32_t rem = krem - cum;
        st->prefix = prefix | ((uint64_t)(4 * tid + d) << shift);
        st->shift = shift;
        st->krem = (int)rem;
        st->done = (hh[d] == rem) ? 1 : 0;
      }
    }
    __syncthreads();
    if (st->done) break;
  }
}

// Bulk eviction of one unit by one workgroup of NT threads, from the
// eviction keys of its L slots (keys[n]; UINT64_MAX for a protected token):
// the n_evict smallest keys are evicted, then the survivors at or above the
// budget move into the evicted slots below it (K and V rows of RB bytes,
// position, importance), and *len_u = beta.  holes and movers are the unit's
// [cap] lists in the workspace.  With nmoves_u given, the moves are left to a
// later launch: the number of rows to move goes to *nmoves_u instead.  Every
// thread of the workgroup calls it.
template <int NT, int RB>
__device__ __forceinline__ void bulk_compact(const uint64_t *keys, int L, int beta, int n_evict, char *kw, char *vw,
                             int32_t *posw, float *impw, int32_t *holes, int32_t *movers,
                             int32_t *len_u, int32_t *status, uint32_t *hist, uint32_t *whist, int *sc,
                             RadixState *rs, int32_t *nmoves_u = nullptr) {
  const int tid = threadIdx.x;
  radix_select_keys<NT, 8>(keys, L, n_evict, hist, whist, rs);
  const uint64_t lim = rs->prefix >> rs->shift;
  const int shift = rs->shift;
  // Slots [n0, n1) of this thread, contiguous; their evicted flags stay in a
  // mask between the counting and the listing pass (up to 64 slots per
  // thread; beyond that the keys are read again).
  const int per = (L + NT - 1) / NT;
  const int n0 = min(tid * per, L), n1 = min(n0 + per, L);
  uint64_t emask = 0;
  int nh = 0, nm = 0;
  for (int g0 = n0; g0 < n1; g0 += 8) {
    uint64_t kk[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) kk[j] = keys[min(g0 + j, n1 - 1)];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = g0 + j;
      const bool e = n < n1 && kk[j] != ~0ull && (kk[j] >> shift) <= lim;
      if (e && n - n0 < 64) emask |= 1ull << (n - n0);
      nh += (n < n1 && n < beta && e);
      nm += (n < n1 && n >= beta && !e);
    }
  }
  int tot_h, tot_m;
  int oh = block_excl_scan<NT>(nh, sc, &tot_h);
  int om = block_excl_scan<NT>(nm, sc, &tot_m);
  for (int n = n0; n < n1; ++n) {
    bool e;
    if (n - n0 < 64) {
      e = (emask >> (n - n0)) & 1;
    } else {
      const uint64_t key = keys[n];
      e = key != ~0ull && (key >> shift) <= lim;
    }
    if (n < beta && e) holes[oh++] = n;
    if (n >= beta && !e) movers[om++] = n;
  }
  __syncthreads();
  if (tot_h != tot_m) {  // cannot happen for distinct positions; fail safe
    if (tid == 0) set_status(status, HIKV_EINVAL);
    return;
  }
  if (nmoves_u) {
    if (tid == 0) {
      *nmoves_u = tot_m;
      *len_u = beta;
    }
    return;
  }
  // A round copies two groups of NT / CPR rows, CPR threads per row, with
  // every load of the round issued before its stores (hole and mover rows are
  // distinct, so nothing a round stores is loaded in it).
  constexpr int CPR = RB / 16, RPG = NT / CPR;
  const int ci = tid % CPR, rr = tid / CPR;
  for (int i0 = 0; i0 < tot_m; i0 += 2 * RPG) {
    const int ia = i0 + rr, ib = i0 + RPG + rr;
    const int ja = min(ia, tot_m - 1), jb = min(ib, tot_m - 1);
    const int sa = movers[ja], da = holes[ja], sb = movers[jb], db = holes[jb];
    const uint4 ka = reinterpret_cast<const uint4 *>(kw + (size_t)sa * RB)[ci];
    const uint4 va = reinterpret_cast<const uint4 *>(vw + (size_t)sa * RB)[ci];
    const uint4 kb = reinterpret_cast<const uint4 *>(kw + (size_t)sb * RB)[ci];
    const uint4 vb = reinterpret_cast<const uint4 *>(vw + (size_t)sb * RB)[ci];
    const int pa = posw[sa], pb = posw[sb];
    const float xa = impw[sa], xb = impw[sb];
    if (ia < tot_m) {
      reinterpret_cast<uint4 *>(kw + (size_t)da * RB)[ci] = ka;
      reinterpret_cast<uint4 *>(vw + (size_t)da * RB)[ci] = va;
      if (ci == 0) posw[da] = pa, impw[da] = xa;
    }
    if (ib < tot_m) {
      reinterpret_cast<uint4 *>(kw + (size_t)db * RB)[ci] = kb;
      reinterpret_cast<uint4 *>(vw + (size_t)db * RB)[ci] = vb;
      if (ci == 0) posw[db] = pb, impw[db] = xb;
    }
  }
  if (tid == 0) *len_u = beta;
}

// ---------------------------------------------------------------------------
// The cache's pending eviction (hikv_cache.evict; see the two-launch step):
// the dead slot of unit u, or -1 when none is pending.  One whole wave; every
// lane returns the slot.
// ---------------------------------------------------------------------------
__device__ inline int pending_slot_wave(const StepArgs &a, int u) {
  const int lane = threadIdx.x & 63;
  const int nbm = imp_blocks(a.cap);
  const int32_t *rec = a.evict + (size_t)u * state_words(a.cap);
  const int n = min(rec[0], nbm);
  uint32_t khi = ~0u, klo = ~0u;
  int slot = -1;
  for (int i = lane; i < n; i += 64) {
    const int4 e = reinterpret_cast<const int4 *>(rec + 4)[i];
    const uint32_t h = (uint32_t)e.y, l = (uint32_t)e.x;
    if (h < khi || (h == khi && l < klo)) khi = h, klo = l, slot = e.z;
  }
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t h = (uint32_t)__shfl_xor((int)khi, off), l = (uint32_t)__shfl_xor((int)klo, off);
    const int s = __shfl_xor(slot, off);
    if (h < khi || (h == khi && l < klo)) khi = h, klo = l, slot = s;
  }
  return (khi == ~0u && klo == ~0u) ? -1 : slot;
}

// Resolve unit u's pending eviction in place (one whole wave): the unit's
// last slot moves into the dead one (K and V rows of rb bytes, position,
// importance), len drops by one and nothing stays pending ([Kelle] Sec. 2.2:
// slot order does not matter).
__device__ inline void settle_unit(const StepArgs &a, int u, int rb) {
  const int lane = threadIdx.x & 63;
  int32_t *rec = a.evict + (size_t)u * state_words(a.cap);
  if (rec[0] == 0) return;
  const int d = pending_slot_wave(a, u);
  if (d >= 0) {
    const int last = a.len[u] - 1;
    if (d != last) {
      const int nc = rb / 16;  // 16-byte pieces of a row; one wave moves a K and a V row
      char *base = static_cast<char *>(lane < nc ? a.k_w : a.v_w) + (size_t)u * a.cap * rb;
      const int off = (lane % nc) * 16;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (lane < 2 * nc) x = *reinterpret_cast<const uint4 *>(base + (size_t)last * rb + off);
      const int32_t p = a.pos[(size_t)u * a.cap + last];
      const float im = a.imp[(size_t)u * a.cap + last];
      if (lane < 2 * nc) *reinterpret_cast<uint4 *>(base + (size_t)d * rb + off) = x;
      if (lane == 0) {
        a.pos[(size_t)u * a.cap + d] = p;
        a.imp[(size_t)u * a.cap + d] = im;
      }
    }
    if (lane == 0) a.len[u] = last;
  }
  if (lane == 0) rec[0] = 0;
}

}  // namespace hikv
