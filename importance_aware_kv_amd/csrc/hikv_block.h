// hikv_block.h -- workgroup-wide scan / reduction / radix-select helpers.
#pragma once

#include "hikv_common.h"

namespace hikv {

// Exclusive prefix sum over the workgroup (NT threads, a multiple of 64):
// a scan within each wave, then the wave totals (sc: at least NT / 64 ints).
template <int NT>
__device__ int block_excl_scan(int v, int *sc, int *total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) sc[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int x = sc[w];
    if (w < wave) base += x;
    tot += x;
  }
  *total = tot;
  __syncthreads();  // sc is free for the next call
  return base + incl - v;
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
        // (named values: a small array indexed at run time goes to scratch)
        const uint32_t c1 = excl + h0, c2 = c1 + h1, c3 = c2 + h2;
        const int d = c1 >= krem ? 0 : (c2 >= krem ? 1 : (c3 >= krem ? 2 : 3));
        const uint32_t cum = d == 0 ? excl : (d == 1 ? c1 : (d == 2 ? c2 : c3));
        const uint32_t hd = d == 0 ? h0 : (d == 1 ? h1 : (d == 2 ? h2 : h3));
        const uint32_t rem = krem - cum;
        st->prefix = prefix | ((uint64_t)(4 * tid + d) << shift);
        st->shift = shift;
        st->krem = (int)rem;
        st->done = (hd == rem) ? 1 : 0;
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
        // (named values: a small array indexed at run time goes to scratch)
        const uint32_t c1 = excl + h0, c2 = c1 + h1, c3 = c2 + h2;
        const int d = c1 >= krem ? 0 : (c2 >= krem ? 1 : (c3 >= krem ? 2 : 3));
        const uint32_t cum = d == 0 ? excl : (d == 1 ? c1 : (d == 2 ? c2 : c3));
        const uint32_t hd = d == 0 ? h0 : (d == 1 ? h1 : (d == 2 ? h2 : h3));
        const uint32_t rem = krem - cum;
        st->prefix = prefix | ((uint64_t)(4 * tid + d) << shift);
        st->shift = shift;
        st->krem = (int)rem;
        st->done = (hd == rem) ? 1 : 0;
      }
    }
    __syncthreads();
    if (st->done) break;
  }
}

// The listing and moves of a unit's bulk eviction, once the threshold is
// known: a slot is evicted when its key (keys[n]; UINT64_MAX for a protected
// token) satisfies (key >> shift) <= lim.  The survivors at or above the
// budget move into the evicted slots below it (K and V rows of RB bytes,
// position, importance), and *len_u = beta.  holes and movers are the unit's
// [cap] lists in the workspace, both in ascending slot order.  With nmoves_u
// given, the moves are left to a later launch: the number of rows to move
// goes to *nmoves_u instead.  ebits: NT words of LDS scratch.  Every thread
// of the workgroup calls it.
template <int NT, int RB>
__device__ __forceinline__ void bulk_list(const uint64_t *keys, int L, int beta, uint64_t lim, int shift,
                                          char *kw, char *vw, int32_t *posw, float *impw, int32_t *holes,
                                          int32_t *movers, int32_t *len_u, int32_t *status, uint64_t *ebits,
                                          int *sc, int32_t *nmoves_u) {
  constexpr int NW = NT / 64, SEG = NT * 64, KPT = 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tot_h = 0, tot_m = 0;  // over the earlier segments
  for (int s0 = 0; s0 < L; s0 += SEG) {
    // The segment's evicted flags, one bit per slot (word w: slots s0 + 64 w
    // ...): keys read coalesced, one ballot per 64 slots.  Words wholly past
    // L are left as they are: no slot of theirs is counted.
    for (int j0 = 0; j0 < SEG / NT && s0 + j0 * NT < L; j0 += KPT) {
      uint64_t kk[KPT];
#pragma unroll
      for (int j = 0; j < KPT; ++j) kk[j] = keys[min(s0 + (j0 + j) * NT + tid, L - 1)];
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int n = s0 + (j0 + j) * NT + tid;
        const uint64_t m = __ballot(n < L && kk[j] != ~0ull && (kk[j] >> shift) <= lim);
        if (lane == 0 && j0 + j < SEG / NT) ebits[(j0 + j) * NW + wave] = m;
      }
    }
    __syncthreads();
    const uint64_t e = ebits[tid];
    const int nb = s0 + 64 * tid;  // the first slot of this thread's word
    auto below = [&](int lim_slot) -> uint64_t {  // the word's bits of slots < lim_slot
      const int c = lim_slot - nb;
      return c <= 0 ? 0ull : (c >= 64 ? ~0ull : ((1ull << c) - 1ull));
    };
    const uint64_t valid = below(L), low = below(beta);
    const uint64_t hm = e & valid & low, mm = ~e & valid & ~low;
    int th, tm;
    int ih = tot_h + block_excl_scan<NT>(__popcll(hm), sc, &th);
    int im = tot_m + block_excl_scan<NT>(__popcll(mm), sc, &tm);
    for (uint64_t x = hm; x; x &= x - 1ull) holes[ih++] = nb + __builtin_ctzll(x);
    for (uint64_t x = mm; x; x &= x - 1ull) movers[im++] = nb + __builtin_ctzll(x);
    tot_h += th;
    tot_m += tm;
    __syncthreads();  // ebits is rebuilt for the next segment
  }
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

// Bulk eviction of one unit by one workgroup of NT threads, from the
// eviction keys of its L slots: the n_evict smallest keys are evicted (a
// radix select over the keys), then bulk_list.
template <int NT, int RB>
__device__ __forceinline__ void bulk_compact(const uint64_t *keys, int L, int beta, int n_evict, char *kw, char *vw,
                             int32_t *posw, float *impw, int32_t *holes, int32_t *movers,
                             int32_t *len_u, int32_t *status, uint32_t *hist, uint32_t *whist, int *sc,
                             RadixState *rs, int32_t *nmoves_u = nullptr) {
  radix_select_keys<NT, 8>(keys, L, n_evict, hist, whist, rs);
  // the select's per-wave histograms (NT / 64 x 256 words) are free again
  bulk_list<NT, RB>(keys, L, beta, rs->prefix >> rs->shift, rs->shift, kw, vw, posw, impw, holes, movers, len_u,
                    status, reinterpret_cast<uint64_t *>(whist), sc, nmoves_u);
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
