// fused.hip -- the Stage I decode step in one launch (bf16 K and V, D = 128),
// and the resolution of the deferred state it leaves in the cache.
//
// Method (pages cited by title and section): decode attention GeMVs ("HiKV",
// Sec. II-A); importance = attention probabilities accumulated over the
// steps, pooled over the q-heads of a KV group ("KV Cache Compression and
// Dynamic Pruning in Production Serving", Sec. 3 H2O, Sec. 5); eviction of
// the lowest importance outside the sinks and the recent window (same page,
// Sec. 3); an unordered slot cache in which the new token takes the evicted
// token's slot ("Kelle" summary, Sec. 2.2 and Sec. 4.1).
//
// Deferred accumulation.  Step t's probabilities P_t are known only once
// every split-K tile of a unit is done.  The step therefore leaves them
// unapplied: the cache keeps step t's softmax statistics (per q-head maximum
// and sum) and its queries q_t, and step t+1's tiles, which stream the same K
// rows anyway, recompute q_t . k on the matrix cores (in the spare columns of
// the same MFMA: this step's G <= 8 heads use at most 8 of its 16 columns)
// and add P_t to the importance of their own slots.
//
// Held-out token.  Step t's victim (lowest eviction key once P_t is added)
// is then known to no single tile.  Each tile leaves its own lowest key out
// of step t+1's softmax and sets that token's logits and V row aside.  The
// unit's last tile to finish (a per-unit ticket) takes the lowest of the
// tiles' keys as the victim, adds every other held-out token back into the
// combined softmax, writes the output, and puts the new token into the
// victim's slot.  No logit leaves the chip and no second launch is needed.
// Outputs and kept sets equal those of the step-by-step method;
// k_settle_lazy applies the deferred part at any point (hikv_settle).

#include <hip/hip_ext.h>

#include "hikv_block.h"
#include "hikv_dev.h"
#include "hikv_launch.h"

namespace hikv {

namespace {

constexpr int kFT = 256;  // threads of a fused-step workgroup (four waves)

// The deferred step's scalars, wave-uniform.
struct LazyView {
  int flag, over, newest, wp, sink, acc;
  float cs;
};

__device__ __forceinline__ LazyView lazy_view(const int32_t *h) {
  LazyView v;
  v.flag = __builtin_amdgcn_readfirstlane(h[kLzFlag]);
  v.over = __builtin_amdgcn_readfirstlane(h[kLzOver]);
  v.newest = __builtin_amdgcn_readfirstlane(h[kLzNewest]);
  v.wp = __builtin_amdgcn_readfirstlane(h[kLzWp]);
  v.sink = __builtin_amdgcn_readfirstlane(h[kLzSink]);
  v.acc = __builtin_amdgcn_readfirstlane(h[kLzAcc]);
  v.cs = __int_as_float(__builtin_amdgcn_readfirstlane(h[kLzCs]));
  return v;
}

// The deferred step's contribution to four tokens of a staged sub-chunk (the
// tokens of one 16-lane row of the MFMA output S): columns G .. 2G-1 of S hold
// q_t . k (raw) for the deferred step's heads; (mc, il) are this lane's head's
// maximum (times the scale, log2 domain) and 1 / sum.  phys: the row is a
// cached token (all of them were live at the deferred step).  Returns in every
// lane of the row each token's importance with the deferred probabilities
// added (or frozen outside the window with HIKV_ACC_RECENT; the logit times
// the scale with HIKV_ACC_LOGIT), whether it changed, and its eviction key
// when it is a candidate of the deferred step's eviction (~0 otherwise).
// Both the fused step and k_settle_lazy call this, so that they agree to the
// bit.
template <int G>
__device__ __forceinline__ void lazy_tokens(const f32x4_t &S, int hl, const LazyView &z, float mc, float il,
                                            const float (&ip)[4], const int (&pp)[4], const bool (&phys)[4],
                                            float (&it)[4], uint64_t (&key)[4], bool (&acc)[4]) {
  const bool col = hl >= G && hl < 2 * G;
  const float snat = z.cs * 0.69314718055994531f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float tm = 0.f;
    if (col) tm = (z.acc == HIKV_ACC_LOGIT) ? S[r] * snat : fast_exp2(fmaf(S[r], z.cs, -mc)) * il;
    tm = row_sum<16>(tm);
    const bool rec = pp[r] > z.newest - z.wp;
    acc[r] = phys[r] && (z.acc != HIKV_ACC_RECENT || rec);
    it[r] = ip[r] + (acc[r] ? tm : 0.f);
    const bool cand = z.over && phys[r] && pp[r] >= z.sink && !rec;
    key[r] = cand ? evict_key(it[r], pp[r]) : ~0ull;
  }
}

// Lowest of a lane's four keys, then over the four 16-lane rows (every lane
// of a row holds the same four tokens): the wave's lowest key and its row in
// the 16-token group, in every lane.
__device__ __forceinline__ void group_min_key(const uint64_t (&key)[4], int qd, uint64_t &bk, int &brow) {
  uint64_t k = key[0];
  int r = 0;
#pragma unroll
  for (int i = 1; i < 4; ++i)
    if (key[i] < k) k = key[i], r = i;
  KeySlot x{(uint32_t)(k >> 32), (uint32_t)k, (uint32_t)(4 * qd + r)};
  auto lo_first = [](KeySlot p, KeySlot q) {
    const bool take_q = (q.hi < p.hi) || (q.hi == p.hi && (q.lo < p.lo || (q.lo == p.lo && q.slot < p.slot)));
    return take_q ? q : p;
  };
  {
    KeySlot p = x, q = x;
    swap16_u(p.hi, q.hi);
    swap16_u(p.lo, q.lo);
    swap16_u(p.slot, q.slot);
    x = lo_first(p, q);
  }
  {
    KeySlot p = x, q = x;
    swap32_u(p.hi, q.hi);
    swap32_u(p.lo, q.lo);
    swap32_u(p.slot, q.slot);
    x = lo_first(p, q);
  }
  bk = ((uint64_t)__builtin_amdgcn_readfirstlane(x.hi) << 32) | (uint32_t)__builtin_amdgcn_readfirstlane(x.lo);
  brow = __builtin_amdgcn_readfirstlane((int)x.slot);
}

// Four 16-byte LDS reads of importance and position words staged by DMA.
// asm for the reason given at lds_read_rows (the ring is one array).
__device__ __forceinline__ void lds_read_ip(float (&ip)[4], int (&pp)[4], uint32_t ai, uint32_t ap) {
  u32x4 x, y;
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(x), "=&v"(y)
               : "v"(ai), "v"(ap)
               : "memory");
  ip[0] = __uint_as_float(x.x), ip[1] = __uint_as_float(x.y), ip[2] = __uint_as_float(x.z), ip[3] = __uint_as_float(x.w);
  pp[0] = (int)y.x, pp[1] = (int)y.y, pp[2] = (int)y.z, pp[3] = (int)y.w;
}

// One bf16 of a staged row (asm: see lds_read_ip).
__device__ __forceinline__ float lds_read_bf16(uint32_t addr) {
  uint32_t v;
  asm volatile("ds_read_u16 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return __uint_as_float(v << 16);
}

// Eight 8-byte LDS reads 32 bytes apart from one per-lane address, one wait.
// asm: the LDS arrays were filled by DMA, and a compiler-visible read of one
// of them makes the compiler wait for every load in flight (the ring's too).
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
__device__ __forceinline__ u32x4 lds_read_b128(uint32_t addr) {
  u32x4 x;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(x) : "v"(addr) : "memory");
  return x;
}
__device__ __forceinline__ uint32_t lds_read_b32(uint32_t addr) {
  uint32_t x;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(x) : "v"(addr) : "memory");
  return x;
}

// The deferred-step record's scalars from LDS (asm reads: see lds_read8_b64).
__device__ __forceinline__ LazyView lazy_view_lds(const void *lz) {
  const uint32_t a0 = lds_addr(lz);
  const u32x4 x = lds_read_b128(a0), y = lds_read_b128(a0 + 16);
  LazyView v;
  v.flag = __builtin_amdgcn_readfirstlane((int)x.x);
  v.over = __builtin_amdgcn_readfirstlane((int)x.y);
  v.newest = __builtin_amdgcn_readfirstlane((int)x.z);
  v.wp = __builtin_amdgcn_readfirstlane((int)x.w);
  v.sink = __builtin_amdgcn_readfirstlane((int)y.x);
  v.acc = __builtin_amdgcn_readfirstlane((int)y.y);
  v.cs = __int_as_float(__builtin_amdgcn_readfirstlane((int)y.z));
  return v;
}

// The MFMA B operand of a lane: column hl < G holds this step's query of head
// hl, column G <= hl < 2G the deferred step's query of head hl - G (q_t), the
// rest zero.  q rows are [G][128] bf16 in LDS (qn may be null: no columns < G).
template <int G>
__device__ __forceinline__ void query_operand(bf16x4_t (&qb)[8], const char *qn, const char *qt, int hl, int qd,
                                              bool with_t) {
  const bool mine = qn && hl < G, prev = with_t && hl >= G && hl < 2 * G;
  const uint32_t addr = mine ? lds_addr(qn + (hl * 128 + 4 * qd) * 2)
                             : lds_addr(qt + ((prev ? hl - G : 0) * 128 + 4 * qd) * 2);
  uint64_t w[8];
  lds_read8_b64(w, addr);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qb[ks] = __builtin_bit_cast(bf16x4_t, (mine || prev) ? w[ks] : 0ull);
}

// Eight K reads of a staged sub-chunk (the q.k A operand), one wait.
__device__ __forceinline__ void mfma_k_operand(uint64_t (&o)[8], const uint32_t (&ad)[12], uint32_t boff) {
  uint32_t x[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = ad[k] + boff;
  asm volatile(
      "ds_read_b64 %0, %8\n\t"
      "ds_read_b64 %1, %9\n\t"
      "ds_read_b64 %2, %10\n\t"
      "ds_read_b64 %3, %11\n\t"
      "ds_read_b64 %4, %12\n\t"
      "ds_read_b64 %5, %13\n\t"
      "ds_read_b64 %6, %14\n\t"
      "ds_read_b64 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
      : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7])
      : "memory");
}

// Largest tile count of one unit that the combine's LDS tables (a factor per
// tile and q-head for the partial and for the held-out token) hold within the
// staging ring, 6 KB of which stay for the reductions.
constexpr int kCombineScratch = 6144;
template <int G>
constexpr int fused_max_unit_tiles() {
  return (3 * 2 * 8192 - kCombineScratch) / (8 * G);
}

// LDS of the tile's end: per wave, its held-out token.
template <int G>
struct HoldW {
  uint32_t khi, klo;
  int32_t slot, pad;
  float hs[8];
  float hv[64];
};

}  // namespace

// ---------------------------------------------------------------------------
// The fused step.  One workgroup (four waves) per split-K tile of the host
// plan; the grid is one resident round.  Per 32-token sub-chunk, wave w takes
// token group w & 1 and channel half w >> 1 of P.V, as the two-launch step's
// attention launch does.
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(kFT) void k_step_fused(StepArgs a) {
  constexpr int EL = 2, D = 128, RB = D * EL, SUBB = 8192, TS = SUBB / RB, NSUB = 3, NI = SUBB / 4096;
  constexpr int QB = G * D * EL;       // the group's queries, bytes
  constexpr int LZB = kLzQ * 4 + QB;   // the deferred-step record, bytes
  static_assert(TS == 32 && 2 * G <= 16, "two 16-token groups per sub-chunk; 2G MFMA columns");
  __shared__ __attribute__((aligned(16))) char smem[NSUB * 2 * SUBB];  // ring: K then V per sub-chunk
  __shared__ __attribute__((aligned(16))) char qs[QB];                  // this step's queries
  __shared__ __attribute__((aligned(16))) char lz[LZB];                 // the deferred-step record
  __shared__ __attribute__((aligned(16))) int32_t ipb[NSUB][64];        // importance [0, 32), positions [32, 64)
  __shared__ __attribute__((aligned(16))) int32_t uw[4];                // len, budget, candidate count, newest
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hp_bend = a.hp.base[lane + 1], hp_len = a.hp.L[lane];
  const Plan pl = host_plan(a, blockIdx.x, hp_bend, hp_len);
  if (!pl.valid) return;
  const int u = pl.u, b = u / a.Hkv, j = u - b * a.Hkv;
  const int Lold = pl.L - 1, t0 = pl.t0, t1 = pl.t1, tile = blockIdx.x;
  const char *kc = static_cast<const char *>(a.k_cache) + (size_t)u * a.cap * RB;
  const char *vc = static_cast<const char *>(a.v_cache) + (size_t)u * a.cap * RB;
  const char *kn = static_cast<const char *>(a.k_new) + (size_t)u * RB;
  const char *vn = static_cast<const char *>(a.v_new) + (size_t)u * RB;
  float *impw = a.imp + (size_t)u * a.cap;
  int32_t *posw = a.pos + (size_t)u * a.cap;
  int32_t *lrec = a.evict + (size_t)u * a.state_stride + state_words(a.cap);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  // This step's queries, the deferred-step record and the unit's words every
  // tile checks before it writes (the two-launch form's candidate count must
  // be 0: that form is settled before this step runs), all by DMA.
  {
    const int off = wave * 1024 + lane * 16;
    const char *qsrc = static_cast<const char *>(a.q) + (size_t)(b * a.Hq + j * G) * D * EL;
    if (off < QB) dma16(qsrc + off, qs + wave * 1024);
    if (off < LZB) dma16(reinterpret_cast<const char *>(lrec) + off, lz + wave * 1024);
    if (wave == 0 && lane < 4) {
      const int32_t *src = lane == 0 ? a.len + u
                         : lane == 1 ? (a.budget ? a.budget + u : a.new_pos + b)
                         : lane == 2 ? a.evict + (size_t)u * a.state_stride
                                     : a.new_pos + b;
      __builtin_amdgcn_global_load_lds(src, uw, 4, 0, 0);
    }
  }

  const float cs = a.scale_log2, tau = 8.f / cs;
  const int grp = wave & 1, half = wave >> 1;
  const int hl = lane & 15, qd = lane >> 4;
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
  float m = -INFINITY, l = 0.f;
  bf16x4_t qb[8];
  // Ring: waves 2 and 3 issue every load (wave 2 also the sub-chunk's
  // importance and position words), waves 0 and 1 every store (see the
  // two-launch step's attention launch for why the roles are split).
  const bool loader = wave >= 2;
  const int nsc = (t1 - t0 + TS - 1) / TS;
  auto stage = [&](int sc, int buf) {
    const int c0 = t0 + sc * TS;
    stage_sub_by<2>(smem + buf * 2 * SUBB, smem + buf * 2 * SUBB + SUBB, kc, vc, kn, vn, c0, min(TS, t1 - c0), t0,
                    Lold, wave - 2, lane);
    if (wave == 2) {
      const int n = min(c0 + (lane & 31), a.cap - 1);
      const void *src = lane < 32 ? static_cast<const void *>(impw + n) : static_cast<const void *>(posw + n);
      __builtin_amdgcn_global_load_lds(src, &ipb[buf][0], 4, 0, 0);
    }
  };
  if (loader) {
#pragma unroll
    for (int sc = 0; sc < NSUB; ++sc)
      if (sc < nsc) stage(sc, sc);
  }
  LazyView z{};
  float mc = 0.f, il = 0.f;
  int err = 0, beta = 0, newest = 0;
  bool lazy = false, lazy_over = false;
  // The wave's held-out token: its key, slot, this step's logit of head hl
  // (lanes hl < G) and its V row at channels half*64 + 16t + hl.
  uint64_t hk = ~0ull;
  int hslot = -1;
  float hs = -INFINITY, hv[4] = {0.f, 0.f, 0.f, 0.f};
  const float *lzf = reinterpret_cast<const float *>(lz);
  const uint32_t ipb_a = lds_addr(&ipb[0][0]);

  // Raise head hl's running maximum to mx (raw q.k), rescaling the sum and
  // the head's output rows; shared by the sub-chunks and the add-back.
  auto raise_max = [&](float mx) {
    if (__ballot(mx > m + tau) != 0ull) {
      const float corr = (mx == -INFINITY) ? 1.f : fast_exp2((m - mx) * cs);
      l *= corr;
      m = mx;
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
  };

  for (int i = 0; i < nsc; ++i) {
    const int c0 = t0 + i * TS, bsel = i % NSUB;
    if (loader) {
      const int ahead = min(nsc, NSUB + max(0, i - 1)) - (i + 1);
      if (wave == 2) vm_wait_ahead<4 * NI + 1, NSUB - 1>(ahead);
      else vm_wait_ahead<4 * NI, NSUB - 1>(ahead);
    } else if (i == 0) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // queries, record, unit words (no store issued yet)
    }
    dma_barrier();  // every wave's rows of sub-chunk i are in; every wave is done with i - 1
    if (loader && i >= 1 && i + NSUB - 1 < nsc) stage(i + NSUB - 1, (i - 1) % NSUB);
    if (i == 0) {
      z = lazy_view_lds(lz);
      lazy = z.flag == 1;
      lazy_over = lazy && z.over != 0;
      query_operand<G>(qb, qs, lz + kLzQ * 4, hl, qd, lazy);
      {
        const int hh = (hl >= G && hl < 2 * G) ? hl - G : 0;
        const float mcv = __uint_as_float(lds_read_b32(lds_addr(lzf + kLzM + hh)));
        const float ilv = __uint_as_float(lds_read_b32(lds_addr(lzf + kLzIL + hh)));
        if (lazy && hl >= G && hl < 2 * G) mc = mcv, il = ilv;
      }
      const u32x4 w4 = lds_read_b128(lds_addr(uw));
      beta = a.budget ? __builtin_amdgcn_readfirstlane((int)w4.y) : a.budget_all;
      const int ldev = __builtin_amdgcn_readfirstlane((int)w4.x);
      const int candn = __builtin_amdgcn_readfirstlane((int)w4.z);
      newest = __builtin_amdgcn_readfirstlane((int)w4.w);
      const int live = Lold + 1 - (lazy_over ? 1 : 0);
      err = (ldev != Lold || candn != 0) ? HIKV_EINVAL
                                         : ((beta < a.n_sink || beta > a.cap) ? HIKV_EBUDGET
                                                                              : ((live - beta > 1) ? HIKV_EINVAL : 0));
    }
    uint64_t rd[12];
    if (bsel == 0) mfma_operands<0, SUBB>(rd, ad);
    else if (bsel == 1) mfma_operands<2 * SUBB, 3 * SUBB>(rd, ad);
    else mfma_operands<4 * SUBB, 5 * SUBB>(rd, ad);
    // Columns < G: this step's raw q.k; columns G .. 2G-1: the deferred step's.
    f32x4_t S = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) S = mfma16(__builtin_bit_cast(bf16x4_t, rd[ks]), qb[ks], S);
    const int nrows = min(TS, t1 - c0);
    const int rowb = grp * 16 + 4 * qd;  // this lane's four token rows in the sub-chunk
    int take = -1;                       // row (in the group) of a token held out in this sub-chunk
    if (lazy) {
      float ip[4], it[4];
      int pp[4];
      bool phys[4], acc[4];
      uint64_t key[4];
      lds_read_ip(ip, pp, ipb_a + (bsel * 64 + rowb) * 4, ipb_a + (bsel * 64 + 32 + rowb) * 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) phys[r] = rowb + r < nrows && c0 + rowb + r != Lold;
      lazy_tokens<G>(S, hl, z, mc, il, ip, pp, phys, it, key, acc);
      // The deferred step's importance of these tokens: the store waves write it.
      if (half == 0 && hl < 4 && !err) {
        const float v = hl == 0 ? it[0] : (hl == 1 ? it[1] : (hl == 2 ? it[2] : it[3]));
        const bool w = hl == 0 ? acc[0] : (hl == 1 ? acc[1] : (hl == 2 ? acc[2] : acc[3]));
        if (w) store_agent_f(impw + c0 + rowb + hl, v);
      }
      if (lazy_over) {
        uint64_t bk;
        int brow;
        group_min_key(key, qd, bk, brow);
        if (bk < hk) {
          if (hk != ~0ull) {
            // The previous held-out token goes back into the softmax.
            raise_max(hl < G ? fmaxf(m, hs) : m);
            const float e = (hl < G) ? fast_exp2((hs - m) * cs) : 0.f;
            if (qd == 0) l += e;
            float fe[4];
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const float fa = lane_value(e, r4 < G ? r4 : G - 1);
              if constexpr (G > 4) {
                const float fb = lane_value(e, 4 + r4);
                fe[r4] = qd == 0 ? fa : fb;
              } else {
                fe[r4] = fa;
              }
            }
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
              for (int r4 = 0; r4 < 4; ++r4) O[t][r4] = fmaf(fe[r4], hv[t], O[t][r4]);
          }
          const int cq = brow >> 2, cr = brow & 3;
          const float sc = cr == 0 ? S[0] : (cr == 1 ? S[1] : (cr == 2 ? S[2] : S[3]));
          hs = __shfl(sc, cq * 16 + hl);
          const uint32_t vrow = lds_addr(smem) + bsel * 2 * SUBB + SUBB;
#pragma unroll
          for (int t = 0; t < 4; ++t) hv[t] = lds_read_bf16(vrow + swz_off(grp * 16 + brow, half * 64 + 16 * t + hl));
          hk = bk;
          hslot = c0 + grp * 16 + brow;
          take = brow;
        }
      }
    }
    float sv[4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int row = rowb + r4;
      sv[r4] = (hl < G && row < nrows && 4 * qd + r4 != take) ? S[r4] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(m, fmaxf(sv[0], sv[1])), fmaxf(sv[2], sv[3]));
    {
      float w2 = mx;
      permlane16_swap(mx, w2);
      mx = fmaxf(mx, w2);
      w2 = mx;
      permlane32_swap(mx, w2);
      mx = fmaxf(mx, w2);
    }
    raise_max(mx);
    const float mcur = (m == -INFINITY) ? 0.f : m * cs;
    float pv[4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      pv[r4] = fast_exp2(fmaf(sv[r4], cs, -mcur));
      l += pv[r4];
    }
    bf16x4_t phi, plo;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      phi[r4] = (__bf16)pv[r4];
      plo[r4] = (__bf16)(pv[r4] - (float)phi[r4]);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16x4_t vb4 = __builtin_bit_cast(bf16x4_t, rd[8 + t]);
      O[t] = mfma16(phi, vb4, O[t]);
      O[t] = mfma16(plo, vb4, O[t]);
    }
    asm volatile("" : "+v"(m), "+v"(l));
    sched_fence();
  }
  // ---- The tile's partial: l over the lane rows of each head; the two token
  // groups of each channel half combined, and the group whose held-out token
  // has the higher key puts it back (the tile holds out only its lowest).
  {
    float w2 = l;
    permlane16_swap(l, w2);
    l += w2;
    w2 = l;
    permlane32_swap(l, w2);
    l += w2;
  }
  lds_barrier();  // the ring becomes merge scratch
  float(*sm_acc)[G][64] = reinterpret_cast<float(*)[G][64]>(smem);
  float(*sm_ml)[G][2] = reinterpret_cast<float(*)[G][2]>(smem + 4 * G * 64 * 4);
  HoldW<G> *hw = reinterpret_cast<HoldW<G> *>(smem + 4 * G * 64 * 4 + 4 * G * 2 * 4);
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
    hw[wave].hs[hl] = hs;
  }
  if (qd == 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) hw[wave].hv[16 * t + hl] = hv[t];
  }
  if (lane == 0) {
    hw[wave].khi = (uint32_t)(hk >> 32);
    hw[wave].klo = (uint32_t)hk;
    hw[wave].slot = hslot;
  }
  lds_barrier();
  const uint64_t k0 = ((uint64_t)hw[0].khi << 32) | hw[0].klo, k1 = ((uint64_t)hw[1].khi << 32) | hw[1].klo;
  const int gs = (k1 < k0) ? 1 : 0, go = 1 - gs;  // group that holds out, group that puts back
  const bool other = (gs == 0 ? k1 : k0) != ~0ull;
  for (int idx = tid; idx < G * D; idx += kFT) {
    const int h = idx / D, ch = idx - h * D, hf = ch >> 6, w0 = 2 * hf, w1 = w0 + 1, wo = 2 * hf + go;
    const float m0 = sm_ml[w0][h][0], m1 = sm_ml[w1][h][0];
    const float so = other ? hw[wo].hs[h] : -INFINITY;
    const float M = fmaxf(fmaxf(m0, m1), so);
    const float Ms = (M == -INFINITY) ? 0.f : M;
    const float e0 = fast_exp2((m0 - Ms) * cs), e1 = fast_exp2((m1 - Ms) * cs);
    const float eo = other ? fast_exp2((so - Ms) * cs) : 0.f;
    const float av = sm_acc[w0][h][ch & 63] * e0 + sm_acc[w1][h][ch & 63] * e1 + eo * hw[wo].hv[ch & 63];
    store_agent_f(a.ws.part_acc + ((size_t)tile * G + h) * D + ch, av);
    if (ch == 0) {
      store_agent_f(a.ws.part_ml + ((size_t)tile * G + h) * 2, M);
      store_agent_f(a.ws.part_ml + ((size_t)tile * G + h) * 2 + 1, sm_ml[w0][h][1] * e0 + sm_ml[w1][h][1] * e1 + eo);
    }
  }
  {
    int32_t *hr = a.ws.hold + (size_t)tile * kHoldWords;
    const uint64_t ks = gs ? k1 : k0;
    if (tid == 0) {
      store_agent(hr + 0, (int32_t)(uint32_t)ks);
      store_agent(hr + 1, (int32_t)(uint32_t)(ks >> 32));
      store_agent(hr + 2, hw[gs].slot);
      store_agent(hr + 3, ks != ~0ull ? 1 : 0);
    }
    if (tid < G) store_agent_f(reinterpret_cast<float *>(hr + 4) + tid, hw[gs].hs[tid]);
    if (tid < 64) {
      // channels 2 tid, 2 tid + 1 of the held-out row: half (2 tid) >> 6 of group gs
      const int c = 2 * tid, w = 2 * (c >> 6) + gs;
      const uint32_t lo = __float_as_uint(hw[w].hv[c & 63]) >> 16, hi = __float_as_uint(hw[w].hv[(c & 63) + 1]) >> 16;
      store_agent(hr + 12 + tid, (int32_t)(lo | (hi << 16)));
    }
  }
  // ---- Ticket: the unit's last tile to arrive combines.  Every store above is
  // device-coherent (write-through) and complete before the count, and the
  // combine reads the other tiles' records with device-coherent loads, so the
  // count needs no cache write-back or invalidation.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) s_last = (int)(ticket_agent(a.ws.ticket + u) + 1 == (uint32_t)pl.nt);
  __syncthreads();
  if (!s_last) return;
  if (tid == 0) store_agent(reinterpret_cast<int32_t *>(a.ws.ticket + u), 0);  // ready for the next step

  // ---- Combine (one workgroup per unit).  Tables in the ring: fac[i][h]
  // the factor of tile i's partial, hfac[i][h] that of its held-out token (0
  // for none and for the victim).
  const int nt = pl.nt, tb = tile - pl.s;
  constexpr int NTAB = fused_max_unit_tiles<G>();
  float *fac = reinterpret_cast<float *>(smem);
  float *hfac = fac + NTAB * G;
  char *red = smem + 2 * NTAB * G * 4;  // reduction scratch (kCombineScratch bytes)
  float *osum = reinterpret_cast<float *>(red);                                  // [256][4] output quads
  float(*rmax)[G] = reinterpret_cast<float(*)[G]>(red + 4096);                   // [4][G]
  float(*rsum)[G] = reinterpret_cast<float(*)[G]>(red + 4096 + 16 * G);          // [4][G]
  uint32_t(*rkey)[4] = reinterpret_cast<uint32_t(*)[4]>(red + 4096 + 32 * G);    // [4]: khi, klo, tile
  float *fin = reinterpret_cast<float *>(red + 4096 + 32 * G + 64);              // [2G]: M, 1/L per head
  static_assert(4096 + 40 * G + 64 <= kCombineScratch, "combine scratch");
  // the victim: lowest held-out key over the unit's tiles
  int vt = -1, vslot = -1;
  if (lazy_over) {
    uint64_t bk = ~0ull;
    int bt = -1;
    for (int i = tid; i < nt; i += kFT) {
      const int32_t *hr = a.ws.hold + (size_t)(tb + i) * kHoldWords;
      const uint64_t k = ((uint64_t)(uint32_t)ld_ag(hr + 1) << 32) | (uint32_t)ld_ag(hr);
      if (ld_ag(hr + 3) && k < bk) bk = k, bt = i;
    }
    wave_min_key(bk, bt);
    if (lane == 0) {
      rkey[wave][0] = (uint32_t)(bk >> 32);
      rkey[wave][1] = (uint32_t)bk;
      rkey[wave][2] = (uint32_t)bt;
    }
    lds_barrier();
    uint64_t best = ~0ull;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint64_t k = ((uint64_t)rkey[w][0] << 32) | rkey[w][1];
      if (k < best) best = k, vt = (int)rkey[w][2];
    }
    if (vt >= 0) vslot = ld_ag(a.ws.hold + (size_t)(tb + vt) * kHoldWords + 2);
  }
  // statistics per head over the tiles' partials and the tokens put back
  float mloc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) mloc[h] = -INFINITY;
  for (int i = tid; i < nt; i += kFT) {
    const int32_t *hr = a.ws.hold + (size_t)(tb + i) * kHoldWords;
    const bool back = i != vt && ld_ag(hr + 3) != 0;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mi = ld_ag(a.ws.part_ml + ((size_t)(tb + i) * G + h) * 2);
      const float si = back ? ld_ag(reinterpret_cast<const float *>(hr + 4) + h) : -INFINITY;
      fac[i * G + h] = mi;
      hfac[i * G + h] = si;
      mloc[h] = fmaxf(mloc[h], fmaxf(mi, si));
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float x = lanes_max<1>(mloc[h]);
    if (lane == 0) rmax[wave][h] = x;
  }
  lds_barrier();
  float Mh[G], lsum[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    Mh[h] = fmaxf(fmaxf(rmax[0][h], rmax[1][h]), fmaxf(rmax[2][h], rmax[3][h]));
    lsum[h] = 0.f;
  }
  for (int i = tid; i < nt; i += kFT) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float Ms = (Mh[h] == -INFINITY) ? 0.f : Mh[h];
      const float li = ld_ag(a.ws.part_ml + ((size_t)(tb + i) * G + h) * 2 + 1);
      const float e = fast_exp2((fac[i * G + h] - Ms) * cs);
      const float si = hfac[i * G + h];
      const float eh = (si == -INFINITY) ? 0.f : fast_exp2((si - Ms) * cs);
      fac[i * G + h] = e;
      hfac[i * G + h] = eh;
      lsum[h] += li * e + eh;
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float x = lanes_sum<1>(lsum[h]);
    if (lane == 0) rsum[wave][h] = x;
  }
  lds_barrier();
  if (tid < G) {
    fin[tid] = Mh[tid];
    fin[G + tid] = 1.f / (rsum[0][tid] + rsum[1][tid] + rsum[2][tid] + rsum[3][tid]);
  }
  __syncthreads();
  // outputs: thread t sums output quad t % NQ over the tiles i = t / NQ (mod TPQ)
  constexpr int NQ = G * D / 4, TPQ = kFT / NQ;
  static_assert(NQ * TPQ == kFT, "output quads split the workgroup evenly");
  {
    const int q = tid % NQ, part = tid / NQ;
    const int h = (4 * q) / D, c4 = (4 * q) % D;
    float4 acc4 = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i = part; i < nt; i += TPQ) {
      const float *pa = a.ws.part_acc + ((size_t)(tb + i) * G + h) * D + c4;
      const int32_t *hv2 = a.ws.hold + (size_t)(tb + i) * kHoldWords + 12 + c4 / 2;
      const float e = fac[i * G + h], eh = hfac[i * G + h];
      const uint32_t w0 = (uint32_t)ld_ag(hv2), w1 = (uint32_t)ld_ag(hv2 + 1);
      acc4.x = fmaf(ld_ag(pa + 0), e, fmaf(__uint_as_float(w0 << 16), eh, acc4.x));
      acc4.y = fmaf(ld_ag(pa + 1), e, fmaf(__uint_as_float(w0 & 0xffff0000u), eh, acc4.y));
      acc4.z = fmaf(ld_ag(pa + 2), e, fmaf(__uint_as_float(w1 << 16), eh, acc4.z));
      acc4.w = fmaf(ld_ag(pa + 3), e, fmaf(__uint_as_float(w1 & 0xffff0000u), eh, acc4.w));
    }
    reinterpret_cast<float4 *>(osum)[tid] = acc4;
  }
  __syncthreads();
  float *outu = a.out + (size_t)(b * a.Hq + j * G) * D;
  if (tid < NQ) {
    float4 s = reinterpret_cast<float4 *>(osum)[tid];
    for (int p = 1; p < TPQ; ++p) {
      const float4 x = reinterpret_cast<float4 *>(osum)[tid + p * NQ];
      s.x += x.x, s.y += x.y, s.z += x.z, s.w += x.w;
    }
    const int h = (4 * tid) / D;
    const float il_h = fin[G + h];
    float4 o = make_float4(s.x * il_h, s.y * il_h, s.z * il_h, s.w * il_h);
    if (err) o = make_float4(0.f, 0.f, 0.f, 0.f);
    reinterpret_cast<float4 *>(outu)[tid] = o;
  }
  if (err) {
    if (tid == 0) set_status(a.ws.status, err);
    return;
  }
  // ---- The new token: into the victim's slot, or appended.  The deferred
  // record then describes this step.
  int slot = Lold;
  if (lazy_over) {
    if (vslot >= 0) slot = vslot;
    else if (tid == 0) set_status(a.ws.status, HIKV_EINVAL);  // no candidate: positions not distinct
  }
  char *kw = static_cast<char *>(a.k_w) + (size_t)u * a.cap * RB;
  char *vw = static_cast<char *>(a.v_w) + (size_t)u * a.cap * RB;
  if (tid < 2 * (RB / 16)) {
    const int half_r = tid / (RB / 16), piece = tid % (RB / 16);
    const uint4 x = reinterpret_cast<const uint4 *>(half_r ? vn : kn)[piece];
    reinterpret_cast<uint4 *>((half_r ? vw : kw) + (size_t)slot * RB)[piece] = x;
  }
  const int len_after = (slot == Lold) ? Lold + 1 : Lold;
  if (tid == 0) {
    posw[slot] = newest;
    impw[slot] = 0.f;
    if (slot == Lold) a.len[u] = len_after;
    lrec[kLzFlag] = 1;
    lrec[kLzOver] = len_after > beta ? 1 : 0;
    lrec[kLzNewest] = newest;
    lrec[kLzWp] = min(a.n_recent, beta - a.n_sink);
    lrec[kLzSink] = a.n_sink;
    lrec[kLzAcc] = a.acc_logit ? HIKV_ACC_LOGIT : (a.acc_recent ? HIKV_ACC_RECENT : HIKV_ACC_ALL);
    lrec[kLzCs] = __float_as_int(cs);
  }
  if (tid < G) {
    reinterpret_cast<float *>(lrec)[kLzM + tid] = fin[tid] * cs;
    reinterpret_cast<float *>(lrec)[kLzIL + tid] = fin[G + tid];
  }
  if (tid < QB / 16) reinterpret_cast<uint4 *>(lrec + kLzQ)[tid] = reinterpret_cast<const uint4 *>(qs)[tid];
}

// ---------------------------------------------------------------------------
// Resolution of a cache's deferred state, one workgroup per unit: the
// deferred step's probabilities are added to the importance (the same
// arithmetic as the fused step's tiles), its victim is found and, with
// apply, the unit's last slot moves into the victim's and len drops by one.
// slot_out (optional) gets the victim (-1: none).  A unit whose record holds
// no deferred step falls back to the two-launch step's candidate form.
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(kFT) void k_settle_lazy(StepArgs a, int32_t *slot_out, int apply) {
  constexpr int D = 128, RB = 256, SUBB = 8192, QB = G * D * 2, LZB = kLzQ * 4 + QB;
  __shared__ __attribute__((aligned(16))) char kb[2 * SUBB];  // two 32-row sub-chunks of K
  __shared__ __attribute__((aligned(16))) int32_t ipb[2][64];
  __shared__ __attribute__((aligned(16))) char lz[LZB];
  __shared__ uint32_t rkey[4][3];
  __shared__ float s_last_imp;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int u = blockIdx.x;
  int32_t *lrec = a.evict + (size_t)u * a.state_stride + state_words(a.cap);
  if (lrec[kLzFlag] != 1) {
    // the two-launch step's form, resolved by one wave
    if (wave == 0) {
      if (slot_out) {
        const int d = pending_slot_wave(a, u);
        if (lane == 0) slot_out[u] = d;
      }
      if (apply) settle_unit(a, u, RB);
    }
    return;
  }
  for (int i = tid; i < LZB / 16; i += kFT)
    reinterpret_cast<uint4 *>(lz)[i] = reinterpret_cast<const uint4 *>(lrec)[i];
  __syncthreads();
  const LazyView z = lazy_view(reinterpret_cast<const int32_t *>(lz));
  const int len = __builtin_amdgcn_readfirstlane(a.len[u]);
  const int hl = lane & 15, qd = lane >> 4, grp = wave & 1, sc = wave >> 1;
  bf16x4_t qb[8];
  query_operand<G>(qb, nullptr, lz + kLzQ * 4, hl, qd, true);
  const float *lzf = reinterpret_cast<const float *>(lz);
  float mc = 0.f, il = 0.f;
  if (hl >= G && hl < 2 * G) {
    mc = lzf[kLzM + hl - G];
    il = lzf[kLzIL + hl - G];
  }
  uint32_t ad[12];
  {
    const uint32_t base = lds_addr(kb);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) ad[ks] = base + swz_off(grp * 16 + hl, 16 * ks + 4 * qd);
#pragma unroll
    for (int t = 0; t < 4; ++t) ad[8 + t] = 0;
  }
  const char *kc = static_cast<const char *>(a.k_cache) + (size_t)u * a.cap * RB;
  float *impw = a.imp + (size_t)u * a.cap;
  const int32_t *posw = a.pos + (size_t)u * a.cap;
  uint64_t best = ~0ull;
  int best_slot = -1;
  for (int c0 = 0; c0 < len; c0 += 64) {
    // stage rows c0 .. c0+63 (clamped): 16 pieces of 1 KB, four per wave, swizzled as the ring
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int piece = p * 4 + wave;
      const int off = (piece << 10) + (lane << 4);
      const int row = off / RB;  // 0 .. 63
      const int col = (((off - row * RB) >> 4) ^ (row & 15)) << 4;
      const int n = min(c0 + row, len - 1);
      __builtin_amdgcn_global_load_lds(kc + (size_t)n * RB + col, kb + (piece << 10), 16, 0, 0);
    }
    if (wave < 2) {
      const int n = min(c0 + 32 * wave + (lane & 31), len - 1);
      const void *src = lane < 32 ? static_cast<const void *>(impw + n) : static_cast<const void *>(posw + n);
      __builtin_amdgcn_global_load_lds(src, &ipb[wave][0], 4, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    uint64_t kr[8];
    mfma_k_operand(kr, ad, (uint32_t)(sc * SUBB));
    f32x4_t S = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) S = mfma16(__builtin_bit_cast(bf16x4_t, kr[ks]), qb[ks], S);
    const int rowb = grp * 16 + 4 * qd, cb = c0 + 32 * sc;
    float ip[4], it[4];
    int pp[4];
    bool phys[4], acc[4];
    uint64_t key[4];
    lds_read_ip(ip, pp, lds_addr(&ipb[sc][rowb]), lds_addr(&ipb[sc][32 + rowb]));
#pragma unroll
    for (int r = 0; r < 4; ++r) phys[r] = cb + rowb + r < len;
    lazy_tokens<G>(S, hl, z, mc, il, ip, pp, phys, it, key, acc);
    if (hl < 4) {
      const float v = hl == 0 ? it[0] : (hl == 1 ? it[1] : (hl == 2 ? it[2] : it[3]));
      const bool w = hl == 0 ? acc[0] : (hl == 1 ? acc[1] : (hl == 2 ? acc[2] : acc[3]));
      const int n = cb + rowb + hl;
      if (apply && w) impw[n] = v;
      if (n == len - 1 && phys[hl]) s_last_imp = v;
    }
    uint64_t bk;
    int brow;
    group_min_key(key, qd, bk, brow);
    if (bk < best) best = bk, best_slot = cb + grp * 16 + brow;
    __syncthreads();  // before the next rows land in the buffers
  }
  if (lane == 0) {
    rkey[wave][0] = (uint32_t)(best >> 32);
    rkey[wave][1] = (uint32_t)best;
    rkey[wave][2] = (uint32_t)best_slot;
  }
  __syncthreads();
  uint64_t vk = ~0ull;
  int vslot = -1;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint64_t k = ((uint64_t)rkey[w][0] << 32) | rkey[w][1];
    if (k < vk) vk = k, vslot = (int)rkey[w][2];
  }
  if (!z.over) vslot = -1;
  if (slot_out && tid == 0) slot_out[u] = vslot;
  if (!apply) return;
  if (vslot >= 0 && wave == 0) {
    const int last = len - 1;
    if (vslot != last) {
      char *kw = static_cast<char *>(a.k_w) + (size_t)u * a.cap * RB;
      char *vw = static_cast<char *>(a.v_w) + (size_t)u * a.cap * RB;
      char *base = lane < 16 ? kw : vw;
      const int off = (lane % 16) * 16;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (lane < 32) x = *reinterpret_cast<const uint4 *>(base + (size_t)last * RB + off);
      const int32_t p = posw[last];
      if (lane < 32) *reinterpret_cast<uint4 *>(base + (size_t)vslot * RB + off) = x;
      if (lane == 0) {
        a.pos[(size_t)u * a.cap + vslot] = p;
        impw[vslot] = s_last_imp;
      }
    }
    if (lane == 0) a.len[u] = last;
  }
  if (tid == 0) lrec[kLzFlag] = 0;
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
template <int G>
static int fused_grid_g() {
  static int per_cu_cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int &pc = per_cu_cache[dev];
  if (pc == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_step_fused<G>, kFT, 0) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    pc = per_cu * cus;
  }
  return min(pc, kMaxGrid);
}

int fused_grid(int G) {
  switch (G) {
    case 1: return fused_grid_g<1>();
    case 2: return fused_grid_g<2>();
    case 4: return fused_grid_g<4>();
    case 8: return fused_grid_g<8>();
    default: return 0;
  }
}

int fused_max_tiles(int G) {
  switch (G) {
    case 1: return fused_max_unit_tiles<1>();
    case 2: return fused_max_unit_tiles<2>();
    case 4: return fused_max_unit_tiles<4>();
    case 8: return fused_max_unit_tiles<8>();
    default: return 0;
  }
}

template <int G>
static hipError_t fused_go(const StepArgs &a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  const dim3 grid((unsigned)a.hp.ntiles), block(kFT);
  if (ev0 && ev1) hipExtLaunchKernelGGL(k_step_fused<G>, grid, block, 0, s, ev0, ev1, 0, a);
  else hipLaunchKernelGGL(k_step_fused<G>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fused_step(const StepArgs &a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  switch (a.G) {
    case 1: return fused_go<1>(a, s, ev0, ev1);
    case 2: return fused_go<2>(a, s, ev0, ev1);
    case 4: return fused_go<4>(a, s, ev0, ev1);
    case 8: return fused_go<8>(a, s, ev0, ev1);
    default: return hipErrorInvalidValue;
  }
}

template <int G>
static hipError_t settle_lazy_go(const StepArgs &a, int32_t *slot_out, bool apply, hipStream_t s) {
  hipLaunchKernelGGL(k_settle_lazy<G>, dim3((unsigned)a.n_units), dim3(kFT), 0, s, a, slot_out, apply ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_settle_lazy(const StepArgs &a, int32_t *slot_out, bool apply, hipStream_t s) {
  switch (a.G) {
    case 1: return settle_lazy_go<1>(a, slot_out, apply, s);
    case 2: return settle_lazy_go<2>(a, slot_out, apply, s);
    case 4: return settle_lazy_go<4>(a, slot_out, apply, s);
    case 8: return settle_lazy_go<8>(a, slot_out, apply, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hikv
