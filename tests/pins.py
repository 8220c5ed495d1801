"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each check raises AssertionError on a violation.  They are run against the
real oracle (test_oracle_pins.py) and against deliberately broken copies of
it (test_oracle_mutants.py), which every one of a set of plausible mistakes
must trip.

What pins what:
  attention_matches_library   -- output = torch's scaled_dot_product_attention
      (a library routine) when nothing is evicted, including the appended
      token attending to itself and the GQA head grouping; the importance a
      step adds = the library's attention weights (obtained as SDPA with
      V = identity), summed over the group.
  rows_sum_to_group           -- softmax rows sum to one: a step adds exactly
      G to a unit's importance.
  streaming_closed_form       -- budget = S + W keeps exactly the first S and
      last W positions, whatever the scores (StreamingLLM set formula).
  eviction_brute_force        -- on tiny caches, the kept set is the unique
      subset (containing the protected tokens) in which every kept candidate
      outranks every evicted one; it also maximises the kept importance.
  golden_cases                -- hand-worked cases in tests/golden.
  permutation_invariance      -- permuting cache slots leaves the output and
      the kept position set unchanged (Kelle: order of [k, v] pairs).
  channel_permutation         -- one channel permutation applied to q and K,
      another to V, permutes the output the same way.
  conservation                -- over a run with eviction, live + evicted
      importance = G * steps.
  stage2_reduces_to_stage1    -- r = D and k_T >= len gives Stage I exactly.
  stage2_selection            -- chosen channels = brute-force top-r of |q|
      (ties: lower index); approximate importance = library attention
      weights of the masked query; output = library attention over the
      chosen tokens.
  equal_keys_closed_form      -- all keys equal: uniform softmax, output =
      mean of the values, each token gains G/L; Stage II's exact set is the
      k_T lowest positions (tie rule).
  prefill_column_sums         -- window 0 with every prompt query = column
      sums of the library's causal attention matrix; window W = its banded
      sums; one query = its softmax row.
  errors_leave_unit_unchanged -- capacity and budget errors.
  heap_worked_examples        -- the model of HiKV's vectorized min-heap
      reproduces the pages' printed HEAPIFY_UP example and the first part
      of the HEAPIFY_DOWN example (tests/golden/hikv_heap_examples.txt).
  heap_keeps_the_top_scores   -- that heap, fed any sequence of ejected
      tokens, holds the top-K of every score it was offered, evicts its
      minimum, stays well formed and touches at most one node per level.
  dual_bank_matches_its_definition -- HiKV's dual bank: after a windowed
      prefill and the bank initialisation, every live token's score is the
      sum of the library's attention weights over the W' steps from its own
      (partial inside the window); the kept set is the sinks, the window and
      the top scores of every token that has left the window (brute force);
      the heap model fed the same ejections holds the same bank.
  stage2_chunks_reduce_to_attention -- HiKV's chunked V side with r = D
      (every channel; every chunk keeps all its entries) is exact attention:
      the library's SDPA.
  stage2_chunks_select_by_probability -- with V rows one-hot by position
      rank, the output reads back what each chunk of D consecutive positions
      kept: min(r, chunk size) entries, equal to the library's softmax of the
      channel-masked query (no renormalisation), none smaller than an entry
      the chunk dropped; permuting the slots changes nothing.
  logit_accumulation_matches_library -- Kelle's importance (accumulate =
      LOGIT): a step adds the group's pre-softmax logits scale * q.k (a
      library matmul; with Stage II on, of the channel-masked query) to every
      live token, and the kept set is the brute-force one for that importance.
  snapkv_pooling_matches_library -- pool = k: every token gains the largest
      of the observation scores (library attention weights) over positions
      p .. p+k-1, computed as a sliding-window maximum (numpy) over the
      position axis with absent positions at -inf; slots shuffled, positions
      with gaps.
"""

from __future__ import annotations

import itertools
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

from importance_aware_kv_amd import workloads as W
from oracle import hikv_heap as HP
from oracle import ref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def widen(a, dtype):
    if dtype == W.BF16:
        return W.bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def sdpa(q, k, v, scale, mask=None):
    """Library attention in float64: q [Hq, n, D], k [Hk, L, D], v [Hk, L, Dv]."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))[None]
    m = None if mask is None else torch.from_numpy(mask)[None]
    o = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m, scale=scale,
                                       enable_gqa=True)
    return o[0].numpy()


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.abs(b).max(), 1e-300)
    return float(np.abs(a - b).max() / den)


def _unit_rows(state, b, j, dtype):
    n = int(state["len"][b, j])
    return (widen(state["k"][b, j, :n], dtype), widen(state["v"][b, j, :n], dtype),
            state["pos"][b, j, :n].copy(), state["imp"][b, j, :n].astype(np.float64))


def attention_matches_library(seed=1, dtype=W.BF16):
    B, Hkv, G, D, cap = 2, 3, 3, 16, 40
    Hq = Hkv * G
    lens = np.array([[0, 7, 23], [1, 38, 12]], dtype=np.int32)
    st = W.random_cache(seed, B, Hq, Hkv, D, dtype, cap, lens)
    step = W.random_step(seed + 1, B, Hq, Hkv, D, dtype, st["newest"])
    before = ref.copy_state(st)
    scale = 1.0 / math.sqrt(D)
    code, out, dbg = ref.decode_step(st, Hq, step["q"], step["k_new"], step["v_new"],
                                     step["new_pos"], budget_all=cap, n_sink=2, n_recent=3)
    assert code == 0
    for b in range(B):
        for j in range(Hkv):
            k, v, pos, imp = _unit_rows(before, b, j, dtype)
            k = np.concatenate([k, widen(step["k_new"][b, j], dtype)[None]])
            v = np.concatenate([v, widen(step["v_new"][b, j], dtype)[None]])
            q = widen(step["q"][b, j * G:(j + 1) * G], dtype)[:, None, :]
            want = sdpa(q, k[None], v[None], scale)[:, 0, :]
            got = out[b, j * G:(j + 1) * G]
            assert rel_err(got, want) < 2e-7, ("output", b, j, rel_err(got, want))
            L = k.shape[0]
            P = sdpa(q, k[None], np.eye(L)[None], scale)[:, 0, :]   # [G, L] weights
            added = dbg["imp_pre_evict"][b, j, :L].astype(np.float64) - np.append(imp, 0.0)
            assert np.abs(added - P.sum(0)).max() < 1e-6 * max(1.0, np.abs(imp).max(initial=0.0)), \
                ("importance increment", b, j)
            # nothing evicted: every position is still there
            assert sorted(ref.live_positions(st, b, j)) == sorted(np.append(pos, st["newest"]))


def rows_sum_to_group(seed=3):
    B, Hkv, G, D, cap = 2, 2, 4, 32, 64
    Hq = Hkv * G
    st = W.random_cache(seed, B, Hq, Hkv, D, W.BF16, cap, [[10, 40], [63 - 1, 3]])
    step = W.random_step(seed + 1, B, Hq, Hkv, D, W.BF16, st["newest"])
    code, _, dbg = ref.decode_step(st, Hq, step["q"], step["k_new"], step["v_new"],
                                   step["new_pos"], budget_all=20, n_sink=4, n_recent=4)
    assert code == 0
    assert np.abs(dbg["prob_sum"] - G).max() < 1e-12


def streaming_closed_form(seed=5, steps=12):
    w = W.workload("tiny", ctx=48, steps=steps)
    d = W.generate(w)
    st = ref.copy_state(d)
    S, R = 3, 5
    for t in range(steps):
        code, _, _ = ref.decode_step(st, w.n_q_heads, d["q"][t], d["k_new"][t], d["v_new"][t],
                                     d["new_pos"][t], budget_all=S + R, n_sink=S, n_recent=R)
        assert code == 0
        newest = int(d["new_pos"][t, 0])
        want = sorted(set(range(S)) | set(range(newest - R + 1, newest + 1)))
        assert list(ref.live_positions(st, 0, 0)) == want, (t, list(ref.live_positions(st, 0, 0)))


def _brute_kept(pos, imp, beta, S, R, newest):
    L = len(pos)
    if L <= beta:
        return set(pos.tolist())
    Wp = min(R, beta - S)
    prot = [i for i in range(L) if pos[i] < S or pos[i] > newest - Wp]
    cand = [i for i in range(L) if i not in prot]
    need = beta - len(prot)

    def outranks(a, b):
        return imp[a] > imp[b] or (imp[a] == imp[b] and pos[a] < pos[b])

    valid = []
    best = -1.0
    best_sets = []
    for sub in itertools.combinations(cand, need):
        s = set(sub)
        rest = [c for c in cand if c not in s]
        if all(outranks(a, b) for a in sub for b in rest):
            valid.append(s)
        tot = sum(float(imp[i]) for i in sub)
        if tot > best + 1e-12:
            best, best_sets = tot, [s]
        elif abs(tot - best) <= 1e-12:
            best_sets.append(s)
    assert len(valid) == 1, "brute force: a strict total order has exactly one valid split"
    assert valid[0] in best_sets, "brute force: the valid split maximises kept importance"
    return set(int(pos[i]) for i in prot) | set(int(pos[i]) for i in valid[0])


def eviction_brute_force(seed=7, trials=150):
    rng = np.random.Generator(np.random.PCG64(seed))
    for t in range(trials):
        L = int(rng.integers(1, 13))
        beta = int(rng.integers(0, 8))
        S = int(rng.integers(0, 3))
        R = int(rng.integers(0, 4))
        if beta < S:
            beta = S
        cap = 16
        newest = L + int(rng.integers(0, 3))
        pos = rng.permutation(np.arange(newest + 1))[:L].astype(np.int32)
        pos[rng.integers(0, L)] = newest  # the newest token is live
        pos = np.unique(pos)
        rng.shuffle(pos)
        L = len(pos)
        imp = (rng.integers(0, 4, size=L) / 4.0).astype(np.float32)  # many ties
        st = dict(k=np.zeros((1, 1, cap, 4), np.float32), v=np.zeros((1, 1, cap, 4), np.float32),
                  pos=np.full((1, 1, cap), -1, np.int32), imp=np.zeros((1, 1, cap), np.float32),
                  len=np.array([[L]], np.int32))
        st["pos"][0, 0, :L] = pos
        st["imp"][0, 0, :L] = imp
        st["k"][0, 0, :L, 0] = pos  # payload follows its token
        code, dbg = ref.evict(st, 1, [newest], budget_all=beta, n_sink=S, n_recent=R)
        assert code == 0
        want = _brute_kept(pos, imp.astype(np.float64), beta, S, R, newest)
        got = set(ref.live_positions(st, 0, 0).tolist())
        assert got == want, (t, sorted(got), sorted(want), beta, S, R)
        n = int(st["len"][0, 0])
        assert n == min(L, beta)
        assert np.all(st["k"][0, 0, :n, 0] == st["pos"][0, 0, :n])
        kept_slots = set(np.nonzero(dbg["kept"][0, 0, :L])[0].tolist())
        assert set(int(pos[i]) for i in kept_slots) == want


def read_golden(name="evict_cases.txt"):
    cases = []
    cur = None
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, rest = line.partition(" ")
        if key == "case":
            cur = dict(name=rest)
            cases.append(cur)
        elif key == "tokens":
            pairs = [tok.split(":") for tok in rest.split()]
            cur["pos"] = np.array([int(p) for p, _ in pairs], np.int32)
            cur["imp"] = np.array([float(v) for _, v in pairs], np.float32)
        elif key == "kept":
            cur["kept"] = sorted(int(x) for x in rest.split())
        else:
            cur[key] = int(rest)
    return cases


def golden_cases():
    for c in read_golden():
        L = len(c["pos"])
        cap = max(L, c["budget"]) + 1
        st = dict(k=np.zeros((1, 1, cap, 4), np.float32), v=np.zeros((1, 1, cap, 4), np.float32),
                  pos=np.full((1, 1, cap), -1, np.int32), imp=np.zeros((1, 1, cap), np.float32),
                  len=np.array([[L]], np.int32))
        st["pos"][0, 0, :L] = c["pos"]
        st["imp"][0, 0, :L] = c["imp"]
        code, _ = ref.evict(st, 1, [c["newest"]], budget_all=c["budget"], n_sink=c["sink"],
                            n_recent=c["recent"])
        assert code == 0, c["name"]
        got = list(ref.live_positions(st, 0, 0))
        assert got == c["kept"], (c["name"], got, c["kept"])


def permutation_invariance(seed=11):
    B, Hkv, G, D, cap = 1, 2, 2, 16, 32
    Hq = Hkv * G
    st = W.random_cache(seed, B, Hq, Hkv, D, W.F32, cap, [[25, 30]], shuffle_pos=False)
    step = W.random_step(seed + 1, B, Hq, Hkv, D, W.F32, st["newest"])
    a = ref.copy_state(st)
    b_ = ref.copy_state(st)
    rng = np.random.Generator(np.random.PCG64(seed + 2))
    for j in range(Hkv):
        n = int(st["len"][0, j])
        perm = rng.permutation(n)
        for f in ("k", "v", "pos", "imp"):
            b_[f][0, j, :n] = st[f][0, j, :n][perm]
    kw = dict(budget_all=20, n_sink=2, n_recent=3)
    _, oa, _ = ref.decode_step(a, Hq, step["q"], step["k_new"], step["v_new"], step["new_pos"], **kw)
    _, ob, _ = ref.decode_step(b_, Hq, step["q"], step["k_new"], step["v_new"], step["new_pos"], **kw)
    assert rel_err(oa, ob) < 1e-6
    for j in range(Hkv):
        ra, rb = ref.live_rows(a, 0, j), ref.live_rows(b_, 0, j)
        assert set(ra) == set(rb)
        for p in ra:
            assert ra[p][0] == rb[p][0] and ra[p][1] == rb[p][1]
            assert abs(ra[p][2] - rb[p][2]) <= 1e-6 * max(1.0, abs(ra[p][2]))


def channel_permutation(seed=13):
    B, Hkv, G, D, cap = 1, 1, 3, 16, 24
    Hq = Hkv * G
    st = W.random_cache(seed, B, Hq, Hkv, D, W.F32, cap, [[20]])
    step = W.random_step(seed + 1, B, Hq, Hkv, D, W.F32, st["newest"])
    rng = np.random.Generator(np.random.PCG64(seed + 2))
    pk, pv = rng.permutation(D), rng.permutation(D)
    a = ref.copy_state(st)
    b_ = ref.copy_state(st)
    b_["k"] = np.ascontiguousarray(b_["k"][..., pk])
    b_["v"] = np.ascontiguousarray(b_["v"][..., pv])
    kw = dict(budget_all=cap, n_sink=0, n_recent=0)
    _, oa, _ = ref.decode_step(a, Hq, step["q"], step["k_new"], step["v_new"], step["new_pos"], **kw)
    _, ob, _ = ref.decode_step(b_, Hq, np.ascontiguousarray(step["q"][..., pk]),
                               np.ascontiguousarray(step["k_new"][..., pk]),
                               np.ascontiguousarray(step["v_new"][..., pv]), step["new_pos"], **kw)
    assert rel_err(ob, oa[..., pv]) < 1e-6


def conservation(seed=17, steps=40):
    w = W.workload("llama8b", ctx=96, steps=steps, batch=1)
    w.n_q_heads, w.n_kv_heads = 4, 2
    d = W.generate(w)
    st = ref.copy_state(d)
    G = w.group
    evicted = np.zeros((w.batch, w.n_kv_heads))
    for t in range(steps):
        code, _, dbg = ref.decode_step(st, w.n_q_heads, d["q"][t], d["k_new"][t], d["v_new"][t],
                                       d["new_pos"][t], budget_all=40, n_sink=4, n_recent=8)
        assert code == 0
        gone = (dbg["kept"] == 0) & ~np.isnan(dbg["imp_pre_evict"])
        evicted += np.where(gone, dbg["imp_pre_evict"], 0.0).sum(-1)
    live = np.array([[st["imp"][b, j, :st["len"][b, j]].astype(np.float64).sum()
                      for j in range(w.n_kv_heads)] for b in range(w.batch)])
    assert np.abs(live + evicted - G * steps).max() < 1e-4 * G * steps
    assert np.all(st["len"] == 40)


def stage2_reduces_to_stage1(seed=19):
    B, Hkv, G, D, cap = 2, 2, 2, 16, 40
    Hq = Hkv * G
    st = W.random_cache(seed, B, Hq, Hkv, D, W.BF16, cap, [[30, 12], [5, 33]])
    step = W.random_step(seed + 1, B, Hq, Hkv, D, W.BF16, st["newest"])
    a, b_ = ref.copy_state(st), ref.copy_state(st)
    kw = dict(budget_all=16, n_sink=2, n_recent=4)
    _, oa, _ = ref.decode_step(a, Hq, step["q"], step["k_new"], step["v_new"], step["new_pos"], **kw)
    _, ob, _ = ref.decode_step(b_, Hq, step["q"], step["k_new"], step["v_new"], step["new_pos"],
                               stage2_channels=D, stage2_tokens=cap, **kw)
    assert rel_err(ob, oa) < 1e-6
    for b in range(B):
        for j in range(Hkv):
            assert list(ref.live_positions(a, b, j)) == list(ref.live_positions(b_, b, j))


def stage2_selection(seed=23):
    B, Hkv, G, D, cap = 1, 2, 2, 32, 48
    Hq = Hkv * G
    r, kT = 8, 10
    st = W.random_cache(seed, B, Hq, Hkv, D, W.BF16, cap, [[40, 6]])
    step = W.random_step(seed + 1, B, Hq, Hkv, D, W.BF16, st["newest"])
    # force ties in |q|: quantise to a coarse grid (the stored bf16 stays exact)
    qf = np.round(W.bf16_bits_to_f32(step["q"]) * 2.0) / 2.0
    step["q"] = W.bf16_bits(qf.astype(np.float32))
    before = ref.copy_state(st)
    scale = 1.0 / math.sqrt(D)
    code, out, dbg = ref.decode_step(st, Hq, step["q"], step["k_new"], step["v_new"],
                                     step["new_pos"], budget_all=cap, stage2_channels=r,
                                     stage2_tokens=kT)
    assert code == 0
    for j in range(Hkv):
        k, v, pos, imp = _unit_rows(before, 0, j, W.BF16)
        k = np.concatenate([k, widen(step["k_new"][0, j], W.BF16)[None]])
        v = np.concatenate([v, widen(step["v_new"][0, j], W.BF16)[None]])
        pos = np.append(pos, st["newest"])
        L = k.shape[0]
        add = np.zeros(L)
        for g in range(G):
            h = j * G + g
            q = widen(step["q"][0, h], W.BF16)
            order = np.lexsort((np.arange(D), -np.abs(q)))   # |q| desc, index asc
            E = np.sort(order[:r])
            assert list(dbg["sel_channels"][0, h]) == list(E), ("channels", h)
            qm = np.where(np.isin(np.arange(D), E), q, 0.0)
            Pt = sdpa(qm[None, None], k[None], np.eye(L)[None], scale)[0, 0]
            add += Pt
            tord = np.lexsort((pos, -Pt))                    # approx score desc, pos asc
            T = tord[:min(kT, L)]
            assert list(dbg["sel_tokens"][0, h, :len(T)]) == sorted(pos[T].tolist()), ("tokens", h)
            want = sdpa(q[None, None], k[T][None], v[T][None], scale)[0, 0]
            assert rel_err(out[0, h], want) < 2e-7, ("output", h)
        got = dbg["imp_pre_evict"][0, j, :L].astype(np.float64) - np.append(imp, 0.0)
        assert np.abs(got - add).max() < 1e-6 * max(1.0, np.abs(imp).max(initial=0.0))


def equal_keys_closed_form(seed=37):
    """All keys equal -> uniform softmax: output = mean of the values attended,
    each token gains G/L; Stage II's exact set = the k_T lowest positions."""
    B, Hkv, G, D, cap = 1, 1, 2, 16, 32
    Hq = Hkv * G
    st = W.random_cache(seed, B, Hq, Hkv, D, W.F32, cap, [[20]])
    step = W.random_step(seed + 1, B, Hq, Hkv, D, W.F32, st["newest"])
    st["k"][0, 0, :] = step["k_new"][0, 0]
    for stage2 in (False, True):
        a = ref.copy_state(st)
        before = ref.copy_state(st)
        kT = 7
        kw = dict(stage2_channels=5, stage2_tokens=kT) if stage2 else {}
        code, out, dbg = ref.decode_step(a, Hq, step["q"], step["k_new"], step["v_new"],
                                         step["new_pos"], budget_all=cap, **kw)
        assert code == 0
        L = 21
        pos = np.append(before["pos"][0, 0, :20], st["newest"])
        v = np.concatenate([before["v"][0, 0, :20], step["v_new"][0, 0][None]]).astype(np.float64)
        rows = np.argsort(pos)[:kT] if stage2 else np.arange(L)
        want = v[rows].mean(0)
        for g in range(G):
            assert rel_err(out[0, g], want) < 1e-6, (stage2, g)
        added = dbg["imp_pre_evict"][0, 0, :L].astype(np.float64) - np.append(before["imp"][0, 0, :20], 0)
        assert np.abs(added - G / L).max() < 1e-6
        if stage2:
            for g in range(G):
                assert list(dbg["sel_tokens"][0, g, :kT]) == sorted(pos)[:kT]


def prefill_column_sums(seed=29):
    B, Hkv, G, D = 1, 2, 2, 16
    Hq = Hkv * G
    L = 24
    rng = np.random.Generator(np.random.PCG64(seed))
    k = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    qo = rng.standard_normal((B, Hq, L, D)).astype(np.float32)
    scale = 1.0 / math.sqrt(D)
    mask = np.tril(np.ones((L, L), dtype=bool))
    P = np.stack([sdpa(qo[0, h][None], k[0, h // G][None], np.eye(L)[None], scale, mask)[0]
                  for h in range(Hq)])                       # [Hq, query, token]
    perm = rng.permutation(L)                                # slots in shuffled order
    for window, n_obs_sel in ((0, slice(None)), (5, slice(None)), (0, slice(L - 1, L))):
        st = dict(k=np.ascontiguousarray(k[:, :, perm]), v=np.zeros_like(k),
                  pos=np.ascontiguousarray(np.broadcast_to(perm.astype(np.int32), (B, Hkv, L))),
                  imp=np.zeros((B, Hkv, L), np.float32), len=np.full((B, Hkv), L, np.int32))
        qsel = np.ascontiguousarray(qo[:, :, n_obs_sel])
        qpos = np.arange(L, dtype=np.int32)[n_obs_sel][None].copy()
        code = ref.prefill_scores(st, Hq, qsel, qpos, window=window)
        assert code == 0
        qi = np.arange(L)[n_obs_sel]
        for j in range(Hkv):
            want = np.zeros(L)
            for g in range(G):
                Pq = P[j * G + g][qi]                         # [n_obs, token]
                if window > 0:
                    band = (qi[:, None] - np.arange(L)[None, :] < window)
                    Pq = Pq * band
                want += Pq.sum(0)
            got = np.zeros(L)
            got[st["pos"][0, j]] = st["imp"][0, j]
            assert np.abs(got - want).max() < 1e-5, (window, j)


def errors_leave_unit_unchanged(seed=31):
    B, Hkv, G, D, cap = 1, 2, 1, 8, 10
    st = W.random_cache(seed, B, G * Hkv, Hkv, D, W.F32, cap, [[10, 4]])
    step = W.random_step(seed + 1, B, G * Hkv, Hkv, D, W.F32, st["newest"])
    before = ref.copy_state(st)
    code, out, _ = ref.decode_step(st, G * Hkv, step["q"], step["k_new"], step["v_new"],
                                   step["new_pos"], budget_all=8, n_sink=2, n_recent=2)
    assert code == -4                       # unit 0 is full
    for f in ("k", "v", "pos", "imp"):
        assert np.array_equal(st[f][0, 0], before[f][0, 0])
    assert st["len"][0, 0] == 10 and st["len"][0, 1] == 5
    assert np.all(out[0, 0] == 0)
    st2 = ref.copy_state(before)
    code, _, _ = ref.decode_step(st2, G * Hkv, step["q"], step["k_new"], step["v_new"],
                                 step["new_pos"], budget=np.array([[8, 1]]), n_sink=2, n_recent=0)
    assert code == -4  # first error wins (unit 0 capacity); unit 1 budget < sinks
    assert st2["len"][0, 1] == 4
    bad = ref.Shape(1, 3, 2, 8, 10, 0, 0.0)  # Hq not a multiple of Hkv
    cache = ref.cache_of(st2)
    pol, _ = ref.policy_of(None, 8, 0, 0)
    import ctypes as C
    assert ref.lib().hikv_ref_decode_step(C.byref(bad), C.byref(cache), C.byref(pol), None, None,
                                          None, None, None, None) == -1


def _read_heap_golden():
    rows = {}
    for line in open(os.path.join(GOLDEN, "hikv_heap_examples.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, *ent = line.split()
        rows[name] = [(float(sc), int(tok)) for sc, tok in (e.split(":") for e in ent)]
    return rows


def heap_worked_examples():
    g = _read_heap_golden()
    a, b = HP.sort_pair(g["up_in_a"], g["up_in_b"])
    assert a == g["up_sorted_a"] and b == g["up_sorted_b"], (a, b)
    lo, hi = HP.partial_merge(a, b)
    assert lo == g["up_smaller"] and hi == g["up_larger"], (lo, hi)
    assert HP.pick(lo) == g["up_node0"] and HP.pick(hi) == g["up_node1"]
    h = HP.VectorHeap.build(g["up_in_a"] + g["up_in_b"], 4)
    assert h.nodes == [g["up_node0"], g["up_node1"]], h.nodes
    h.check()
    root = list(g["down_root"])
    root[0] = g["down_new"][0]
    assert root == g["down_replaced"] and HP.pick(root) == g["down_picked"]
    h = HP.VectorHeap(4)
    h.nodes = [list(g["down_root"])]
    assert h.offer(g["down_new"][0]) == g["down_root"][0]
    assert h.nodes[0] == g["down_picked"]
    assert h.offer((0.5, 99)) == (0.5, 99)           # below the minimum: discarded
    assert h.offer((2.0, 98)) == (2.0, 98)           # equal to it: discarded too


def heap_keeps_the_top_scores(seed=43, trials=80):
    rng = np.random.Generator(np.random.PCG64(seed))
    key = lambda e: e[0]
    for t in range(trials):
        w = int(rng.integers(1, 6))
        K = w * int(rng.integers(1, 10))
        m = int(rng.integers(0, 50))
        sc = rng.permutation(K + m).astype(np.float64) / 3.0   # distinct scores
        ent = [(float(sc[i]), i) for i in range(K + m)]
        h = HP.VectorHeap.build(ent[:K], w)
        h.check()
        assert sorted(h.entries()) == sorted(ent[:K])
        offered = list(ent[:K])
        for e in ent[K:]:
            before = sorted(h.entries())
            mn = h.minimum()
            assert mn == min(before, key=key)
            ev = h.offer(e)
            h.check()
            assert h.visited <= h.depth(), (t, h.visited, h.depth())
            if e[0] > mn[0]:
                assert ev == mn
                want = sorted([x for x in before if x != mn] + [e])
            else:
                assert ev == e
                want = before
            assert sorted(h.entries()) == want
            offered.append(e)
            assert sorted(h.entries()) == sorted(sorted(offered, key=key, reverse=True)[:K])


def dual_bank_matches_its_definition(seed=41):
    rng = np.random.Generator(np.random.PCG64(seed))
    Hkv, G, D = 2, 2, 16
    Hq = Hkv * G
    scale = 1.0 / math.sqrt(D)
    # (budget, sinks, n_recent, prompt, decode steps, heap node width): the
    # pages' own split (no sinks, window = half the budget), then a window
    # that the budget caps (W' = budget - sinks, no bank left).
    for beta, S, R, Lp, T, width in ((16, 0, 8, 40, 18, 4), (8, 2, 16, 14, 10, 0)):
        Wp = min(R, beta - S)
        K = beta - S - Wp
        n = Lp + T
        keys = rng.standard_normal((Hkv, n, D)).astype(np.float32)
        vals = rng.standard_normal((Hkv, n, D)).astype(np.float32)
        qs = rng.standard_normal((Hq, n, D)).astype(np.float32)  # the query of every position
        cap = Lp + 2
        st = dict(k=np.zeros((1, Hkv, cap, D), np.float32), v=np.zeros((1, Hkv, cap, D), np.float32),
                  pos=np.full((1, Hkv, cap), -1, np.int32), imp=np.zeros((1, Hkv, cap), np.float32),
                  len=np.full((1, Hkv), Lp, np.int32))
        st["k"][0, :, :Lp] = keys[:, :Lp]
        st["v"][0, :, :Lp] = vals[:, :Lp]
        st["pos"][0, :, :Lp] = np.arange(Lp, dtype=np.int32)
        # contrib[j, s, l]: the weight token l received from the group's
        # queries at step s (prompt steps: the causal prompt attention)
        contrib = np.zeros((Hkv, n, n))
        mask = np.tril(np.ones((Lp, Lp), dtype=bool))
        for j in range(Hkv):
            P = sdpa(qs[j * G:(j + 1) * G, :Lp], keys[j, :Lp][None], np.eye(Lp)[None], scale, mask)
            contrib[j, :Lp, :Lp] = P.sum(0)
        qpos = np.arange(Lp, dtype=np.int32)[None]
        assert ref.prefill_scores(st, Hq, qs[None, :, :Lp], qpos, window=Wp) == 0
        code, _ = ref.evict(st, Hq, [Lp - 1], budget_all=beta, n_sink=S, n_recent=R)
        assert code == 0

        def score(j, l, upto):  # steps l .. l + W' - 1, as far as they have run
            return float(contrib[j, l:min(l + Wp, upto + 1), l].sum())

        heaps = {}
        for t in range(T + 1):
            newest = Lp - 1 + t
            if t > 0:
                before = {j: ref.live_positions(st, 0, j).copy() for j in range(Hkv)}
                code, _, _ = ref.decode_step(
                    st, Hq, qs[None, :, newest].copy(), keys[None, :, newest].copy(),
                    vals[None, :, newest].copy(), np.array([newest], np.int32), budget_all=beta,
                    n_sink=S, n_recent=R, accumulate=ref.ACC_RECENT)
                assert code == 0
                for j in range(Hkv):
                    A = np.append(before[j], newest)
                    P = sdpa(qs[j * G:(j + 1) * G, newest][:, None], keys[j, A][None],
                             np.eye(len(A))[None], scale)[:, 0, :]
                    contrib[j, newest, A] = P.sum(0)
            for j in range(Hkv):
                nl = int(st["len"][0, j])
                live = st["pos"][0, j, :nl]
                for l, got in zip(live, st["imp"][0, j, :nl]):
                    want = score(j, int(l), newest)
                    assert abs(float(got) - want) <= 1e-5 * max(1.0, want), (beta, t, j, int(l), got, want)
                left = list(range(S, newest - Wp + 1))  # every token that has left the window
                top = sorted(left, key=lambda l: score(j, l, newest), reverse=True)[:K]
                want_set = set(range(S)) | set(range(newest - Wp + 1, newest + 1)) | set(top)
                assert set(live.tolist()) == want_set, (beta, t, j)
                if width:
                    if t == 0:
                        heaps[j] = HP.VectorHeap.build([(score(j, l, newest), l) for l in top], width)
                    else:
                        heaps[j].offer((score(j, newest - Wp, newest), newest - Wp))
                    heaps[j].check()
                    assert sorted(l for _, l in heaps[j].entries()) == sorted(top), (t, j)


def stage2_chunks_reduce_to_attention(seed=47):
    B, Hkv, G, D, cap = 1, 2, 2, 16, 64
    Hq = Hkv * G
    st = W.random_cache(seed, B, Hq, Hkv, D, W.F32, cap, [[40, 17]])   # 41 and 18 tokens: ragged chunks
    step = W.random_step(seed + 1, B, Hq, Hkv, D, W.F32, st["newest"])
    before = ref.copy_state(st)
    scale = 1.0 / math.sqrt(D)
    code, out, dbg = ref.decode_step(st, Hq, step["q"], step["k_new"], step["v_new"], step["new_pos"],
                                     budget_all=cap, stage2_channels=D, stage2_v=ref.S2V_CHUNK)
    assert code == 0
    for j in range(Hkv):
        k, v, _, _ = _unit_rows(before, 0, j, W.F32)
        k = np.concatenate([k, widen(step["k_new"][0, j], W.F32)[None]])
        v = np.concatenate([v, widen(step["v_new"][0, j], W.F32)[None]])
        q = widen(step["q"][0, j * G:(j + 1) * G], W.F32)[:, None, :]
        want = sdpa(q, k[None], v[None], scale)[:, 0, :]
        assert rel_err(out[0, j * G:(j + 1) * G], want) < 1e-6, j
        assert np.all(dbg["sel_count"][0, j * G:(j + 1) * G] == k.shape[0])


def stage2_chunks_select_by_probability(seed=53):
    G, D, cap, r, n_old = 3, 16, 64, 5, 39              # 40 tokens: chunks of 16, 16 and 8
    st0 = W.random_cache(seed, 1, G, 1, D, W.F32, cap, [[n_old]])
    step = W.random_step(seed + 1, 1, G, 1, D, W.F32, st0["newest"])
    L = n_old + 1
    scale = 1.0 / math.sqrt(D)
    pos = np.append(st0["pos"][0, 0, :n_old], step["new_pos"][0])
    order = np.argsort(pos, kind="stable")               # slots by position
    rank = np.empty(L, dtype=np.int64)
    rank[order] = np.arange(L)
    k = np.concatenate([widen(st0["k"][0, 0, :n_old], W.F32), widen(step["k_new"][0, 0], W.F32)[None]])
    P = []
    for g in range(G):
        qg = widen(step["q"][0, g], W.F32)
        E = np.argsort(-np.abs(qg), kind="stable")[:r]    # the r largest |q_d|, lower index first
        qm = np.zeros_like(qg)
        qm[E] = qg[E]
        P.append(sdpa(qm[None, None], k[None], np.eye(L)[None], scale)[0, 0])
    outs = []
    for c0 in range(0, L, D):
        m = min(D, L - c0)
        st = ref.copy_state(st0)
        st["v"][0, 0] = 0.0
        vnew = np.zeros((1, 1, D), np.float32)
        for s in range(L):                                # V row of a chunk member: one-hot of its rank
            if c0 <= rank[s] < c0 + m:
                if s < n_old:
                    st["v"][0, 0, s, rank[s] - c0] = 1.0
                else:
                    vnew[0, 0, rank[s] - c0] = 1.0
        kw = dict(budget_all=cap, stage2_channels=r, stage2_v=ref.S2V_CHUNK)
        code, out, _ = ref.decode_step(st, G, step["q"], step["k_new"], vnew, step["new_pos"], **kw)
        assert code == 0
        outs.append(out)
        members = order[c0:c0 + m]
        for g in range(G):
            got = out[0, g, :m].astype(np.float64)
            assert np.all(out[0, g, m:] == 0)
            kept = got > 0
            assert kept.sum() == min(r, m), (c0, g, int(kept.sum()))
            want = P[g][members]
            assert np.abs(got[kept] - want[kept]).max() <= 1e-6 * want[kept].max(), (c0, g)
            if (~kept).any():
                assert want[kept].min() >= want[~kept].max(), (c0, g)
        # the same chunk with the cache's slots permuted
        perm = np.random.Generator(np.random.PCG64(seed + c0)).permutation(n_old)
        sp = ref.copy_state(st0)
        for f in ("k", "v", "pos", "imp"):
            src = (st if f == "v" else st0)[f][0, 0, :n_old]
            sp[f][0, 0, :n_old] = src[perm]
        code, outp, _ = ref.decode_step(sp, G, step["q"], step["k_new"], vnew, step["new_pos"], **kw)
        assert code == 0 and np.abs(outp - out).max() <= 1e-12, c0


def logit_accumulation_matches_library(seed=59):
    B, Hkv, G, D, cap = 1, 2, 3, 16, 40
    Hq = Hkv * G
    st0 = W.random_cache(seed, B, Hq, Hkv, D, W.F32, cap, [[15, 8]])
    step = W.random_step(seed + 1, B, Hq, Hkv, D, W.F32, st0["newest"])
    scale = 1.0 / math.sqrt(D)
    beta, S, R = 12, 2, 4
    newest = int(step["new_pos"][0])
    for r in (0, 5):
        st = ref.copy_state(st0)
        code, _, dbg = ref.decode_step(st, Hq, step["q"], step["k_new"], step["v_new"], step["new_pos"],
                                       budget_all=beta, n_sink=S, n_recent=R, stage2_channels=r,
                                       stage2_tokens=8 if r else 0, accumulate=ref.ACC_LOGIT)
        assert code == 0
        for j in range(Hkv):
            k, _, pos, imp = _unit_rows(st0, 0, j, W.F32)
            k = np.concatenate([k, widen(step["k_new"][0, j], W.F32)[None]])
            pos = np.append(pos, newest)
            L = k.shape[0]
            q = widen(step["q"][0, j * G:(j + 1) * G], W.F32)
            if r:
                for g in range(G):
                    keep_ch = np.argsort(-np.abs(q[g]), kind="stable")[:r]
                    mask = np.zeros(D, dtype=bool)
                    mask[keep_ch] = True
                    q[g, ~mask] = 0.0
            want = np.matmul(q, k.T).sum(0) * scale            # [L]
            got = dbg["imp_pre_evict"][0, j, :L].astype(np.float64) - np.append(imp, 0.0)
            assert np.abs(got - want).max() <= 1e-5 * max(1.0, np.abs(want).max()), (r, j)
            kept = _brute_kept(pos, dbg["imp_pre_evict"][0, j, :L].astype(np.float64), beta, S, R, newest)
            assert set(ref.live_positions(st, 0, j).tolist()) == kept, (r, j)


def snapkv_pooling_matches_library(seed=67):
    from numpy.lib.stride_tricks import sliding_window_view
    B, Hkv, G, D = 1, 2, 2, 16
    Hq = Hkv * G
    L, n_obs, k = 30, 6, 5
    rng = np.random.Generator(np.random.PCG64(seed))
    scale = 1.0 / math.sqrt(D)
    for gaps in (False, True):
        posv = (np.arange(L) * (3 if gaps else 1) + (rng.integers(0, 2, L) if gaps else 0)).astype(np.int32)
        posv = np.sort(posv)
        keys = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
        qo = rng.standard_normal((B, Hq, n_obs, D)).astype(np.float32)
        qpos = posv[-n_obs:][None].copy()                     # the last prompt tokens observe
        perm = rng.permutation(L)
        st = dict(k=np.ascontiguousarray(keys[:, :, perm]), v=np.zeros_like(keys),
                  pos=np.ascontiguousarray(np.broadcast_to(posv[perm], (B, Hkv, L))),
                  imp=np.zeros((B, Hkv, L), np.float32), len=np.full((B, Hkv), L, np.int32))
        assert ref.prefill_scores(st, Hq, qo, qpos, window=0, pool=k) == 0
        for j in range(Hkv):
            A = np.zeros(L)                                    # observation scores, position order
            for g in range(G):
                mask = qpos[0][:, None] >= posv[None, :]
                P = sdpa(qo[0, j * G + g][None], keys[0, j][None], np.eye(L)[None], scale, mask)[0]
                A += P.sum(0)
            span = np.full(int(posv[-1]) + k, -np.inf)
            span[posv] = A
            pooled = sliding_window_view(span, k).max(axis=1)[posv]
            got = np.zeros(L)
            got[np.searchsorted(posv, st["pos"][0, j])] = st["imp"][0, j]
            assert np.abs(got - pooled).max() < 1e-5, (gaps, j)



# ---------------------------------------------------------------------------
# Block-granular eviction ("KV Cache Compression and Dynamic Pruning in
# Production Serving", Sec. 5, PagedAttention block fragmentation).
# ---------------------------------------------------------------------------
def _evict_state(pos, imp, cap):
    L = len(pos)
    st = dict(k=np.zeros((1, 1, cap, 4), np.float32), v=np.zeros((1, 1, cap, 4), np.float32),
              pos=np.full((1, 1, cap), -1, np.int32), imp=np.zeros((1, 1, cap), np.float32),
              len=np.array([[L]], np.int32))
    st["pos"][0, 0, :L] = pos
    st["imp"][0, 0, :L] = imp
    return st


def paged_block_golden():
    """The page's block-allocation figure and two variants worked by hand
    (tests/golden/paged_blocks.txt)."""
    cases, cur = [], None
    for line in open(os.path.join(GOLDEN, "paged_blocks.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, rest = line.partition(" ")
        if key == "case":
            cur = dict(name=rest)
            cases.append(cur)
        elif key == "fill":
            cur["fill"] = {int(b): float(v) for b, v in (t.split(":") for t in rest.split())}
        elif key == "kept_blocks":
            cur["kept_blocks"] = [int(x) for x in rest.split()]
        else:
            cur[key] = int(rest)
    assert len(cases) == 3
    for c in cases:
        P = c["block"]
        pos = np.arange(c["newest"] + 1, dtype=np.int32)
        imp = np.array([c["fill"][int(p) // P] for p in pos], np.float32)
        st = _evict_state(pos, imp, len(pos) + 1)
        code, _ = ref.evict(st, 1, [c["newest"]], budget_all=c["budget"], n_sink=c["sink"],
                            n_recent=c["recent"], block_tokens=P)
        assert code == 0, c["name"]
        got = list(ref.live_positions(st, 0, 0))
        want = [p for b in c["kept_blocks"] for p in range(b * P, b * P + P)]
        assert got == want, (c["name"], got[:40], want[:40])


def blocks_of_one_token_match_token_eviction(seed=71, trials=60):
    """Positions P apart put one token in each block: block sums are the
    tokens' importances, the tie rules agree (higher block id = higher
    position goes first), and a block is protected exactly when its token is,
    so block-granular eviction must keep the token-granular set."""
    rng = np.random.Generator(np.random.PCG64(seed))
    for t in range(trials):
        P = int(rng.choice([2, 3, 8, 16]))
        L = int(rng.integers(4, 40))
        slots = rng.permutation(L)
        pos = (slots * P + rng.integers(0, P, L)).astype(np.int32)
        imp = rng.integers(0, 6, L).astype(np.float32) * 0.25  # exact ties
        S = int(rng.integers(0, 3))
        beta = int(rng.integers(S, L + 2))
        R = int(rng.integers(0, 4))
        newest = int(pos.max())
        a, b = _evict_state(pos, imp, L + 1), _evict_state(pos, imp, L + 1)
        ca, _ = ref.evict(a, 1, [newest], budget_all=beta, n_sink=S, n_recent=R)
        cb, _ = ref.evict(b, 1, [newest], budget_all=beta, n_sink=S, n_recent=R, block_tokens=P)
        assert ca == 0 and cb == 0
        assert list(ref.live_positions(a, 0, 0)) == list(ref.live_positions(b, 0, 0)), (t, P)


def block_eviction_brute_force(seed=73, trials=120):
    """Every set of whole unprotected blocks is tried; exactly one satisfies
    the rule's defining properties -- the unit fits (or no unprotected block
    is left), every evicted block ranks below every kept unprotected block
    (lower sum, equal sums: higher id), and without its best-ranked evicted
    block the unit would not fit -- and it is the one the oracle evicts."""
    rng = np.random.Generator(np.random.PCG64(seed))
    for t in range(trials):
        P = int(rng.choice([2, 3, 4, 8]))
        L = int(rng.integers(3, min(28, 10 * P) + 1))
        pos = rng.choice(np.arange(0, 10 * P), L, replace=False).astype(np.int32)  # <= 10 blocks
        imp = rng.integers(0, 5, L).astype(np.float32) * 0.5
        S = int(rng.integers(0, 3))
        R = int(rng.integers(0, 5))
        beta = int(rng.integers(S, L + 2))
        newest = int(pos.max())
        W_ = min(R, beta - S)
        prot = (pos < S) | (pos > newest - W_)
        ids = pos // P
        blocks = sorted(set(ids.tolist()))
        score = {b: float(np.sum(imp[ids == b].astype(np.float64))) for b in blocks}
        count = {b: int(np.sum(ids == b)) for b in blocks}
        bprot = {b: bool(np.any(prot[ids == b])) for b in blocks}
        free = [b for b in blocks if not bprot[b]]
        rank = lambda b: (score[b], -b)  # lower ranks go first
        valid = []
        for mask in range(1 << len(free)):
            ev = [free[i] for i in range(len(free)) if mask >> i & 1]
            kept_free = [b for b in free if b not in ev]
            live = L - sum(count[b] for b in ev)
            fits = live <= beta or not kept_free
            ordered = all(rank(e) < rank(k) for e in ev for k in kept_free)
            minimal = not ev or live + count[max(ev, key=rank)] > beta
            if fits and ordered and minimal:
                valid.append(set(ev))
        assert len(valid) == 1, (t, valid)
        st = _evict_state(pos, imp, L + 1)
        code, _ = ref.evict(st, 1, [newest], budget_all=beta, n_sink=S, n_recent=R, block_tokens=P)
        assert code == 0
        want = sorted(int(p) for p in pos if int(p) // P not in valid[0])
        assert sorted(ref.live_positions(st, 0, 0)) == want, (t, P)

ALL = [attention_matches_library, rows_sum_to_group, streaming_closed_form, eviction_brute_force,
       golden_cases, permutation_invariance, channel_permutation, conservation,
       stage2_reduces_to_stage1, stage2_selection, equal_keys_closed_form, prefill_column_sums,
       errors_leave_unit_unchanged, heap_worked_examples, heap_keeps_the_top_scores,
       dual_bank_matches_its_definition, stage2_chunks_reduce_to_attention,
       stage2_chunks_select_by_probability, logit_accumulation_matches_library,
       snapkv_pooling_matches_library,
       paged_block_golden, blocks_of_one_token_match_token_eviction, block_eviction_brute_force]
