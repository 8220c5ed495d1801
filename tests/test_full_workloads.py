"""Parity over whole workloads at full size: every decode step of each seeded
workload, in the launch configuration the benchmark times (the caller's
lengths passed as hints).  One GPU run per workload feeds two oracle tracks:

  lockstep     -- each step the oracle starts from the GPU's settled state
                  before the step; outputs, Stage II sets and kept sets
                  (with the tie rules of gpu_harness) are compared on every
                  unit, or on sampled units where the oracle's time demands;
  free-running -- the oracle runs the workload on its own from the prompt;
                  outputs and kept sets are compared each step until the
                  first step at which the kept sets differ, which must be a
                  near-tie of the importance (1e-6 relative); that step is
                  reported (fp32 sums on the GPU against fp64 in the oracle
                  drift apart by rounding, so such a step may come).
"""

import time

import numpy as np
import pytest
import torch

from gpu_harness import (GpuRun, OUT_TOL, TIE_RTOL, check_kept, check_stage2, chunk_alternatives,
                         chunk_row_errors, row_errors, say)
from importance_aware_kv_amd import hikv as H
from importance_aware_kv_amd import workloads as W
from oracle import ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H.lib()


def _sub(state, units):
    """The state of some units, each a batch row of one KV head."""
    return {k: np.ascontiguousarray(np.stack([state[k][b, j] for b, j in units])[:, None])
            for k in ("k", "v", "pos", "imp", "len")}


def _step_inputs(d, t, units, G):
    q = np.ascontiguousarray(np.stack([d["q"][t][b, j * G:(j + 1) * G] for b, j in units]))
    kn = np.ascontiguousarray(np.stack([d["k_new"][t][b, j:j + 1] for b, j in units]))
    vn = np.ascontiguousarray(np.stack([d["v_new"][t][b, j:j + 1] for b, j in units]))
    npos = np.ascontiguousarray(np.array([d["new_pos"][t][b] for b, j in units], dtype=np.int32))
    return q, kn, vn, npos


def _kept_differ_by_ties(post_gpu, post_ref, pre_ref, dref, kw, npos):
    """True when the kept sets are equal; False when they differ only on
    near-ties (checked); raises otherwise."""
    same = True
    B, Hkv = post_ref["len"].shape
    for b in range(B):
        for j in range(Hkv):
            g = set(ref.live_positions(post_gpu, b, j).tolist())
            r = set(ref.live_positions(post_ref, b, j).tolist())
            if g == r:
                continue
            same = False
            L = int(pre_ref["len"][b, j]) + 1
            pos = np.append(pre_ref["pos"][b, j, :L - 1], npos[b])
            imp = dref["imp_pre_evict"][b, j, :L].astype(np.float64)
            kept = dref["kept"][b, j, :L].astype(bool)
            beta = int(kw["budget"][b, j])
            Wp = min(kw["n_recent"], beta - kw["n_sink"])
            prot = (pos < kw["n_sink"]) | (pos > npos[b] - Wp)
            thr = imp[kept & ~prot].min()
            for p in g ^ r:
                i = np.nonzero(pos == p)[0]
                assert len(i) == 1 and not prot[i[0]], ("free-running: protected or unknown token differs", b, j, p)
                assert abs(imp[i[0]] - thr) <= TIE_RTOL * abs(thr), \
                    ("free-running: kept sets differ beyond a near-tie", b, j, p, imp[i[0]], thr)
    return same


# workload, full-attention pass, units sampled for the oracle (None: all),
# steps (None: the workload's own count), overrides of the workload's fields
CASES = [
    ("llama8b", False, None, None, None),
    ("headkv32k", False, None, None, None),
    ("longctx128k", False, None, None, None),
    ("longctx128k", True, [(0, 2), (1, 7)], None, None),
    ("twostage", False, None, None, None),
    ("hikv_dualbank", False, None, 48, None),
    ("hikv_hier", False, None, 48, None),
    # HiKV's chunked Stage II V side on 131072-token units: the first step
    # orders and chunks 131073 live tokens per unit, then steady steps
    ("longctx128k", False, [(0, 1), (1, 6)], 6,
     dict(stage2_channels=32, stage2_v=H.HIKV_S2V_CHUNK, name="longctx128k_chunks")),
]


@pytest.mark.parametrize("name,full,sample,steps,over", CASES,
                         ids=[(c[4] or {}).get("name", c[0] + ("_full" if c[1] else "")) for c in CASES])
def test_whole_workload_lockstep_and_free_running(name, full, sample, steps, over):
    t_start = time.time()
    w = W.workload(name, full=full, steps=steps)
    for k, v in (over or {}).items():
        setattr(w, k, v)
    say(f"[gpu] {w.name}: {w.steps} steps, B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} ctx={w.ctx}; generating")
    d = W.generate(w)
    G = w.group
    budget = w.budget_array()
    units = sample if sample is not None else [(b, j) for b in range(w.batch) for j in range(w.n_kv_heads)]
    run = GpuRun(ref.copy_state(d), w.n_q_heads, budget=budget if w.budgets is not None else None,
                 budget_all=w.budget_all, n_sink=w.n_sink, n_recent=w.n_recent, r=w.stage2_channels,
                 kT=w.stage2_tokens, hint=True, accumulate=w.accumulate, stage2_v=w.stage2_v)
    kw = dict(budget=np.ascontiguousarray(np.array([[budget[b, j]] for b, j in units], dtype=np.int32)),
              budget_all=0, n_sink=w.n_sink, n_recent=w.n_recent, stage2_channels=w.stage2_channels,
              stage2_tokens=w.stage2_tokens, scale=0.0, accumulate=w.accumulate, stage2_v=w.stage2_v)
    free = _sub(d, units)
    free_same = True
    first_diff = None
    worst_lock = worst_free = 0.0
    swaps = ties2 = 0
    for t in range(w.steps):
        pre = run.state(units=units, room=1)
        out, dbg = run.step(d["q"][t], d["k_new"][t], d["v_new"][t], d["new_pos"][t])
        post = run.state(units=units, room=0)
        q, kn, vn, npos = _step_inputs(d, t, units, G)
        gout = np.ascontiguousarray(np.stack([out[b, j * G:(j + 1) * G] for b, j in units]))
        # lockstep
        st = ref.copy_state(pre)
        code, want, dref = ref.decode_step(st, G, q, kn, vn, npos, **kw)
        assert code == 0
        if w.stage2_channels and w.stage2_v == H.HIKV_S2V_CHUNK:
            alts, _ = chunk_alternatives(dref, pre, npos, q, kn, vn, G, w.stage2_channels, want)
            e = chunk_row_errors(gout, alts)
        else:
            e = row_errors(gout, want)
        if w.stage2_channels:
            gdbg = {k: np.ascontiguousarray(np.stack([dbg[k][b, j * G:(j + 1) * G] for b, j in units]))
                    for k in ("sel_channels", "sel_tokens", "sel_count")}
            assert np.array_equal(gdbg["sel_count"], dref["sel_count"]), (w.name, t)
            if w.stage2_v == H.HIKV_S2V_TOPK:
                ties2 += check_stage2(gdbg, dref, pre, npos, G, w.stage2_tokens, where=f"{w.name} {t}",
                                      q=q, k_new=kn)
            else:
                assert np.array_equal(gdbg["sel_channels"], dref["sel_channels"]), (w.name, t)
        worst_lock = max(worst_lock, float(e.max()))
        assert e.max() <= OUT_TOL[w.dtype], (w.name, "lockstep output", t, float(e.max()))
        assert np.array_equal(post["len"], st["len"]), (w.name, t)
        swaps += check_kept(pre, post, st, dref, kw, npos, where=f"{w.name} lockstep {t}", q=q, k_new=kn)
        # free-running
        if free_same:
            fpre = ref.copy_state(free)
            code, fwant, fdref = ref.decode_step(free, G, q, kn, vn, npos, **kw)
            assert code == 0
            if w.stage2_channels and w.stage2_v == H.HIKV_S2V_CHUNK:
                falts, _ = chunk_alternatives(fdref, fpre, npos, q, kn, vn, G, w.stage2_channels, fwant)
                fe = chunk_row_errors(gout, falts)
            else:
                fe = row_errors(gout, fwant)
            worst_free = max(worst_free, float(fe.max()))
            assert fe.max() <= OUT_TOL[w.dtype], (w.name, "free-running output", t, float(fe.max()))
            free_same = _kept_differ_by_ties(post, free, fpre, fdref, kw, npos)
            if not free_same:
                first_diff = t
        if t % 16 == 0 or t == w.steps - 1:
            say(f"[gpu] {w.name} step {t}: lockstep worst {worst_lock:.2e}, free-running "
                f"{'in step' if free_same else f'kept sets first differ (near-tie) at step {first_diff}'}, "
                f"{time.time() - t_start:.0f}s")
    say(f"[gpu] {w.name}: {w.steps} steps on {len(units)} units, lockstep worst row error {worst_lock:.2e}, "
        f"{swaps} near-tie swaps, {ties2} Stage II token-set near-ties; free-running worst {worst_free:.2e}, "
        f"kept sets {'equal on every step' if first_diff is None else f'first differ at step {first_diff}'}")
