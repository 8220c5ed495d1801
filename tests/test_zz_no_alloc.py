"""The allocation-free decode step (hikv_decode_step_static: the library's
static per-GPU scratch instead of a caller's workspace) against
hikv_decode_step on the same inputs: calls in a row on shrinking shapes (so
each call's workspace layout lies over the previous call's leftovers in the
scratch), through the Stage I bulk cut with the caller's lengths, Stage II
(whose per-unit counters must start at zero) and the multi-launch sequence,
then a budget error.  Outputs, caches and pending-eviction state must be
identical to the bit (the same kernels on the same inputs), and device
errors must reach the caller's status word."""

import numpy as np
import pytest
import torch

from importance_aware_kv_amd import hikv as H
from importance_aware_kv_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H.lib()


# (B, Hkv, G, D, dtype, cap, budget, n_sink, n_recent, r, kT, hint, path)
CALLS = [
    (4, 8, 4, 128, W.BF16, 1500, 600, 4, 64, 0, 0, True, H.HIKV_PATH_AUTO),       # bulk cut, host plan
    (2, 4, 4, 128, W.BF16, 700, 300, 4, 32, 32, 64, False, H.HIKV_PATH_AUTO),     # Stage II
    (1, 2, 8, 64, W.F32, 300, 100, 2, 16, 0, 0, False, H.HIKV_PATH_MULTI_LAUNCH),  # multi-launch
]


def _one_call(i, B, Hkv, G, D, dtype, cap, budget, n_sink, n_recent, r, kT, hint, path, budget_override=None):
    Hq = G * Hkv
    rng = np.random.Generator(np.random.PCG64(300 + i))
    lens = rng.integers(budget - 5, cap - 2, size=(B, Hkv))
    st = W.random_cache(400 + i, B, Hq, Hkv, D, dtype, cap, lens)
    data = W.random_step(500 + i, B, Hq, Hkv, D, dtype, st["newest"])
    bud = np.full((B, Hkv), budget, dtype=np.int32) if budget_override is None else budget_override
    bt = torch.from_numpy(bud).cuda()
    lh = np.ascontiguousarray(lens, dtype=np.int32) if hint else None
    pol = H.make_policy(bt, 0, n_sink, n_recent, r, kT, len_hint=lh, budget_hint=bud if hint else None)
    dbg = H.hikv_debug(None, None, None, None, None, path)
    a = H.DeviceCache(st, Hq)
    b = H.DeviceCache(st, Hq)
    ws = H.workspace(a.shape, pol)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out_a = torch.full((B, Hq, D), -1.0, dtype=torch.float32, device="cuda")
    out_b = torch.full((B, Hq, D), -2.0, dtype=torch.float32, device="cuda")
    q, kn, vn = H.to_device(data["q"]), H.to_device(data["k_new"]), H.to_device(data["v_new"])
    pt = torch.from_numpy(data["new_pos"]).cuda()
    print(f"[gpu] static call {i}: B={B} Hkv={Hkv} G={G} D={D} cap={cap} r={r} path={path}", flush=True)
    assert H.hikv_decode_step(a.shape, a.cache, pol, q, kn, vn, pt, out_a, ws, debug=dbg) == H.HIKV_OK
    assert H.hikv_decode_step_static(b.shape, b.cache, pol, q, kn, vn, pt, out_b, status, debug=dbg) == H.HIKV_OK
    torch.cuda.synchronize()
    return a, b, ws, status, out_a, out_b


def test_static_scratch_calls_match_the_workspace_entry_point():
    for i, c in enumerate(CALLS):
        a, b, ws, status, out_a, out_b = _one_call(i, *c)
        assert H.hikv_device_status(ws) == H.HIKV_OK
        assert int(status.item()) == H.HIKV_OK
        assert torch.equal(out_a, out_b), i
        sa, sb = a.to_numpy(), b.to_numpy()
        for f in ("k", "v", "pos", "imp", "len"):
            assert np.array_equal(sa[f], sb[f]), (i, f)
        assert torch.equal(a.evict, b.evict), i
    # a device-side error reaches the caller's status word (budget below the sinks)
    B, Hkv = 1, 2
    bad = np.array([[100, 1]], dtype=np.int32)
    a, b, ws, status, out_a, out_b = _one_call(9, B, Hkv, 4, 128, W.BF16, 300, 100, 4, 16, 0, 0, False,
                                               H.HIKV_PATH_AUTO, budget_override=bad)
    assert H.hikv_device_status(ws) == H.HIKV_EBUDGET
    assert int(status.item()) == H.HIKV_EBUDGET
    assert torch.equal(out_a, out_b)
