"""The C-ABI library loads and exports every entry point include/hikv.h
declares; host-side argument checks return their codes without touching a
GPU (no compute calls here)."""
import ctypes as C
import os
import re
import subprocess

import pytest

from importance_aware_kv_amd import hikv as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hikv.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hikv_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("hikv_decode_step", "hikv_evict", "hikv_settle", "hikv_pending", "hikv_prefill_scores",
                 "hikv_workspace_bytes", "hikv_device_status", "hikv_status_string"):
        assert want in names
    assert set(names) == set(H.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = H.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", H.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (hikv_\w+)", out))
    assert set(declared_functions()) <= exported


CALIB_HEADER = os.path.join(ROOT, "include", "hikv_calib.h")


def test_calibration_library_exports_its_header():
    """The measurement aids (a streaming read, an empty kernel) are a library
    of their own; argument checks return codes without a GPU."""
    src = re.sub(r"/\*.*?\*/", "", open(CALIB_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(hikv_[a-z_]+)\s*\(", src)))
    assert set(names) == set(H.CALIB_EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", H.CALIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    assert set(names) <= set(re.findall(r"\bT (hikv_\w+)", out))
    L = H.calib_lib()
    fake = C.c_void_p(16)
    assert L.hikv_calib_stream(None, fake, 64, 256, fake, 1, fake, None, None, None) == -1
    assert L.hikv_calib_stream(fake, fake, 64, 100, fake, 1, fake, None, None, None) == -1   # row bytes % 16
    assert L.hikv_calib_stream(fake, fake, 64, 256, fake, 1, fake, fake, None, None) == -1   # one event
    assert L.hikv_calib_stream(fake, fake, 64, 256, fake, 0, fake, None, None, None) == 0    # nothing to do
    assert L.hikv_calib_empty(-1, None) == -1


def _shape(**kw):
    d = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, capacity=64, kv_dtype=H.HIKV_BF16,
             scale=0.0)
    d.update(kw)
    return H.make_shape(**d)


def test_workspace_sizing_and_bad_shapes():
    pol = H.make_policy(budget_all=32, n_sink=4, n_recent=8)
    assert H.hikv_workspace_bytes(_shape(), pol) > 0
    assert H.hikv_workspace_bytes(_shape(n_q_heads=6, n_kv_heads=4), pol) == 0   # Hq % Hkv
    assert H.hikv_workspace_bytes(_shape(head_dim=96), pol) == 0                  # D
    assert H.hikv_workspace_bytes(_shape(n_q_heads=32, n_kv_heads=2), pol) == 0   # G = 16
    assert H.hikv_workspace_bytes(_shape(kv_dtype=7), pol) == 0
    bad_pol = H.make_policy(budget_all=32, n_sink=-1)
    assert H.hikv_workspace_bytes(_shape(), bad_pol) == 0
    s2 = H.make_policy(budget_all=32, stage2_channels=32, stage2_tokens=256)
    assert H.hikv_workspace_bytes(_shape(), s2) > H.hikv_workspace_bytes(_shape(), pol)
    assert H.hikv_workspace_bytes(_shape(), H.make_policy(stage2_channels=200, stage2_tokens=1)) == 0


def test_decode_step_host_checks():
    L = H.lib()
    pol = H.make_policy(budget_all=32, n_sink=4, n_recent=8)
    fake = C.c_void_p(0x1000)
    cache = H.hikv_cache(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)

    def call(shape, cache=cache, pol=pol, q=fake, ws=fake, ws_bytes=1 << 30):
        return L.hikv_decode_step(C.byref(shape), C.byref(cache), C.byref(pol), q, fake, fake, fake,
                                  fake, ws, ws_bytes, None, None)

    assert call(_shape(n_q_heads=6, n_kv_heads=4)) == H.HIKV_EINVAL
    assert call(_shape(head_dim=96)) == H.HIKV_EUNSUPPORTED
    assert call(_shape(n_q_heads=48, n_kv_heads=3)) == H.HIKV_EUNSUPPORTED          # G = 16
    assert call(_shape(batch=4096, n_kv_heads=2, n_q_heads=2)) == H.HIKV_EUNSUPPORTED  # units
    assert call(_shape(), cache=H.hikv_cache(0, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)) == H.HIKV_EINVAL
    assert call(_shape(), cache=H.hikv_cache(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0)) == H.HIKV_EINVAL
    assert call(_shape(), cache=H.hikv_cache(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1004)) == H.HIKV_EINVAL
    # pending-eviction state: 4 words per unit plus 4 per 2048-slot importance block
    assert H.hikv_state_bytes(_shape()) == 4 * 2 * 2 * 8
    assert H.hikv_state_bytes(_shape(capacity=5000)) == 4 * 2 * 2 * 16
    assert H.hikv_state_bytes(_shape(head_dim=96)) == 0
    assert call(_shape(), q=None) == H.HIKV_EINVAL
    assert call(_shape(), q=C.c_void_p(0x1008)) == H.HIKV_EINVAL                    # alignment
    assert call(_shape(), ws_bytes=16) == H.HIKV_EINVAL                             # workspace
    assert call(_shape(), pol=H.make_policy(budget_all=8, n_recent=-2)) == H.HIKV_EINVAL
    assert call(_shape(), pol=H.make_policy(budget_all=8, accumulate=3)) == H.HIKV_EINVAL  # unknown mode
    assert call(_shape(), pol=H.make_policy(budget_all=8, stage2_channels=8, stage2_v=2)) == H.HIKV_EINVAL
    # the chunked V side needs no k_T; the exact top-k_T side does
    assert call(_shape(batch=0), pol=H.make_policy(budget_all=8, stage2_channels=8,
                                                   stage2_v=H.HIKV_S2V_CHUNK)) == H.HIKV_OK
    assert call(_shape(), pol=H.make_policy(budget_all=8, stage2_channels=8)) == H.HIKV_EINVAL
    assert call(_shape(batch=0), pol=H.make_policy(budget_all=8, accumulate=H.HIKV_ACC_RECENT)) == H.HIKV_OK
    assert call(_shape(batch=0)) == H.HIKV_OK                                       # empty batch
    assert L.hikv_evict(C.byref(_shape()), C.byref(cache), C.byref(pol), None, fake, 1 << 30,
                        None) == H.HIKV_EINVAL
    assert L.hikv_prefill_scores(C.byref(_shape()), C.byref(cache), fake, fake, 0, 0, -1, fake,
                                 1 << 30, None) == H.HIKV_EINVAL
    assert L.hikv_prefill_scores(C.byref(_shape()), C.byref(cache), fake, fake, -1, 0, 0, fake,
                                 1 << 30, None) == H.HIKV_EINVAL
    assert L.hikv_prefill_scores(C.byref(_shape()), C.byref(cache), fake, fake, 0, 0, 0, fake,
                                 1 << 30, None) == H.HIKV_OK
    import numpy as np
    bad_hint = np.array([10, 64, 3, 3], dtype=np.int32)   # 64 + 1 > capacity 64
    assert call(_shape(), pol=H.make_policy(budget_all=8, len_hint=bad_hint)) == H.HIKV_EINVAL
    neg_hint = np.array([10, -1, 3, 3], dtype=np.int32)
    assert call(_shape(), pol=H.make_policy(budget_all=8, len_hint=neg_hint)) == H.HIKV_EINVAL
    # the launch-sequence selector of the debug struct: only the two documented values
    dbg = H.hikv_debug(None, None, None, None, None, 5)
    assert L.hikv_decode_step(C.byref(_shape()), C.byref(cache), C.byref(pol), fake, fake, fake, fake,
                              fake, fake, 1 << 30, C.byref(dbg), None) == H.HIKV_EINVAL
    # the allocation-free variant: no status word, or a workspace beyond its static scratch
    assert L.hikv_decode_step_static(C.byref(_shape()), C.byref(cache), C.byref(pol), fake, fake, fake, fake,
                                     fake, None, None, None) == H.HIKV_EINVAL
    big = _shape(batch=64, n_kv_heads=8, n_q_heads=64, capacity=200000)
    assert H.hikv_workspace_bytes(big, pol) > H.HIKV_STATIC_SCRATCH_BYTES
    assert L.hikv_decode_step_static(C.byref(big), C.byref(cache), C.byref(pol), fake, fake, fake, fake,
                                     fake, fake, None, None) == H.HIKV_EINVAL
    assert H.status_string(H.HIKV_ECAPACITY) == "cache capacity exceeded"
    # settle / pending: host checks only (no device work is enqueued on error)
    assert L.hikv_settle(C.byref(_shape()), C.byref(cache), C.byref(pol), None, 1 << 30, None) == H.HIKV_EINVAL
    assert L.hikv_settle(C.byref(_shape()), C.byref(cache), C.byref(pol), fake, 16, None) == H.HIKV_EINVAL
    assert L.hikv_settle(C.byref(_shape(head_dim=96)), C.byref(cache), C.byref(pol), fake, 1 << 30,
                         None) == H.HIKV_EUNSUPPORTED
    assert L.hikv_pending(C.byref(_shape()), C.byref(cache), C.byref(pol), fake, 1 << 30, None,
                          None) == H.HIKV_EINVAL                                      # no output
    assert L.hikv_settle(C.byref(_shape(batch=0)), C.byref(cache), C.byref(pol), fake, 1 << 30,
                         None) == H.HIKV_OK
