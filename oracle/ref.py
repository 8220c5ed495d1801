"""ctypes wrapper of the CPU oracle (libhikv_ref.so).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the package smoke check
and the benchmark's CPU-baseline leg; never by the product path.

State is a dict of numpy arrays mutated in place:
  k, v  [B][Hkv][cap][D] (uint16 bf16 bits or float32), pos int32, imp float32
  [B][Hkv][cap], len int32 [B][Hkv].
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhikv_ref.so")

F32, BF16 = 0, 1


class Shape(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("capacity", C.c_int32), ("kv_dtype", C.c_int32),
                ("scale", C.c_float)]


class Cache(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("pos", C.c_void_p),
                ("imp", C.c_void_p), ("len", C.c_void_p)]


class Policy(C.Structure):
    _fields_ = [("budget", C.c_void_p), ("budget_all", C.c_int32), ("n_sink", C.c_int32),
                ("n_recent", C.c_int32), ("stage2_channels", C.c_int32),
                ("stage2_tokens", C.c_int32), ("accumulate", C.c_int32), ("stage2_v", C.c_int32),
                ("block_tokens", C.c_int32)]


ACC_ALL, ACC_RECENT, ACC_LOGIT = 0, 1, 2
S2V_TOPK, S2V_CHUNK = 0, 1


class Debug(C.Structure):
    _fields_ = [("sel_channels", C.c_void_p), ("sel_tokens", C.c_void_p),
                ("sel_count", C.c_void_p), ("approx_logits", C.c_void_p),
                ("imp_pre_evict", C.c_void_p), ("kept", C.c_void_p), ("prob_sum", C.c_void_p)]


_libs = {}
_active = [LIB_PATH]


def use_library(path):
    """Point every oracle call at another build of the oracle (mutation tests)."""
    prev = _active[0]
    _active[0] = path
    return prev


def lib():
    path = _active[0]
    if path not in _libs:
        if path == LIB_PATH and not os.path.exists(LIB_PATH):
            from oracle import build as _b  # noqa: WPS433
            _b.build()
        L = C.CDLL(path)
        P = C.POINTER
        L.hikv_ref_decode_step.argtypes = [P(Shape), P(Cache), P(Policy), C.c_void_p, C.c_void_p,
                                           C.c_void_p, C.c_void_p, C.c_void_p, P(Debug)]
        L.hikv_ref_evict.argtypes = [P(Shape), P(Cache), P(Policy), C.c_void_p, P(Debug)]
        L.hikv_ref_prefill_scores.argtypes = [P(Shape), P(Cache), C.c_void_p, C.c_void_p,
                                              C.c_int32, C.c_int32, C.c_int32]
        for f in (L.hikv_ref_decode_step, L.hikv_ref_evict, L.hikv_ref_prefill_scores):
            f.restype = C.c_int
        _libs[path] = L
    return _libs[path]


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "arrays passed to the oracle must be C-contiguous"
    return a.ctypes.data


def shape_of(state, n_q_heads: int, scale: float = 0.0) -> Shape:
    k = state["k"]
    B, Hkv, cap, D = k.shape
    dt = F32 if k.dtype == np.float32 else BF16
    return Shape(B, n_q_heads, Hkv, D, cap, dt, scale)


def cache_of(state) -> Cache:
    return Cache(_ptr(state["k"]), _ptr(state["v"]), _ptr(state["pos"]), _ptr(state["imp"]),
                 _ptr(state["len"]))


def policy_of(budget=None, budget_all=0, n_sink=0, n_recent=0, stage2_channels=0,
              stage2_tokens=0, accumulate=ACC_ALL, stage2_v=S2V_TOPK, block_tokens=0):
    keep = None
    if budget is not None:
        keep = np.ascontiguousarray(budget, dtype=np.int32)
    pol = Policy(_ptr(keep), int(budget_all), int(n_sink), int(n_recent), int(stage2_channels),
                 int(stage2_tokens), int(accumulate), int(stage2_v), int(block_tokens))
    return pol, keep


def copy_state(state):
    return {k: np.array(v, copy=True) for k, v in state.items() if k in ("k", "v", "pos", "imp", "len")}


def decode_step(state, n_q_heads, q, k_new, v_new, new_pos, *, budget=None, budget_all=0,
                n_sink=0, n_recent=0, stage2_channels=0, stage2_tokens=0, scale=0.0,
                debug=True, accumulate=ACC_ALL, stage2_v=S2V_TOPK, block_tokens=0):
    """One oracle decode step; mutates ``state``.  Returns (status, out, dbg)."""
    L = lib()
    sh = shape_of(state, n_q_heads, scale)
    B, Hkv, cap = sh.batch, sh.n_kv_heads, sh.capacity
    pol, _keep = policy_of(budget, budget_all, n_sink, n_recent, stage2_channels, stage2_tokens,
                           accumulate, stage2_v, block_tokens)
    out = np.zeros((B, n_q_heads, sh.head_dim), dtype=np.float32)
    q = np.ascontiguousarray(q)
    k_new = np.ascontiguousarray(k_new)
    v_new = np.ascontiguousarray(v_new)
    new_pos = np.ascontiguousarray(new_pos, dtype=np.int32)
    dbg = None
    dbg_c = None
    if debug:
        r = max(stage2_channels, 1)
        kT = max(stage2_tokens, 1)
        dbg = dict(
            sel_channels=np.full((B, n_q_heads, r), -1, dtype=np.int32),
            sel_tokens=np.full((B, n_q_heads, kT), -1, dtype=np.int32),
            sel_count=np.zeros((B, n_q_heads), dtype=np.int32),
            approx_logits=np.full((B, n_q_heads, cap), np.nan, dtype=np.float64),
            imp_pre_evict=np.full((B, Hkv, cap), np.nan, dtype=np.float32),
            kept=np.zeros((B, Hkv, cap), dtype=np.uint8),
            prob_sum=np.zeros((B, Hkv), dtype=np.float64),
        )
        dbg_c = Debug(*[_ptr(dbg[f]) for f, _ in Debug._fields_])
    cache = cache_of(state)
    st = L.hikv_ref_decode_step(C.byref(sh), C.byref(cache), C.byref(pol), _ptr(q), _ptr(k_new),
                                _ptr(v_new), _ptr(new_pos), _ptr(out),
                                C.byref(dbg_c) if dbg_c is not None else None)
    return st, out, dbg


def evict(state, n_q_heads, newest_pos, *, budget=None, budget_all=0, n_sink=0, n_recent=0,
          debug=True, block_tokens=0):
    L = lib()
    sh = shape_of(state, n_q_heads)
    B, Hkv, cap = sh.batch, sh.n_kv_heads, sh.capacity
    pol, _keep = policy_of(budget, budget_all, n_sink, n_recent, block_tokens=block_tokens)
    newest_pos = np.ascontiguousarray(newest_pos, dtype=np.int32)
    dbg = None
    dbg_c = None
    if debug:
        dbg = dict(imp_pre_evict=np.full((B, Hkv, cap), np.nan, dtype=np.float32),
                   kept=np.zeros((B, Hkv, cap), dtype=np.uint8))
        dbg_c = Debug(None, None, None, None, _ptr(dbg["imp_pre_evict"]), _ptr(dbg["kept"]), None)
    cache = cache_of(state)
    st = L.hikv_ref_evict(C.byref(sh), C.byref(cache), C.byref(pol), _ptr(newest_pos),
                          C.byref(dbg_c) if dbg_c is not None else None)
    return st, dbg


def prefill_scores(state, n_q_heads, q_obs, q_pos, window=0, scale=0.0, pool=0):
    L = lib()
    sh = shape_of(state, n_q_heads, scale)
    q_obs = np.ascontiguousarray(q_obs)
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int32)
    n_obs = q_obs.shape[2] if q_obs.ndim == 4 else 0
    cache = cache_of(state)
    return L.hikv_ref_prefill_scores(C.byref(sh), C.byref(cache), _ptr(q_obs), _ptr(q_pos),
                                     int(n_obs), int(window), int(pool))


def live_positions(state, b, j):
    n = int(state["len"][b, j])
    return np.sort(state["pos"][b, j, :n])


def live_rows(state, b, j):
    """Rows of one unit as a dict keyed by position: pos -> (k bytes, v bytes, imp)."""
    n = int(state["len"][b, j])
    out = {}
    for s in range(n):
        p = int(state["pos"][b, j, s])
        out[p] = (state["k"][b, j, s].tobytes(), state["v"][b, j, s].tobytes(),
                  float(state["imp"][b, j, s]))
    return out
