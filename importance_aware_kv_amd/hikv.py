"""ctypes binding of libhikv.so (include/hikv.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libhikv.so.  There is no fallback; if the library is not built the
import of this module's functions raises.  torch provides device memory and
the stream.
"""

from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libhikv.so")

HIKV_F32, HIKV_BF16 = 0, 1
HIKV_ACC_ALL, HIKV_ACC_RECENT, HIKV_ACC_LOGIT = 0, 1, 2
HIKV_S2V_TOPK, HIKV_S2V_CHUNK = 0, 1
HIKV_PATH_AUTO, HIKV_PATH_MULTI_LAUNCH = 0, 1
HIKV_OK, HIKV_EINVAL, HIKV_EUNSUPPORTED, HIKV_EDEVICE, HIKV_ECAPACITY, HIKV_EBUDGET = 0, -1, -2, -3, -4, -5
HIKV_STATIC_SCRATCH_BYTES = 128 << 20

EXPORTS = ("hikv_state_bytes", "hikv_workspace_bytes", "hikv_decode_step", "hikv_decode_step_static", "hikv_evict",
           "hikv_settle", "hikv_pending",
           "hikv_prefill_workspace_bytes", "hikv_prefill_scores", "hikv_device_status", "hikv_status_string")


class hikv_shape(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("capacity", C.c_int32), ("kv_dtype", C.c_int32),
                ("scale", C.c_float)]


class hikv_cache(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("pos", C.c_void_p), ("imp", C.c_void_p),
                ("len", C.c_void_p), ("evict", C.c_void_p)]


class hikv_policy(C.Structure):
    _fields_ = [("budget", C.c_void_p), ("budget_all", C.c_int32), ("n_sink", C.c_int32),
                ("n_recent", C.c_int32), ("stage2_channels", C.c_int32),
                ("stage2_tokens", C.c_int32), ("len_hint", C.c_void_p), ("budget_hint", C.c_void_p),
                ("accumulate", C.c_int32), ("stage2_v", C.c_int32), ("block_tokens", C.c_int32)]


class hikv_debug(C.Structure):
    _fields_ = [("sel_channels", C.c_void_p), ("sel_tokens", C.c_void_p), ("sel_count", C.c_void_p),
                ("attend_start", C.c_void_p), ("attend_stop", C.c_void_p), ("stage1_path", C.c_int32)]


_lib = None


class LibraryMissing(RuntimeError):
    pass


def lib():
    """Load libhikv.so (built in-tree).  Raises if it is missing: no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryMissing(f"{LIB_PATH} is not built; run `python -m importance_aware_kv_amd.build`")
        L = C.CDLL(LIB_PATH)
        P = C.POINTER
        vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
        L.hikv_state_bytes.argtypes = [P(hikv_shape)]
        L.hikv_state_bytes.restype = sz
        L.hikv_workspace_bytes.argtypes = [P(hikv_shape), P(hikv_policy)]
        L.hikv_workspace_bytes.restype = sz
        L.hikv_decode_step.argtypes = [P(hikv_shape), P(hikv_cache), P(hikv_policy), vp, vp, vp, vp,
                                       vp, vp, sz, P(hikv_debug), vp]
        L.hikv_decode_step.restype = C.c_int
        L.hikv_decode_step_static.argtypes = [P(hikv_shape), P(hikv_cache), P(hikv_policy), vp, vp, vp, vp,
                                              vp, vp, P(hikv_debug), vp]
        L.hikv_decode_step_static.restype = C.c_int
        L.hikv_evict.argtypes = [P(hikv_shape), P(hikv_cache), P(hikv_policy), vp, vp, sz, vp]
        L.hikv_evict.restype = C.c_int
        L.hikv_settle.argtypes = [P(hikv_shape), P(hikv_cache), P(hikv_policy), vp, sz, vp]
        L.hikv_settle.restype = C.c_int
        L.hikv_pending.argtypes = [P(hikv_shape), P(hikv_cache), P(hikv_policy), vp, sz, vp, vp]
        L.hikv_pending.restype = C.c_int
        L.hikv_prefill_workspace_bytes.argtypes = [P(hikv_shape), i32]
        L.hikv_prefill_workspace_bytes.restype = sz
        L.hikv_prefill_scores.argtypes = [P(hikv_shape), P(hikv_cache), vp, vp, i32, i32, i32, vp, sz, vp]
        L.hikv_prefill_scores.restype = C.c_int
        L.hikv_device_status.argtypes = [vp, C.c_int, vp]
        L.hikv_device_status.restype = C.c_int
        L.hikv_status_string.argtypes = [C.c_int]
        L.hikv_status_string.restype = C.c_char_p
        _lib = L
    return _lib


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)


def make_shape(batch, n_q_heads, n_kv_heads, head_dim, capacity, kv_dtype, scale=0.0) -> hikv_shape:
    return hikv_shape(batch, n_q_heads, n_kv_heads, head_dim, capacity, kv_dtype, scale)


def make_policy(budget=None, budget_all=0, n_sink=0, n_recent=0, stage2_channels=0,
                stage2_tokens=0, len_hint=None, budget_hint=None, accumulate=HIKV_ACC_ALL,
                stage2_v=HIKV_S2V_TOPK, block_tokens=0) -> hikv_policy:
    """len_hint, budget_hint: optional host int32 numpy arrays (kept alive by the caller)."""
    hint = None if len_hint is None else len_hint.ctypes.data
    bhint = None if budget_hint is None else budget_hint.ctypes.data
    return hikv_policy(None if budget is None else budget.data_ptr(), budget_all, n_sink, n_recent,
                       stage2_channels, stage2_tokens, hint, bhint, accumulate, stage2_v, block_tokens)


def status_string(code: int) -> str:
    return lib().hikv_status_string(code).decode()


def check(code: int, what: str = "hikv call"):
    if code != HIKV_OK:
        raise RuntimeError(f"{what} failed: {code} ({status_string(code)})")


def hikv_state_bytes(shape: hikv_shape) -> int:
    return lib().hikv_state_bytes(C.byref(shape))


def hikv_workspace_bytes(shape: hikv_shape, policy: Optional[hikv_policy]) -> int:
    return lib().hikv_workspace_bytes(C.byref(shape), C.byref(policy) if policy is not None else None)


def hikv_prefill_workspace_bytes(shape: hikv_shape, n_obs: int) -> int:
    return lib().hikv_prefill_workspace_bytes(C.byref(shape), n_obs)


def hikv_decode_step(shape, cache, policy, q, k_new, v_new, new_pos, out, ws, debug=None,
                     stream=None) -> int:
    return lib().hikv_decode_step(C.byref(shape), C.byref(cache), C.byref(policy), _p(q), _p(k_new),
                                  _p(v_new), _p(new_pos), _p(out), _p(ws), ws.numel() * ws.element_size(),
                                  C.byref(debug) if debug is not None else None, _stream(stream))


def hikv_decode_step_static(shape, cache, policy, q, k_new, v_new, new_pos, out, status, debug=None,
                            stream=None) -> int:
    """hikv_decode_step on the library's static scratch; status: a device int32 tensor (one word)."""
    return lib().hikv_decode_step_static(C.byref(shape), C.byref(cache), C.byref(policy), _p(q), _p(k_new),
                                         _p(v_new), _p(new_pos), _p(out), _p(status),
                                         C.byref(debug) if debug is not None else None, _stream(stream))


def hikv_evict(shape, cache, policy, newest_pos, ws, stream=None) -> int:
    return lib().hikv_evict(C.byref(shape), C.byref(cache), C.byref(policy), _p(newest_pos), _p(ws),
                            ws.numel() * ws.element_size(), _stream(stream))


def hikv_settle(shape, cache, policy, ws, stream=None) -> int:
    return lib().hikv_settle(C.byref(shape), C.byref(cache), C.byref(policy), _p(ws),
                             ws.numel() * ws.element_size(), _stream(stream))


def hikv_pending(shape, cache, policy, ws, slot_out, stream=None) -> int:
    return lib().hikv_pending(C.byref(shape), C.byref(cache), C.byref(policy), _p(ws),
                              ws.numel() * ws.element_size(), _p(slot_out), _stream(stream))


def hikv_prefill_scores(shape, cache, q_obs, q_pos, n_obs, window, ws, stream=None, pool=0) -> int:
    return lib().hikv_prefill_scores(C.byref(shape), C.byref(cache), _p(q_obs), _p(q_pos), n_obs,
                                     window, pool, _p(ws), ws.numel() * ws.element_size(), _stream(stream))


# ---------------------------------------------------------------------------
# Measurement aids (include/hikv_calib.h, libhikv_calib.so): used by the
# benchmark only, not part of the decode path.
# ---------------------------------------------------------------------------
CALIB_PATH = os.path.join(PKG, "libhikv_calib.so")
CALIB_EXPORTS = ("hikv_calib_stream", "hikv_calib_empty")
_calib = None


def calib_lib():
    global _calib
    if _calib is None:
        if not os.path.exists(CALIB_PATH):
            raise LibraryMissing(f"{CALIB_PATH} is not built; run `python -m importance_aware_kv_amd.build`")
        L = C.CDLL(CALIB_PATH)
        vp = C.c_void_p
        L.hikv_calib_stream.argtypes = [vp, vp, C.c_int64, C.c_int64, vp, C.c_int32, vp, vp, vp, vp]
        L.hikv_calib_stream.restype = C.c_int
        L.hikv_calib_empty.argtypes = [C.c_int32, vp]
        L.hikv_calib_empty.restype = C.c_int
        _calib = L
    return _calib


def hikv_calib_stream(k, v, cap, row_bytes, tiles, sink, ev_start=None, ev_stop=None, stream=None) -> int:
    """tiles: device int32 [n][3] (unit, t0, t1); sink: device uint32-sized [n]."""
    return calib_lib().hikv_calib_stream(_p(k), _p(v), cap, row_bytes, _p(tiles), tiles.shape[0], _p(sink),
                                         ev_start, ev_stop, _stream(stream))


def hikv_calib_empty(n, stream=None) -> int:
    return calib_lib().hikv_calib_empty(n, _stream(stream))


def hikv_device_status(ws, clear=True, stream=None) -> int:
    return lib().hikv_device_status(_p(ws), 1 if clear else 0, _stream(stream))


# ---------------------------------------------------------------------------
# Device-side state (torch owns the memory) built from the seeded workloads.
# ---------------------------------------------------------------------------
class DeviceCache:
    """The cache of one layer on the GPU plus the descriptors the ABI wants."""

    def __init__(self, state: dict, n_q_heads: int, device="cuda", scale: float = 0.0):
        import torch
        self.torch = torch
        k = state["k"]
        B, Hkv, cap, D = k.shape
        self.dtype = HIKV_F32 if k.dtype == np.float32 else HIKV_BF16
        self.shape = make_shape(B, n_q_heads, Hkv, D, cap, self.dtype, scale)
        self.k = self._to(state["k"], device)
        self.v = self._to(state["v"], device)
        self.pos = torch.from_numpy(np.ascontiguousarray(state["pos"])).to(device)
        self.imp = torch.from_numpy(np.ascontiguousarray(state["imp"])).to(device)
        self.len = torch.from_numpy(np.ascontiguousarray(state["len"])).to(device)
        # the pending-eviction state: zero (nothing pending) with a fresh cache
        n = hikv_state_bytes(self.shape)
        if n == 0:
            raise RuntimeError("invalid cache shape")
        self.evict = torch.zeros((n + 15) // 16 * 4, dtype=torch.int32, device=device)
        self.cache = self.make_cache()

    def clone(self) -> "DeviceCache":
        """A device copy of this cache (rows, positions, importance, lengths and
        the pending-eviction state)."""
        c = DeviceCache.__new__(DeviceCache)
        c.torch = self.torch
        c.dtype, c.shape = self.dtype, self.shape
        for f in ("k", "v", "pos", "imp", "len", "evict"):
            setattr(c, f, getattr(self, f).clone())
        c.cache = c.make_cache()
        return c

    def make_cache(self) -> "hikv_cache":
        return hikv_cache(self.k.data_ptr(), self.v.data_ptr(), self.pos.data_ptr(),
                          self.imp.data_ptr(), self.len.data_ptr(), self.evict.data_ptr())

    def _to(self, a, device):
        t = self.torch.from_numpy(np.ascontiguousarray(a))
        if a.dtype == np.uint16:
            t = t.view(self.torch.int16)
        return t.to(device)

    def to_numpy(self, units=None, slots=None) -> dict:
        """Host copy of the cache.  units: optional list of (b, j) pairs, each
        becoming a batch row with one KV head; slots: copy only the first
        `slots` slots of every unit (the rest of the capacity is left out)."""
        torch = self.torch
        n = self.k.shape[2] if slots is None else min(int(slots), self.k.shape[2])

        def take(t):
            if units is None:
                return t[:, :, :n]
            return torch.stack([t[b, j, :n] for b, j in units])[:, None]

        k = take(self.k).cpu().numpy()
        v = take(self.v).cpu().numpy()
        if self.dtype == HIKV_BF16:
            k = k.view(np.uint16)
            v = v.view(np.uint16)
        ln = self.len.cpu().numpy()
        if units is not None:
            ln = np.array([[ln[b, j]] for b, j in units], dtype=ln.dtype)
        return dict(k=np.ascontiguousarray(k), v=np.ascontiguousarray(v),
                    pos=np.ascontiguousarray(take(self.pos).cpu().numpy()),
                    imp=np.ascontiguousarray(take(self.imp).cpu().numpy()), len=ln)

    def load(self, state: dict):
        """Overwrite the device state with a host state of the same shape."""
        for name in ("k", "v"):
            src = self.torch.from_numpy(np.ascontiguousarray(state[name]))
            if state[name].dtype == np.uint16:
                src = src.view(self.torch.int16)
            getattr(self, name).copy_(src)
        for name in ("pos", "imp", "len"):
            getattr(self, name).copy_(self.torch.from_numpy(np.ascontiguousarray(state[name])))
        self.evict.zero_()  # a host state has no eviction pending


def to_device(a: np.ndarray, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.int16)
    return t.to(device)


def workspace(shape: hikv_shape, policy: hikv_policy, device="cuda"):
    import torch
    n = hikv_workspace_bytes(shape, policy)
    if n == 0:
        raise RuntimeError("invalid shape/policy for workspace sizing")
    return torch.zeros(n, dtype=torch.uint8, device=device)
