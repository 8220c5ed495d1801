"""Seeded synthetic inputs for the importance-aware KV decode step.

This module only draws random numbers and packs them; it holds none of the
method's arithmetic (no attention, no scoring, no eviction).  Both the CPU
oracle (tests only) and the HIP path take their inputs from here, so the two
always see byte-identical data.

Workloads (shapes follow the pages; the data are synthetic stand-ins for the
pages' benchmark suites, which are not available):

* ``tiny``   -- batch 1, one head, D=64, fp32, 256-token prefill, budget 64 =
  4 sinks + 16 recent + 44 heavy hitters, 32 decode steps.  All values N(0,1).
* ``llama8b`` -- batch 8, 32 q / 8 KV heads (GQA), D=128, bf16, 8192-token
  prefill, budget 1024 (4 sinks, 128 recent), 128 steps.  Heavy-hitter
  planting: per (batch, KV head) a unit direction u; queries are
  sqrt(D)*u + N(0,I); 5% of the prompt positions (drawn without replacement
  from [4, ctx)) get keys 3*u + N(0,I); the 4 sink keys are 4*N(0,I).
* ``headkv32k`` -- batch 4, 32/8 heads, D=128, bf16, 32768-token prefill,
  per-KV-head budgets from one Dirichlet(0.5) draw scaled to a total of
  8*2048 and clamped to [64, 8192]; planting as ``llama8b``; 64 steps.
* ``longctx128k`` -- batch 2, 64/8 heads, D=128, bf16, 131072-token prefill,
  budget 4096 (4 sinks, 256 recent); keys k = rho*z with z ~ N(0,I) and
  rho ~ LogNormal(0, 0.5); q, v ~ N(0,I); 32 steps.  The full-attention
  variant uses budget = ctx + steps, so nothing is ever evicted.
* ``twostage`` -- ``llama8b`` shapes with Stage II on: r = 32 of 128 key
  channels chosen per q-head, exact softmax over the top 256 tokens.

Decode-step keys and values are N(0,I) in every workload; decode queries
follow the same recipe as the prefill queries of that workload.  Prompt
positions are 0..ctx-1 and decode step t carries position ctx+t.

bf16 values are produced by rounding fp32 draws to nearest-even and are
stored as their uint16 bit patterns.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

F32 = 0
BF16 = 1


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_x = x.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 22
    for i in range(0, flat_x.size, step):         # chunked: bounded temporaries
        u = flat_x[i:i + step].view(np.uint32)
        r = (u >> 16) & 1
        r += 0x7FFF
        r += u                                     # wraps only for NaN patterns, fixed below
        r >>= 16
        o = r.astype(np.uint16)
        o[np.isnan(flat_x[i:i + step])] = 0x7FC0
        flat_o[i:i + step] = o
    return out


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: int               # F32 or BF16
    ctx: int                 # prefilled tokens per (batch, KV head)
    steps: int               # decode steps
    budget_all: int          # used when budgets is None
    n_sink: int
    n_recent: int
    budgets: Optional[np.ndarray] = None   # int32 [batch][n_kv_heads] or None
    stage2_channels: int = 0
    stage2_tokens: int = 0
    recipe: str = "normal"   # normal | planted | lognormal_keys
    capacity: int = 0        # slots per (batch, KV head); 0 -> ctx + steps
    accumulate: int = 0      # 0: every live token accumulates; 1: only the recent window (HiKV dual bank)
    stage2_v: int = 0        # Stage II V side: 0 exact softmax over top-k_T; 1 HiKV's per-chunk top-r of P

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_units(self) -> int:
        return self.batch * self.n_kv_heads

    @property
    def cap(self) -> int:
        return self.capacity if self.capacity > 0 else self.ctx + self.steps

    @property
    def el(self) -> int:
        return 4 if self.dtype == F32 else 2

    def budget_array(self) -> np.ndarray:
        if self.budgets is not None:
            return np.ascontiguousarray(self.budgets, dtype=np.int32)
        return np.full((self.batch, self.n_kv_heads), self.budget_all, dtype=np.int32)


def dirichlet_budgets(seed: int, n_kv_heads: int, total: int, lo: int, hi: int) -> np.ndarray:
    """One Dirichlet(0.5) draw over KV heads -> integer budgets, clamped, not renormalised."""
    rng = np.random.Generator(np.random.PCG64(seed))
    w = rng.dirichlet(np.full(n_kv_heads, 0.5))
    return np.clip(np.rint(total * w), lo, hi).astype(np.int32)


def workload(name: str, *, ctx: Optional[int] = None, steps: Optional[int] = None,
             batch: Optional[int] = None, full: bool = False) -> Workload:
    """Named workload; ``ctx``/``steps``/``batch`` shrink it for quick tests."""
    if name == "tiny":
        w = Workload("tiny", 1000, 1, 1, 1, 64, F32, 256, 32, 64, 4, 16)
    elif name == "llama8b":
        w = Workload("llama8b", 1001, 8, 32, 8, 128, BF16, 8192, 128, 1024, 4, 128,
                     recipe="planted")
    elif name == "headkv32k":
        b = dirichlet_budgets(1002 + 7919, 8, 8 * 2048, 64, 8192)
        w = Workload("headkv32k", 1002, 4, 32, 8, 128, BF16, 32768, 64, 0, 4, 128,
                     budgets=np.tile(b, (4, 1)), recipe="planted")
    elif name == "longctx128k":
        w = Workload("longctx128k", 1003, 2, 64, 8, 128, BF16, 131072, 32, 4096, 4, 256,
                     recipe="lognormal_keys")
    elif name == "hikv_dualbank":
        # HiKV Stage I on its evaluation prompt length (4096): B_I = L_p / r_I
        # with r_I = 4, split into a recent bank and an important bank of
        # B_I / 2 each, no sinks; a serving batch of 8.
        w = Workload("hikv_dualbank", 1005, 8, 32, 8, 128, BF16, 4096, 128, 1024, 0, 512,
                     recipe="planted", accumulate=1)
    elif name == "hikv_hier":
        # HiKV's two stages together, on its evaluation prompt length: the
        # dual bank (B_I = 4096 / 4, banks of 512, no sinks) and Stage II
        # with r_II = 4 (B_II = 32 channels of q, 32 tokens per chunk of 128
        # entries of P).
        w = Workload("hikv_hier", 1006, 8, 32, 8, 128, BF16, 4096, 128, 1024, 0, 512,
                     stage2_channels=32, recipe="planted", accumulate=1, stage2_v=1)
    elif name == "twostage":
        w = Workload("twostage", 1004, 8, 32, 8, 128, BF16, 8192, 128, 1024, 4, 128,
                     stage2_channels=32, stage2_tokens=256, recipe="planted")
    else:
        raise KeyError(name)
    if ctx is not None:
        w.ctx = ctx
    if steps is not None:
        w.steps = steps
    if batch is not None:
        w.batch = batch
        if w.budgets is not None:
            w.budgets = w.budgets[:batch]
    if full:
        w.name += "_full"
        w.budget_all = w.ctx + w.steps
        w.budgets = None
    return w


WORKLOAD_NAMES = ("tiny", "llama8b", "headkv32k", "longctx128k", "twostage", "hikv_dualbank", "hikv_hier")


def _pack(x: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    return bf16_bits(x)


def generate(w: Workload):
    """Draw the prefilled cache and every decode step's q, k, v.

    Returns a dict of numpy arrays:
      k, v        [B][Hkv][cap][D]  (uint16 bf16 bits or float32); slots >= ctx are zero
      pos         int32 [B][Hkv][cap]  (prompt positions 0..ctx-1, -1 beyond)
      imp         float32 [B][Hkv][cap] zeros
      len         int32 [B][Hkv] = ctx
      q           [steps][B][Hq][D]
      k_new, v_new [steps][B][Hkv][D]
      new_pos     int32 [steps][B]
      budget      int32 [B][Hkv]
    """
    rng = np.random.Generator(np.random.PCG64(w.seed))
    B, Hq, Hkv, D, ctx, cap, T = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, w.cap, w.steps
    G = w.group
    f32 = np.float32

    kf = rng.standard_normal((B, Hkv, ctx, D), dtype=f32)
    vf = rng.standard_normal((B, Hkv, ctx, D), dtype=f32)
    u = None
    if w.recipe == "planted":
        u = rng.standard_normal((B, Hkv, D), dtype=f32)
        u /= np.linalg.norm(u, axis=-1, keepdims=True)
        n_plant = int(round(0.05 * ctx))
        for b in range(B):
            for j in range(Hkv):
                if ctx > 4 and n_plant > 0:
                    idx = rng.choice(np.arange(4, ctx), size=min(n_plant, ctx - 4), replace=False)
                    kf[b, j, idx] += 3.0 * u[b, j]
        ns = min(4, ctx)
        kf[:, :, :ns] *= 4.0
    elif w.recipe == "lognormal_keys":
        rho = rng.lognormal(0.0, 0.5, size=(B, Hkv, ctx, 1)).astype(f32)
        kf *= rho

    qf = rng.standard_normal((T, B, Hq, D), dtype=f32)
    if u is not None:
        qf += math.sqrt(D) * np.repeat(u, G, axis=1)[None]
    knf = rng.standard_normal((T, B, Hkv, D), dtype=f32)
    vnf = rng.standard_normal((T, B, Hkv, D), dtype=f32)

    if w.dtype == F32:
        k = np.zeros((B, Hkv, cap, D), dtype=f32)
        v = np.zeros((B, Hkv, cap, D), dtype=f32)
    else:
        k = np.zeros((B, Hkv, cap, D), dtype=np.uint16)
        v = np.zeros((B, Hkv, cap, D), dtype=np.uint16)
    k[:, :, :ctx] = _pack(kf, w.dtype)
    v[:, :, :ctx] = _pack(vf, w.dtype)
    del kf, vf
    pos = np.full((B, Hkv, cap), -1, dtype=np.int32)
    pos[:, :, :ctx] = np.arange(ctx, dtype=np.int32)
    return dict(
        k=k, v=v, pos=pos,
        imp=np.zeros((B, Hkv, cap), dtype=f32),
        len=np.full((B, Hkv), ctx, dtype=np.int32),
        q=_pack(qf, w.dtype), k_new=_pack(knf, w.dtype), v_new=_pack(vnf, w.dtype),
        new_pos=(ctx + np.arange(T, dtype=np.int32))[:, None].repeat(B, axis=1).copy(),
        budget=w.budget_array(),
    )


def random_cache(seed: int, B: int, Hq: int, Hkv: int, D: int, dtype: int, cap: int,
                 lens, imp_scale: float = 1.0, shuffle_pos: bool = True):
    """A cache in an arbitrary mid-run state: random rows, distinct positions
    in random slot order, random non-negative importance.  For edge-case tests."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = np.broadcast_to(np.asarray(lens, dtype=np.int32), (B, Hkv)).copy()
    kf = rng.standard_normal((B, Hkv, cap, D), dtype=np.float32)
    vf = rng.standard_normal((B, Hkv, cap, D), dtype=np.float32)
    pos = np.full((B, Hkv, cap), -1, dtype=np.int32)
    imp = np.zeros((B, Hkv, cap), dtype=np.float32)
    newest = int(lens.max()) + 8
    for b in range(B):
        for j in range(Hkv):
            n = int(lens[b, j])
            ns = min(4, n)
            rest = rng.choice(np.arange(4, newest), size=n - ns, replace=False)
            p = np.concatenate([np.arange(ns), np.sort(rest)]).astype(np.int32)
            if shuffle_pos:
                p = rng.permutation(p)
            pos[b, j, :n] = p
            imp[b, j, :n] = (imp_scale * rng.exponential(1.0, size=n)).astype(np.float32)
    return dict(k=_pack(kf, dtype), v=_pack(vf, dtype), pos=pos, imp=imp, len=lens,
                newest=newest)


def random_step(seed: int, B: int, Hq: int, Hkv: int, D: int, dtype: int, new_pos):
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, Hq, D), dtype=np.float32)
    kn = rng.standard_normal((B, Hkv, D), dtype=np.float32)
    vn = rng.standard_normal((B, Hkv, D), dtype=np.float32)
    return dict(q=_pack(q, dtype), k_new=_pack(kn, dtype), v_new=_pack(vn, dtype),
                new_pos=np.broadcast_to(np.asarray(new_pos, dtype=np.int32), (B,)).copy())


def random_steps(seed: int, n: int, B: int, Hq: int, Hkv: int, D: int, dtype: int, first_pos: int):
    """n decode steps of random q, k, v (positions first_pos, first_pos + 1, ...),
    stacked on a leading step axis."""
    steps = [random_step(seed + 7919 * t, B, Hq, Hkv, D, dtype, first_pos + t) for t in range(n)]
    return {k: np.stack([s[k] for s in steps]) for k in steps[0]}
