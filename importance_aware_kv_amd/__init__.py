"""Importance-aware KV cache decode step for AMD MI355X (gfx950).

One decode step of single-query GQA attention over a budgeted, slot-indexed
KV cache, fused with H2O/StreamingLLM-style importance eviction, per-head
budgets and a HiKV-style channel-selected Stage II.  The work runs in
hand-written HIP kernels behind the C ABI in include/hikv.h; this package is
the thin ctypes binding plus the seeded synthetic workloads.
"""
