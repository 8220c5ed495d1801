"""Algorithmic byte counts of the decode step (what the method must move).

Per decode step and per (batch, KV head) unit with L live tokens after the
append, the step reads every live K and V row (2*D*el bytes), reads the
position and reads + writes the importance of every live token (12 bytes);
it reads q (Hq*D*el per batch row), the new k and v, and writes the fp32
output; an eviction that relocates a row reads and writes one K row, one V
row, one position and one importance value.

The cache-size closed form is the one on "KV Cache Compression and Dynamic
Pruning in Production Serving", Sec. 1: M_KV = 2 * B * L * N_L * N_KV * D * P.
"""

from __future__ import annotations

import numpy as np


def kv_cache_bytes(batch: int, tokens: int, n_layers: int, n_kv_heads: int, head_dim: int,
                   bytes_per_elem: int) -> int:
    return 2 * batch * tokens * n_layers * n_kv_heads * head_dim * bytes_per_elem


def decode_step_bytes(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, el: int,
                      live_after_append, moves: int) -> int:
    """Bytes one decode step must move; live_after_append: per-unit token counts."""
    live = int(np.asarray(live_after_append, dtype=np.int64).sum())
    row = head_dim * el
    return (live * (2 * row + 12)
            + batch * n_q_heads * row          # q
            + batch * n_kv_heads * 2 * row     # new k, v
            + batch * n_q_heads * head_dim * 4 # fp32 output
            + moves * 2 * (2 * row + 8))       # relocated rows (read + write)


def attend_bytes(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, el: int,
                 live_after_append) -> int:
    """Bytes the attention launch must read: every live K and V row (the new
    token's row included) and the queries."""
    live = int(np.asarray(live_after_append, dtype=np.int64).sum())
    row = head_dim * el
    return live * 2 * row + batch * n_q_heads * row
