"""HiKV's chunk-based selection against a global sort of P (the HiKV page,
Sec. III-C and Fig. 7), measured on the seeded synthetic workload.

For a query and N live tokens, P is the softmax of the reduced logits (the
B_II = D / r_II channels of largest |q|).  The chunked selection keeps the
B_II largest entries of each chunk of D tokens in position order; the global
selection keeps the same number of largest entries of the whole P.  Recall
is the share of the global selection that the chunked one also keeps.  The
pages report it on real model activations (over 95 % at r_I = 4, r_II = 2);
these inputs are synthetic, so the values printed here describe this data
only.  What holds on any data: recall is 1 when N <= D (one chunk) and when
r_II = 1 (every chunk keeps everything).
"""

import math

import numpy as np

from importance_aware_kv_amd import workloads as W


def chunk_recall(q, keys, pos, r):
    D = q.shape[0]
    E = np.argsort(-np.abs(q), kind="stable")[:r]
    s = (keys[:, E] @ q[E]) / math.sqrt(D)
    p = np.exp(s - s.max())
    p /= p.sum()
    order = np.argsort(pos, kind="stable")
    chunk = set()
    for c0 in range(0, len(pos), D):
        ids = order[c0:c0 + D]
        chunk.update(ids[np.argsort(-p[ids], kind="stable")[:min(r, len(ids))]].tolist())
    glob = set(np.argsort(-p, kind="stable")[:len(chunk)].tolist())
    return len(chunk & glob) / len(glob)


def test_chunk_recall_sweep():
    w = W.workload("hikv_hier", ctx=4096, steps=1, batch=1)
    d = W.generate(w)
    D, G = w.head_dim, w.group
    rows = []
    for r_I in (1, 2, 4):
        N = w.ctx // r_I                                   # tokens after Stage I
        for r_II in (1, 2, 4):
            r = D // r_II
            rec = []
            for j in range(w.n_kv_heads):
                keys = W.bf16_bits_to_f32(d["k"][0, j, :w.ctx]).astype(np.float64)
                pos = d["pos"][0, j, :w.ctx]
                keep = np.sort(np.random.Generator(np.random.PCG64(j)).choice(w.ctx, N, replace=False))
                for g in range(G):
                    q = W.bf16_bits_to_f32(d["q"][0, 0, j * G + g]).astype(np.float64)
                    rec.append(chunk_recall(q, keys[keep], pos[keep], r))
            rows.append((r_I, r_II, N, float(np.mean(rec)), float(np.min(rec))))
            if r_II == 1:
                assert min(rec) == 1.0
    print("\n r_I r_II     N  mean recall  min recall")
    for r_I, r_II, N, m, mn in rows:
        print(f" {r_I:3d} {r_II:4d} {N:5d}  {m:11.4f}  {mn:10.4f}")
    assert all(0.0 < m <= 1.0 for *_, m, _ in rows)


def test_chunk_recall_is_one_within_one_chunk():
    rng = np.random.Generator(np.random.PCG64(3))
    for N in (1, 17, 128):
        keys = rng.standard_normal((N, 128))
        q = rng.standard_normal(128)
        pos = rng.permutation(N)
        for r in (1, 32, 64, 128):
            assert chunk_recall(q, keys, pos, r) == 1.0
