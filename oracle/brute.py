"""Pure-Python brute force for tiny attention cases (test infrastructure).

Only the test suite may import this module. It restates attention one scalar
at a time with math.exp and math.fsum (exactly rounded sums), with no NumPy
arithmetic, so that the vectorised oracle is checked against an independent
evaluation on tiny shapes. Semantics are those of the oracle module: scores
scale*q.k, keys hidden by the mask left out of the softmax, natural-log lse,
O = 0 and lse = -inf for a row that sees no key.

Source: the-ai.news, "Snelle attention-kernels en operatorfusie versnellen
AI-modellen", section "FlashAttention-type aandacht en gepagineerde aandacht"
(score matrix per head, softmax, weighted sum of values; paged positions
translated through the block table).
"""
from __future__ import annotations

import math

import numpy as np


def _row(qi, keys, vals, scale):
    """One query row against a list of visible (key, value) vectors."""
    if not keys:
        return [0.0] * len(qi), -math.inf
    s = [scale * math.fsum(a * b for a, b in zip(qi, kj)) for kj in keys]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    l = math.fsum(e)
    out = [math.fsum(e[j] * vals[j][d] for j in range(len(keys))) / l for d in range(len(qi))]
    return out, m + math.log(l)


def prefill(q, k, v, scale, causal=False, seq_lens=None):
    q, k, v = (np.asarray(a, dtype=np.float64).tolist() for a in (q, k, v))
    scale = float(np.float32(scale))
    B, Hq, Tq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, Tk = len(k[0]), len(k[0][0])
    G = Hq // Hkv
    o = [[[[0.0] * D for _ in range(Tq)] for _ in range(Hq)] for _ in range(B)]
    lse = [[[-math.inf] * Tq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        Lq = Tq if seq_lens is None else int(seq_lens[b])
        Lk = Tk if seq_lens is None else int(seq_lens[b])
        for h in range(Hq):
            kh = h // G
            for i in range(Lq):
                vis = [j for j in range(Lk) if (not causal) or j <= i + (Lk - Lq)]
                out, ls = _row(q[b][h][i], [k[b][kh][j] for j in vis], [v[b][kh][j] for j in vis], scale)
                o[b][h][i] = out
                lse[b][h][i] = ls
    return np.array(o), np.array(lse)


def decode_paged(q, k_cache, v_cache, block_table, ctx_lens, scale):
    q = np.asarray(q, dtype=np.float64).tolist()
    kc = np.asarray(k_cache, dtype=np.float64).tolist()
    vc = np.asarray(v_cache, dtype=np.float64).tolist()
    bt = np.asarray(block_table).tolist()
    scale = float(np.float32(scale))
    B, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv, blk = len(kc[0]), len(kc[0][0])
    G = Hq // Hkv
    o = [[None] * Hq for _ in range(B)]
    lse = [[None] * Hq for _ in range(B)]
    for b in range(B):
        L = int(ctx_lens[b])
        for h in range(Hq):
            kh = h // G
            keys = [kc[bt[b][t // blk]][kh][t % blk] for t in range(L)]
            vals = [vc[bt[b][t // blk]][kh][t % blk] for t in range(L)]
            o[b][h], lse[b][h] = _row(q[b][h], keys, vals, scale)
    return np.array(o), np.array(lse)


def prefill_paged(q, k_cache, v_cache, block_table, ctx_lens, q_lens, scale, causal=True):
    """Chunked prefill through the paged cache, one scalar at a time."""
    q = np.asarray(q, dtype=np.float64).tolist()
    kc = np.asarray(k_cache, dtype=np.float64).tolist()
    vc = np.asarray(v_cache, dtype=np.float64).tolist()
    bt = np.asarray(block_table).tolist()
    scale = float(np.float32(scale))
    B, Hq, Tq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, blk = len(kc[0]), len(kc[0][0])
    G = Hq // Hkv
    o = [[[[0.0] * D for _ in range(Tq)] for _ in range(Hq)] for _ in range(B)]
    lse = [[[-math.inf] * Tq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        L = int(ctx_lens[b])
        n = Tq if q_lens is None else int(q_lens[b])
        for h in range(Hq):
            kh = h // G
            for i in range(n):
                pos = L - n + i  # this query's own position
                vis = [t for t in range(L) if (not causal) or t <= pos]
                keys = [kc[bt[b][t // blk]][kh][t % blk] for t in vis]
                vals = [vc[bt[b][t // blk]][kh][t % blk] for t in vis]
                o[b][h][i], lse[b][h][i] = _row(q[b][h][i], keys, vals, scale)
    return np.array(o), np.array(lse)
