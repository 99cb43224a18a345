"""CPU oracle for fused scaled-dot-product attention (test infrastructure).

This module is test infrastructure. Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import or run it; the library never does.
It shares no code with the HIP path.

What it computes is the plain definition of attention, written out in float64
on the exact input values, with the T x T score matrix materialised:

    s_ij = scale * q_i . k_j          (scores, one row per query)
    s_ij = -inf where the mask hides key j from query i
    P_ij = exp(s_ij - max_j s_ij) / sum_j exp(s_ij - max_j s_ij)
    O_i  = sum_j P_ij v_j,   lse_i = ln sum_j exp(s_ij)

Sources: the-ai.news, "Snelle attention-kernels en operatorfusie versnellen
AI-modellen", section "FlashAttention-type aandacht en gepagineerde aandacht":
classic attention builds a T^2 score matrix per head; FlashAttention reaches
the same result block by block (the page's opening paragraph says the fused
forms leave the mathematical function unchanged up to operation order and
precision). The paged cache of the same section stores keys/values in
fixed-size blocks with a table that maps logical positions to physical blocks;
the kernel translates every position through that table. The block size of
16 tokens is the vLLM example in that section.

Readings where the pages are silent (each is listed in the design notes):
  * scale is a float32 argument; the oracle uses float64(float32(scale)).
  * natural-log lse; an empty row (no visible key) gives O = 0, lse = -inf.
  * causal mask is bottom-right aligned and inclusive: key j is visible to
    query i iff j <= i + (Lk - Lq).
  * ragged batches use a padded [B, H, Tmax, D] layout plus seq_lens[b],
    applied to queries and keys alike (self-attention, Tq == Tk); rows
    i >= seq_lens[b] are padding (O = 0, lse = -inf).
  * GQA: query head hq reads kv head hq // (Hq // Hkv).
  * decode: ctx_lens[b] counts every cached token including the current one;
    the single query sees positions 0 .. ctx_lens[b]-1.

Layouts: prefill q,o [B,Hq,Tq,D], k,v [B,Hkv,Tk,D]; decode q,o [B,Hq,D],
k_cache,v_cache [num_blocks,Hkv,block,D], block_table [B,max_blocks],
ctx_lens [B].
"""
from __future__ import annotations

import numpy as np

__all__ = ["scale64", "head_rows", "prefill", "prefill_rows", "probs", "decode_paged",
           "gather_paged", "combine", "prefill_paged", "cache_append"]


def scale64(scale: float) -> float:
    """The scale the library receives (float32), as a float64."""
    return float(np.float32(scale))


def _visible(i: np.ndarray, Lq: int, Lk: int, causal: bool) -> np.ndarray:
    """Boolean [len(i), Lk]: key j visible to query row i (rows i < Lq only)."""
    j = np.arange(Lk)[None, :]
    vis = np.ones((i.shape[0], Lk), dtype=bool)
    if causal:
        vis &= j <= (i[:, None] + (Lk - Lq))
    return vis


def head_rows(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, scale: float, causal: bool,
              Lq: int, Lk: int, rows: np.ndarray):
    """Attention for some query rows of one head (the definition, in float64).

    qh [Tq,D], kh/vh [Tk,D] for the head's kv head; rows = query indices.
    Keys j >= Lk are outside the sequence and take no part (the padding may
    hold anything, NaN included). Returns (o [n,D], lse [n], P [n,Lk]).
    """
    rows = np.asarray(rows, dtype=np.int64)
    n, Dv = rows.shape[0], vh.shape[1]
    o = np.zeros((n, Dv), dtype=np.float64)
    lse = np.full(n, -np.inf, dtype=np.float64)
    P = np.zeros((n, max(Lk, 0)), dtype=np.float64)
    live = rows < Lq
    if Lk <= 0 or not live.any():
        return o, lse, P
    r = rows[live]
    Q = qh[r].astype(np.float64)
    K = kh[:Lk].astype(np.float64)
    V = vh[:Lk].astype(np.float64)
    s = scale64(scale) * (Q @ K.T)                       # the score rows
    vis = _visible(r, Lq, Lk, causal)
    s = np.where(vis, s, -np.inf)                        # mask by selection
    m = s.max(axis=1)
    nonempty = m > -np.inf
    e = np.zeros_like(s)
    e[nonempty] = np.exp(s[nonempty] - m[nonempty, None])
    l = e.sum(axis=1)
    p = np.zeros_like(s)
    p[nonempty] = e[nonempty] / l[nonempty, None]
    out = p @ V
    ls = np.full(r.shape[0], -np.inf)
    ls[nonempty] = m[nonempty] + np.log(l[nonempty])
    out[~nonempty] = 0.0
    o[live] = out
    lse[live] = ls
    P[live] = p
    return o, lse, P


def _lens(B, Tq, Tk, seq_lens):
    if seq_lens is None:
        return [(Tq, Tk)] * B
    if Tq != Tk:
        raise ValueError("seq_lens requires Tq == Tk")
    return [(int(L), int(L)) for L in np.asarray(seq_lens)]


def prefill(q, k, v, scale, causal=False, seq_lens=None, row_block=2048):
    """Full prefill attention. Returns (o [B,Hq,Tq,D], lse [B,Hq,Tq]) in float64."""
    B, Hq, Tq, _ = q.shape
    Hkv, Tk, Dv = k.shape[1], k.shape[2], v.shape[3]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    o = np.zeros((B, Hq, Tq, Dv), dtype=np.float64)
    lse = np.full((B, Hq, Tq), -np.inf, dtype=np.float64)
    for b, (Lq, Lk) in enumerate(_lens(B, Tq, Tk, seq_lens)):
        for hq in range(Hq):
            kvh = hq // G
            for r0 in range(0, Tq, row_block):
                rows = np.arange(r0, min(Tq, r0 + row_block))
                ob, lb, _ = head_rows(q[b, hq], k[b, kvh], v[b, kvh], scale, causal, Lq, Lk, rows)
                o[b, hq, rows] = ob
                lse[b, hq, rows] = lb
    return o, lse


def prefill_rows(q, k, v, scale, causal, seq_lens, picks):
    """Sampled outputs: picks is an int array [n,3] of (b, hq, i). Returns (o [n,D], lse [n])."""
    B, Hq, Tq, _ = q.shape
    Hkv, Tk, Dv = k.shape[1], k.shape[2], v.shape[3]
    G = Hq // Hkv
    lens = _lens(B, Tq, Tk, seq_lens)
    picks = np.asarray(picks, dtype=np.int64)
    o = np.zeros((picks.shape[0], Dv))
    lse = np.zeros(picks.shape[0])
    # group by head so each head's K/V is upcast once
    order = np.lexsort((picks[:, 2], picks[:, 1], picks[:, 0]))
    start = 0
    while start < len(order):
        b, hq = picks[order[start], 0], picks[order[start], 1]
        end = start
        while end < len(order) and picks[order[end], 0] == b and picks[order[end], 1] == hq:
            end += 1
        idx = order[start:end]
        Lq, Lk = lens[b]
        ob, lb, _ = head_rows(q[b, hq], k[b, hq // G], v[b, hq // G], scale, causal, Lq, Lk,
                              picks[idx, 2])
        o[idx] = ob
        lse[idx] = lb
        start = end
    return o, lse


def probs(q, k, v, scale, causal=False, seq_lens=None):
    """The softmax matrix P [B,Hq,Tq,Tk] (small shapes only; zero where masked)."""
    B, Hq, Tq, D = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    P = np.zeros((B, Hq, Tq, Tk))
    for b, (Lq, Lk) in enumerate(_lens(B, Tq, Tk, seq_lens)):
        for hq in range(Hq):
            _, _, p = head_rows(q[b, hq], k[b, hq // G], v[b, hq // G], scale, causal, Lq, Lk,
                                np.arange(Tq))
            P[b, hq, :, :Lk] = p
    return P


def gather_paged(k_cache, v_cache, block_table, ctx_len, b, kvh):
    """Keys/values of sequence b, kv head kvh, positions 0..ctx_len-1, via the block table.

    Position t lives in physical block block_table[b, t // block] at slot t % block.
    """
    block = k_cache.shape[2]
    t = np.arange(int(ctx_len))
    phys = np.asarray(block_table)[b, t // block]
    if t.size and (phys < 0).any():
        raise ValueError("block table entry < 0 inside the context")
    return k_cache[phys, kvh, t % block], v_cache[phys, kvh, t % block]


def decode_paged(q, k_cache, v_cache, block_table, ctx_lens, scale):
    """One-token decode through the paged cache. Returns (o [B,Hq,D], lse [B,Hq]) in float64.

    The query is the newest position, so every cached position 0..ctx-1 is
    visible: no further mask applies.
    """
    B, Hq, _ = q.shape
    Hkv, Dv = k_cache.shape[1], v_cache.shape[3]
    G = Hq // Hkv
    o = np.zeros((B, Hq, Dv))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        L = int(ctx_lens[b])
        for kvh in range(Hkv):
            K, V = gather_paged(k_cache, v_cache, block_table, L, b, kvh)
            for g in range(G):
                hq = kvh * G + g
                ob, lb, _ = head_rows(q[b, hq][None, :], K, V, scale, False, 1, L, np.array([0]))
                o[b, hq] = ob[0]
                lse[b, hq] = lb[0]
    return o, lse


def combine(o_parts, lse_parts):
    """Merge attention results computed over disjoint key subsets.

    With lse_s = ln sum_{j in S} exp(s_j) and O_s the softmax-weighted mean of
    v over subset S, the result over the union is lse = ln sum_s exp(lse_s)
    and O = sum_s exp(lse_s - lse) O_s: a restatement of the softmax
    statistics update that blockwise attention performs. Empty parts carry
    lse = -inf and contribute nothing.
    """
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    o_parts = np.asarray(o_parts, dtype=np.float64)
    M = lse_parts.max(axis=0)
    fin = np.isfinite(M)
    Ms = np.where(fin, M, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - Ms), 0.0)
    W = w.sum(axis=0)
    lse = np.where(fin, Ms + np.log(np.where(fin, W, 1.0)), -np.inf)
    wn = np.where(fin, w / np.where(fin, W, 1.0), 0.0)
    o = (wn[..., None] * o_parts).sum(axis=0)
    return o, lse


def prefill_paged(q, k_cache, v_cache, block_table, ctx_lens, q_lens, scale, causal=True):
    """Chunked prefill through the paged cache. Returns (o [B,Hq,Tq,D], lse [B,Hq,Tq]).

    Row i of q[b] (i < q_lens[b]) is position ctx_lens[b] - q_lens[b] + i of
    sequence b: the newest q_lens[b] positions, whose keys/values are already
    in the cache. Keys/values are positions 0 .. ctx_lens[b]-1, read through
    the block table. With causal, row i sees keys j <= i + (ctx - q_len) (the
    bottom-right alignment of the prefill definition); rows >= q_lens[b] are
    padding (O = 0, lse = -inf). q_lens None means every row is a query.
    """
    B, Hq, Tq, _ = q.shape
    Hkv, Dv = k_cache.shape[1], v_cache.shape[3]
    G = Hq // Hkv
    o = np.zeros((B, Hq, Tq, Dv))
    lse = np.full((B, Hq, Tq), -np.inf)
    for b in range(B):
        Lk = int(ctx_lens[b])
        Lq = Tq if q_lens is None else int(q_lens[b])
        if Lq > Lk:
            raise ValueError("q_lens[b] > ctx_lens[b]")
        for kvh in range(Hkv):
            K, V = gather_paged(k_cache, v_cache, block_table, Lk, b, kvh)
            for g in range(G):
                hq = kvh * G + g
                ob, lb, _ = head_rows(q[b, hq], K, V, scale, causal, Lq, Lk, np.arange(Tq))
                o[b, hq] = ob
                lse[b, hq] = lb
    return o, lse


def cache_append(k_new, v_new, k_cache, v_cache, block_table, start_pos, new_lens=None):
    """Write new tokens into copies of the paged caches and return them.

    Token i < new_lens[b] of k_new[b] / v_new[b] ([B,Hkv,Tnew,D]) becomes
    position start_pos[b] + i of sequence b: physical block
    block_table[b, pos // block], slot pos % block (the address translation
    of the paged cache). Nothing else changes.
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    B, Hkv, Tnew, _ = k_new.shape
    block = kc.shape[2]
    table = np.asarray(block_table)
    for b in range(B):
        n = Tnew if new_lens is None else int(new_lens[b])
        pos = int(start_pos[b]) + np.arange(n)
        phys = table[b, pos // block]
        if n and (phys < 0).any():
            raise ValueError("block table entry < 0 where a token is written")
        for kvh in range(Hkv):
            kc[phys, kvh, pos % block] = k_new[b, kvh, :n]
            vc[phys, kvh, pos % block] = v_new[b, kvh, :n]
    return kc, vc
