"""Error budgets of the GPU arithmetic against the float64 definition (test infrastructure).

This module is test infrastructure. Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import or run it; the library never does.
It shares no code with the HIP path.

The-ai.news page ("Snelle attention-kernels en operatorfusie versnellen
AI-modellen", opening paragraph) states that the fused forms change only the
order and the precision of the operations, not the function. These functions
turn that statement into a number per output element: the largest difference
between the exact result (oracle.py) and a computation that follows the
library's stated arithmetic, derived below from that arithmetic alone. The
parity tests allow max(stated tolerance, budget) per element; the five
measured workloads are held to the stated tolerance itself.

Arithmetic covered ("16-bit" form, every attention call except attn_fwd_fp8):
  * scores s_j = scale * q . k_j from exact 16-bit products summed in fp32;
  * p_j = 2^(x_j - m) with x_j = s_j log2(e) in fp32 and a running max m that
    may lag the true one (lazily moved; the terms computed under an earlier m
    are rescaled in fp32), so every p_j carries a relative error eta;
  * r_j = p_j rounded to the 16-bit type (relative error <= u, u = 2^-8 for
    bf16, 2^-11 for fp16; fp16 below 2^-14 has an absolute error <= 2^-25);
  * O = (sum_j r_j v_j) / (sum_j r_j), both sums in fp32, then rounded to the
    16-bit type. (The decode merges per-split results with fp32 weights; the
    weights' own relative error is added to eta.)
Since O divides by the sum of the weights it applies, O - O_exact =
sum_j (w'_j - w_j)(v_j - c) for any constant c (w the exact softmax weights,
w' the applied ones, both summing to 1), and |w'_j - w_j| <= w_j 2 zeta/(1 -
zeta) with zeta = (1 + eta)(1 + u) - 1. With c = O_exact:

  |dO_id| <= 2 zeta/(1 - zeta) * A_id                       (rounding of P)
           + [fp16] 2^-25 * Pmax_i * C_id * (1 + zeta)/(1 - zeta)
           + 2 gamma_n * B_id * (1 + zeta)/(1 - zeta)        (fp32 sums)
           + 6 * 2^-24 * |O_id|                              (division, scales)
  then + half a unit in the last place of the output type at |O| + the above,

A_id = sum_j P_ij |v_jd - O_id|, B_id = sum_j P_ij |v_jd|, C_id = sum_j
|v_jd - O_id| over the visible keys, Pmax_i = max_j P_ij (1/sum_j p_j <=
Pmax_i because the running max never exceeds the true one and the key that
set it has p = 1), gamma_n = n 2^-24 / (1 - n 2^-24). The kernels form each
sum per key tile (at most 64 terms, inside one matrix instruction or an
in-register reduction) and add the tiles' partial sums in fp32 one after
another (steps of at least 32 keys), so at most n = 64 + L/32 + rescales + 4
roundings lie on any term's path for L visible keys.

FP8 form (attn_fwd_fp8): the running max lags by at most 1 (log2 units), so
p_j <= 2; p_j 2^7 is rounded to E4M3 (relative error <= 2^-4 above 2^-13 in p,
absolute <= 2^-17 below), and O divides by the fp32 sum of the unrounded p:

  |dO_id| <= 2^-4 (1 + eta)/(1 - eta) * B_id + 2^-17 (1 + eta) Pmax_i * C'_id
           + 2 eta/(1 - eta) * A_id + (2 gamma_n + F8_DOT) * B_id (1 + 2^-3)
           + 6 * 2^-24 |O_id|
  then + half a unit in the last place of the output type,

with C'_id = sum_j |v_jd| over the visible keys. The fp8 matrix instruction
does not sum its 64 products in full fp32: its result is taken to lie within
F8_DOT = 2^-13 of sum |products| of the exact sum (measured on MI355X through
the library: at most 2^-15.2 at D = 64 and 2^-16.1 at D = 128 over 4096 random
E4M3 rows each; a GPU test keeps checking it), which enters eta through the
scores and the budget through each tile's P.V product. The 16-bit
instructions' sums measured at 2^-24 of sum |products|, inside gamma_D.

eta (relative error of an unrounded p_j): the fp32 dot product (gamma_D
times sum_e |q_e k_je|), the fp32 rounding of the scale and of the exponent
argument, and at most 2^-21 per evaluation of exp2 (v_exp_f32: about one unit
in the last place) for the exponential and each lazy rescale; the number of
rescales is at most 2 + (growth of the running max)/margin.

Tests pin these budgets: a float32 simulation of the stated arithmetic stays
inside them, on random and on adversarial inputs built to approach them, and
planted deviations from the arithmetic (coarser rounding of P, normalising by
the unrounded sum, a dropped key tile) exceed them.
"""
from __future__ import annotations

import numpy as np

from . import oracle as O
from .gemm import ulp16

__all__ = ["U16", "F8_DOT", "row_budget", "prefill", "prefill_rows", "decode_paged", "prefill_paged", "prefill_fp8_rows",
           "prefill_fp8", "fp8_model_row", "prefill_fp8_model_rows"]

U32 = 2.0 ** -24
U16 = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}
F8_DOT = 2.0 ** -13  # accuracy of the fp8 matrix instruction's dot products, relative to sum |products|
LAZY = {"16": 8.0, "fp8": 1.0}  # margin (log2 units) by which the running max may lag before it moves


def _gamma(n):
    n = np.asarray(n, dtype=np.float64)
    return n * U32 / (1.0 - n * U32)


def _n_sum(L, n_resc):
    """Roundings on a term's path through a tiled fp32 sum of L terms (see the module notes)."""
    return 64.0 + np.ceil(np.asarray(L, dtype=np.float64) / 32.0) + n_resc + 4.0


def _visible(rows, Lq, Lk, causal):
    j = np.arange(Lk)[None, :]
    vis = np.broadcast_to(rows[:, None] < Lq, (rows.shape[0], Lk)).copy()
    if causal:
        vis &= j <= rows[:, None] + (Lk - Lq)
    return vis


def row_budget(Q, K, V, P, o, vis, scale, dtype, form="16", merge=False):
    """Budget [n, D] for n query rows against their keys.

    Q [n, D] (the rows' queries), K / V [Lk, D] (keys / values, the row's visible ones marked in vis
    [n, Lk]), P [n, Lk] the exact softmax (0 where masked), o [n, D] the exact output; dtype is the
    output type ("bf16" / "fp16"); form "16" or "fp8"; merge adds the decode merge's weight error."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.where(vis.any(axis=0)[:, None], np.asarray(K, dtype=np.float64), 0.0)
    V = np.where(vis.any(axis=0)[:, None], np.asarray(V, dtype=np.float64), 0.0)
    n, D = o.shape
    Dq = Q.shape[1]
    L = vis.sum(axis=1).astype(np.float64)
    c = abs(float(np.float32(scale))) * np.log2(np.e)
    S = np.where(vis, np.abs(Q) @ np.abs(K).T, 0.0).max(axis=1, initial=0.0)   # max_j sum_e |q_e k_je|
    n_resc = 2.0 + 2.0 * c * S / LAZY[form]
    dot = F8_DOT if form == "fp8" else _gamma(Dq)
    eta = np.log(2.0) * c * S * (dot + 4 * U32) + (1.0 + n_resc) * (2.0 ** -21 + U32)
    if merge:
        eta = eta + 2.0 ** -20 * (4.0 + c * S)
    absV = np.abs(V)
    A = np.zeros((n, D))
    C = np.zeros((n, D))
    for r in range(n):  # sum_j P_j |v_jd - O_d| and sum_j |v_jd - O_d| over visible keys
        dv = np.abs(V[vis[r]] - o[r][None, :])
        A[r] = P[r, vis[r]] @ dv
        C[r] = dv.sum(axis=0)
    B = P @ absV
    Pmax = P.max(axis=1, initial=0.0)
    gam = 2.0 * _gamma(_n_sum(L, n_resc))[:, None]
    e = eta[:, None]
    if form == "16":
        u = U16[dtype]
        z = (1.0 + e) * (1.0 + u) - 1.0
        g = (1.0 + z) / (1.0 - z)
        b1 = 2.0 * z / (1.0 - z) * A + gam * B * g + 6 * U32 * np.abs(o)
        if dtype == "fp16":
            b1 = b1 + 2.0 ** -25 * Pmax[:, None] * C * g
    else:
        Cp = vis.astype(np.float64) @ absV
        b1 = (2.0 ** -4 * (1.0 + e) / (1.0 - e) * B + 2.0 ** -17 * (1.0 + e) * Pmax[:, None] * Cp
              + 2.0 * e / (1.0 - e) * A + (gam + F8_DOT) * B * (1.0 + 2.0 ** -3) + 6 * U32 * np.abs(o))
    return b1 + 0.5 * ulp16(np.abs(o) + b1, dtype)


def _head(qh, kh, vh, scale, causal, Lq, Lk, rows, dtype, form="16", merge=False):
    rows = np.asarray(rows, dtype=np.int64)
    o, lse, P = O.head_rows(qh, kh, vh, scale, causal, Lq, Lk, rows)
    vis = _visible(rows, Lq, Lk, causal)
    b = np.zeros_like(o)
    live = vis.any(axis=1)
    if live.any():
        r = rows[live]
        b[live] = row_budget(qh[r], kh[:Lk], vh[:Lk], P[live], o[live], vis[live], scale, dtype, form, merge)
    return b


def prefill(q, k, v, scale, causal=False, seq_lens=None, dtype="bf16", row_block=1024):
    """Budget [B, Hq, Tq, D] for attn_fwd (the arguments of oracle.prefill plus the output dtype)."""
    B, Hq, Tq, _ = q.shape
    Hkv, Tk, Dv = k.shape[1], k.shape[2], v.shape[3]
    G = Hq // Hkv
    out = np.zeros((B, Hq, Tq, Dv))
    for b in range(B):
        Lq, Lk = (Tq, Tk) if seq_lens is None else (int(seq_lens[b]), int(seq_lens[b]))
        for hq in range(Hq):
            for r0 in range(0, Tq, row_block):
                rows = np.arange(r0, min(Tq, r0 + row_block))
                out[b, hq, rows] = _head(q[b, hq], k[b, hq // G], v[b, hq // G], scale, causal, Lq, Lk, rows, dtype)
    return out


def prefill_rows(q, k, v, scale, causal, seq_lens, picks, dtype="bf16", form="16"):
    """Budget [n, D] for sampled outputs picks [n, 3] of (b, hq, i) (as oracle.prefill_rows)."""
    B, Hq, Tq, _ = q.shape
    Hkv, Tk, Dv = k.shape[1], k.shape[2], v.shape[3]
    G = Hq // Hkv
    picks = np.asarray(picks, dtype=np.int64)
    out = np.zeros((picks.shape[0], Dv))
    for key in sorted({(int(b), int(h)) for b, h, _ in picks}):
        b, hq = key
        idx = np.nonzero((picks[:, 0] == b) & (picks[:, 1] == hq))[0]
        Lq, Lk = (Tq, Tk) if seq_lens is None else (int(seq_lens[b]), int(seq_lens[b]))
        out[idx] = _head(q[b, hq], k[b, hq // G], v[b, hq // G], scale, causal, Lq, Lk, picks[idx, 2], dtype, form)
    return out


def decode_paged(q, k_cache, v_cache, block_table, ctx_lens, scale, dtype="bf16"):
    """Budget [B, Hq, D] for the paged decode (as oracle.decode_paged; caches already dequantized for the
    E4M3 form). Includes the merge of per-split results."""
    B, Hq, _ = q.shape
    Hkv, Dv = k_cache.shape[1], v_cache.shape[3]
    G = Hq // Hkv
    out = np.zeros((B, Hq, Dv))
    for b in range(B):
        L = int(ctx_lens[b])
        for kvh in range(Hkv):
            K, V = O.gather_paged(k_cache, v_cache, block_table, L, b, kvh)
            for g in range(G):
                hq = kvh * G + g
                out[b, hq] = _head(q[b, hq][None, :], K, V, scale, False, 1, L, np.array([0]), dtype,
                                   merge=True)[0]
    return out


def prefill_paged(q, k_cache, v_cache, block_table, ctx_lens, q_lens, scale, causal=True, dtype="bf16"):
    """Budget [B, Hq, Tq, D] for the chunked prefill (as oracle.prefill_paged)."""
    B, Hq, Tq, _ = q.shape
    Hkv, Dv = k_cache.shape[1], v_cache.shape[3]
    G = Hq // Hkv
    out = np.zeros((B, Hq, Tq, Dv))
    for b in range(B):
        Lk = int(ctx_lens[b])
        Lq = Tq if q_lens is None else int(q_lens[b])
        for kvh in range(Hkv):
            K, V = O.gather_paged(k_cache, v_cache, block_table, Lk, b, kvh)
            for g in range(G):
                hq = kvh * G + g
                out[b, hq] = _head(q[b, hq], K, V, scale, causal, Lq, Lk, np.arange(Tq), dtype)
    return out


def prefill_fp8(qd, kd, vd, scale, causal=False, seq_lens=None, dtype="bf16", row_block=1024):
    """Budget [B, Hq, Tq, D] for attn_fwd_fp8 on the dequantized inputs qd, kd, vd (the scales applied)."""
    B, Hq, Tq, _ = qd.shape
    Hkv, Tk, Dv = kd.shape[1], kd.shape[2], vd.shape[3]
    G = Hq // Hkv
    out = np.zeros((B, Hq, Tq, Dv))
    for b in range(B):
        Lq, Lk = (Tq, Tk) if seq_lens is None else (int(seq_lens[b]), int(seq_lens[b]))
        for hq in range(Hq):
            for r0 in range(0, Tq, row_block):
                rows = np.arange(r0, min(Tq, r0 + row_block))
                out[b, hq, rows] = _head(qd[b, hq], kd[b, hq // G], vd[b, hq // G], scale, causal, Lq, Lk, rows,
                                         dtype, "fp8")
    return out


def prefill_fp8_rows(qd, kd, vd, scale, causal, seq_lens, picks, dtype="bf16"):
    """Budget [n, D] of attn_fwd_fp8 for sampled outputs (b, hq, i) on the dequantized inputs."""
    return prefill_rows(qd, kd, vd, scale, causal, seq_lens, picks, dtype, form="fp8")


def _e4m3(y):
    """E4M3 value of float64 magnitudes y (round to nearest even, saturating at 448): the oracle's codec."""
    from .fp8 import e4m3_to_float, float_to_e4m3
    return e4m3_to_float(float_to_e4m3(np.asarray(y, dtype=np.float64).astype(np.float32)))


def fp8_model_row(q, K, V, scale, tile=64, margin=1.0, pscale=7):
    """The FP8 prefill's arithmetic (reading R29) carried out in float64 for one query row over its
    visible keys K, V [L, D] (dequantized), plus the budget of what evaluating it in fp32 can change.

    Steps, in the kernel's order: keys in tiles of `tile`; for each tile the tile max of the exponent
    arguments x_j = scale q.k_j log2(e); the running max m moves to the tile max when that exceeds m by
    more than `margin`; p_j = 2^(x_j - m), earlier sums rescaled when m moves; p_j 2^pscale rounded to
    E4M3 (q_j); O = sum_j q_j v_j / sum_j p_j 2^pscale.

    Returns (o [D], budget [D], ambiguous). A key whose rounding could fall either way under the fp32
    error of its p (relative eta, as in row_budget) adds the difference of the two codes to the budget;
    a tile whose max lies within the fp32 error of the moving threshold makes the row ambiguous (the
    schedule itself could differ), and the caller then uses the worst-case budget instead."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L, D = V.shape
    c = abs(float(np.float32(scale))) * np.log2(np.e)
    x = (K @ q) * c * (1.0 if scale >= 0 else -1.0)
    S = float((np.abs(K) @ np.abs(q)).max(initial=0.0))
    dx = c * S * (F8_DOT + 6 * U32) + 2.0 ** -20  # error of an exponent argument (log2 units)
    n_resc = 2.0 + 2.0 * c * S / margin
    eta = np.log(2.0) * 2.0 * dx + (1.0 + n_resc) * (2.0 ** -21 + U32)
    m = -np.inf
    num = np.zeros(D)
    den = 0.0
    amb = np.zeros(D)   # sum over ambiguous keys of |code difference| |v|, in the current scale
    absnum = np.zeros(D)
    ambiguous = False
    for t0 in range(0, L, tile):
        xt = x[t0:t0 + tile]
        mt = xt.max()
        if abs(mt - (m + margin)) <= 2.0 * dx:
            ambiguous = True
        if mt > m + margin:
            alpha = 0.0 if not np.isfinite(m) else 2.0 ** (m - mt)
            num *= alpha
            den *= alpha
            amb *= alpha
            absnum *= alpha
            m = mt
        p = np.exp2(xt - m + pscale)
        qc = _e4m3(p)
        lo, hi = _e4m3(p * (1.0 - eta)), _e4m3(p * (1.0 + eta))
        Vt = V[t0:t0 + tile]
        num += qc @ Vt
        den += p.sum()
        absnum += qc @ np.abs(Vt)
        amb += (hi - lo) @ np.abs(Vt)
    o = num / den
    b1 = amb / den + (2.0 * eta / (1.0 - eta) + 2.0 * _gamma(_n_sum(L, n_resc)) + F8_DOT) * absnum / den * 1.01 \
        + 6 * U32 * np.abs(o)
    return o, b1, ambiguous


def prefill_fp8_model_rows(qd, kd, vd, scale, causal, seq_lens, picks, dtype="bf16"):
    """fp8_model_row for sampled outputs picks [n, 3] of (b, hq, i) of attn_fwd_fp8 on the dequantized
    inputs (keys visible under the prefill's mask, in order). Returns (o [n, D], budget [n, D] including
    the output rounding, ambiguous [n]); rows without a visible key give o = 0, budget 0."""
    B, Hq, Tq, _ = qd.shape
    Hkv, Tk, Dv = kd.shape[1], kd.shape[2], vd.shape[3]
    G = Hq // Hkv
    picks = np.asarray(picks, dtype=np.int64)
    o = np.zeros((picks.shape[0], Dv))
    bud = np.zeros((picks.shape[0], Dv))
    amb = np.zeros(picks.shape[0], dtype=bool)
    for n, (b, hq, i) in enumerate(picks):
        Lq, Lk = (Tq, Tk) if seq_lens is None else (int(seq_lens[b]), int(seq_lens[b]))
        if i >= Lq:
            continue
        nvis = Lk if not causal else min(Lk, int(i) + (Lk - Lq) + 1)
        if nvis <= 0:
            continue
        oo, b1, a = fp8_model_row(qd[b, hq, i], kd[b, hq // G, :nvis], vd[b, hq // G, :nvis], scale)
        o[n] = oo
        bud[n] = b1 + 0.5 * ulp16(np.abs(oo) + b1, dtype)
        amb[n] = a
    return o, bud, amb
