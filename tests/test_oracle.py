"""Pins of the CPU oracle against what the definition and mathematics fix.

Each test checks the oracle against something other than itself: hand-derived
worked examples (tests/golden), a pure-Python brute force, a library routine
(torch's scaled_dot_product_attention on CPU in float64, the routine the
fast-attention page names), closed forms, invariants and the split/merge
identity. A planted-mistake test shows that plausible bugs in the oracle are
caught by these pins.
"""
import json
import math
import os

import numpy as np
import pytest

import workloads as W
from oracle import brute
from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "attention_worked_examples.json")
RNG = np.random.default_rng(1234)


def _arr(x):
    return np.array(x, dtype=np.float64)


def _rand(*shape, rng=None):
    rng = rng or RNG
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- worked examples
def _golden_cases():
    with open(GOLDEN) as f:
        data = json.load(f)
    assert "Snelle attention-kernels" in data["citation"]
    return data["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_worked_examples(case):
    if case["kind"] == "prefill":
        o, lse = O.prefill(_arr(case["q"]), _arr(case["k"]), _arr(case["v"]), case["scale"],
                           causal=case["causal"], seq_lens=case["seq_lens"])
    else:
        o, lse = O.decode_paged(_arr(case["q"]), _arr(case["k_cache"]), _arr(case["v_cache"]),
                                np.array(case["block_table"]), np.array(case["ctx_lens"]), case["scale"])
    exp_lse = np.array(case["lse"], dtype=object)
    exp_lse = np.vectorize(lambda x: -math.inf if x == "-inf" else float(x))(exp_lse).astype(np.float64)
    np.testing.assert_allclose(o, _arr(case["o"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, exp_lse, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P-1 brute force
@pytest.mark.parametrize("B,Hq,Hkv,Tq,Tk,D,causal,ragged", [
    (1, 1, 1, 5, 5, 3, False, False),
    (2, 4, 2, 7, 7, 4, True, False),
    (2, 2, 1, 9, 9, 2, False, True),
    (2, 4, 4, 6, 6, 3, True, True),
    (1, 2, 1, 3, 8, 4, True, False),   # Tq < Tk: bottom-right causal
    (1, 2, 2, 8, 3, 2, True, False),   # Tq > Tk: early rows see no key
])
def test_brute_force_prefill(B, Hq, Hkv, Tq, Tk, D, causal, ragged):
    rng = np.random.default_rng(B * 100 + Tq * 10 + Tk)
    q, k, v = _rand(B, Hq, Tq, D, rng=rng), _rand(B, Hkv, Tk, D, rng=rng), _rand(B, Hkv, Tk, D, rng=rng)
    seq = rng.integers(1, Tq + 1, B) if ragged else None
    scale = 0.7
    o1, l1 = O.prefill(q, k, v, scale, causal, seq)
    o2, l2 = brute.prefill(q, k, v, scale, causal, seq)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def test_brute_force_decode():
    rng = np.random.default_rng(7)
    B, Hq, Hkv, D, blk, NB = 3, 4, 2, 3, 4, 9
    kc, vc = _rand(NB, Hkv, blk, D, rng=rng), _rand(NB, Hkv, blk, D, rng=rng)
    q = _rand(B, Hq, D, rng=rng)
    ctx = np.array([5, 1, 12])
    table = np.array([[3, 7, -1], [0, -1, -1], [8, 1, 2]])
    o1, l1 = O.decode_paged(q, kc, vc, table, ctx, 0.9)
    o2, l2 = brute.decode_paged(q, kc, vc, table, ctx, 0.9)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P-2 library routine
def _sdpa_fp64(q, k, v, scale, causal, seq_lens, rows=None):
    """torch SDPA (CPU, float64) with GQA expanded and an explicit boolean mask."""
    import torch
    F = torch.nn.functional
    B, Hq, Tq, D = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Hq, Tq if rows is None else len(rows), D))
    for b in range(B):
        L = None if seq_lens is None else int(seq_lens[b])
        Lk = Tk if L is None else L
        Lq = Tq if L is None else L
        r = np.arange(Lq) if rows is None else np.asarray(rows)
        qt = torch.from_numpy(np.ascontiguousarray(q[b][:, r].astype(np.float64)))
        kt = torch.from_numpy(np.ascontiguousarray(k[b][:, :Lk].astype(np.float64))).repeat_interleave(G, 0)
        vt = torch.from_numpy(np.ascontiguousarray(v[b][:, :Lk].astype(np.float64))).repeat_interleave(G, 0)
        j = torch.arange(Lk)[None, :]
        mask = torch.ones(len(r), Lk, dtype=torch.bool)
        if causal:
            mask = j <= (torch.from_numpy(r)[:, None] + (Lk - Lq))
        o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=O.scale64(scale))
        if rows is None:
            out[b, :, :Lq] = o.numpy()
        else:
            out[b] = o.numpy()
    return out


@pytest.mark.parametrize("case", [W.TINY, W.BERT, W.LLAMA], ids=lambda c: c.name)
def test_sdpa_cross_check_full(case):
    x = W.prefill_inputs(case)
    o, _ = O.prefill(x["q"], x["k"], x["v"], case.scale, case.causal, x["seq_lens"])
    ref = _sdpa_fp64(x["q"], x["k"], x["v"], case.scale, case.causal, x["seq_lens"])
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-10)


def test_sdpa_cross_check_long_sampled():
    """16384-token causal case: sampled rows of two heads (all rows would take minutes)."""
    case = W.LONG
    x = W.prefill_inputs(case)
    rows = np.array([0, 1, 127, 128, 4095, 8191, 12000, 16383])
    picks = np.array([(0, h, i) for h in (0, 31) for i in rows])
    o, _ = O.prefill_rows(x["q"], x["k"], x["v"], case.scale, True, None, picks)
    for hi, h in enumerate((0, 31)):
        q = x["q"][:, h:h + 1]
        kv = h // (case.Hq // case.Hkv)
        ref = _sdpa_fp64(q, x["k"][:, kv:kv + 1], x["v"][:, kv:kv + 1], case.scale, True, None, rows=rows)
        np.testing.assert_allclose(o[hi * len(rows):(hi + 1) * len(rows)], ref[0, 0], rtol=0, atol=1e-10)


def test_sdpa_cross_check_decode():
    case = W.DecodeCase("small decode", B=6, Hq=12, Hkv=2, D=128, dtype="bf16", ctx_lo=1, ctx_hi=300, seed=11)
    x = W.decode_inputs(case, nan_fill=True)
    o, _ = O.decode_paged(x["q"], x["k_cache"], x["v_cache"], x["block_table"], x["ctx_lens"], case.scale)
    for b in range(case.B):
        for kvh in range(case.Hkv):
            K, V = O.gather_paged(x["k_cache"], x["v_cache"], x["block_table"], x["ctx_lens"][b], b, kvh)
            g = case.Hq // case.Hkv
            q = x["q"][b, kvh * g:(kvh + 1) * g][None, :, None, :]
            ref = _sdpa_fp64(q, K[None, None], V[None, None], case.scale, False, None)
            np.testing.assert_allclose(o[b, kvh * g:(kvh + 1) * g], ref[0, :, 0], rtol=0, atol=1e-10)


# ---------------------------------------------------------------- closed forms
def test_single_key_returns_value():
    """P-3: Tk = 1 gives O = v0 exactly and lse = scale q.k0."""
    q, k, v = _rand(2, 3, 4, 8), _rand(2, 3, 1, 8), _rand(2, 3, 1, 8)
    o, lse = O.prefill(q, k, v, 0.3)
    np.testing.assert_array_equal(o, np.broadcast_to(v, o.shape))
    np.testing.assert_allclose(lse, O.scale64(0.3) * np.einsum("bhtd,bhd->bht", q, k[:, :, 0]), atol=1e-13)


def test_identical_keys_give_mean():
    """P-4: all keys equal -> O = mean of v, lse = s + ln n."""
    n = 37
    q = _rand(1, 2, 5, 16)
    k = np.broadcast_to(_rand(1, 2, 1, 16), (1, 2, n, 16)).copy()
    v = _rand(1, 2, n, 16)
    o, lse = O.prefill(q, k, v, 0.25)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), atol=1e-13)
    s = O.scale64(0.25) * np.einsum("bhtd,bhd->bht", q, k[:, :, 0])
    np.testing.assert_allclose(lse, s + math.log(n), atol=1e-12)


def test_scale_zero_pins_mask_geometry():
    """P-5: scale 0 -> mean of visible values, lse = ln(#visible): causal, bottom-right, ragged."""
    T = 40
    v = _rand(3, 2, T, 5)
    q, k = _rand(3, 2, T, 5), _rand(3, 2, T, 5)
    o, lse = O.prefill(q, k, v, 0.0, causal=True)
    csum = np.cumsum(v, axis=2) / np.arange(1, T + 1)[None, None, :, None]
    np.testing.assert_allclose(o, csum, atol=1e-12)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(np.arange(1, T + 1)), lse.shape), atol=1e-13)
    # ragged, causal and non-causal
    seq = np.array([40, 17, 1])
    o, lse = O.prefill(q, k, v, 0.0, causal=False, seq_lens=seq)
    for b, L in enumerate(seq):
        np.testing.assert_allclose(o[b, :, :L], np.broadcast_to(v[b, :, :L].mean(1, keepdims=True), (2, L, 5)),
                                   atol=1e-12)
        assert np.all(o[b, :, L:] == 0) and np.all(np.isneginf(lse[b, :, L:]))
        np.testing.assert_allclose(lse[b, :, :L], math.log(L), atol=1e-13)
    o, lse = O.prefill(q, k, v, 0.0, causal=True, seq_lens=seq)
    for b, L in enumerate(seq):
        np.testing.assert_allclose(o[b, :, :L], csum[b, :, :L], atol=1e-12)
    # bottom-right with Tq < Tk
    qs = q[:, :, :7]
    o, lse = O.prefill(qs, k, v, 0.0, causal=True)
    for i in range(7):
        n = i + (T - 7) + 1
        np.testing.assert_allclose(o[:, :, i], v[:, :, :n].mean(2), atol=1e-12)
        np.testing.assert_allclose(lse[:, :, i], math.log(n), atol=1e-13)
    # decode partial last block: ctx 35 on 16-token blocks
    kc, vc = _rand(5, 1, 16, 5), _rand(5, 1, 16, 5)
    table = np.array([[4, 0, 2, -1]])
    od, ld = O.decode_paged(_rand(1, 3, 5), kc, vc, table, np.array([35]), 0.0)
    allv = np.concatenate([vc[4, 0], vc[0, 0], vc[2, 0, :3]])
    np.testing.assert_allclose(od[0], np.broadcast_to(allv.mean(0), (3, 5)), atol=1e-12)
    np.testing.assert_allclose(ld, math.log(35), atol=1e-13)


def test_causal_row0_is_first_value():
    """P-6: causal row 0 sees only key 0."""
    q, k, v = _rand(2, 4, 9, 6), _rand(2, 2, 9, 6), _rand(2, 2, 9, 6)
    o, lse = O.prefill(q, k, v, 0.5, causal=True)
    np.testing.assert_array_equal(o[:, :, 0], np.repeat(v[:, :, 0], 2, axis=1))
    s = O.scale64(0.5) * np.einsum("bhd,bhd->bh", q[:, :, 0], np.repeat(k[:, :, 0], 2, axis=1))
    np.testing.assert_allclose(lse[:, :, 0], s, atol=1e-13)


# ---------------------------------------------------------------- invariants
def test_probability_rows_and_bounds():
    """P-7: rows of P sum to 1; O within the visible values' range; lse within [m, m + ln n]."""
    q, k, v = _rand(2, 4, 12, 6), _rand(2, 2, 12, 6), _rand(2, 2, 12, 6)
    seq = np.array([12, 5])
    for causal in (False, True):
        P = O.probs(q, k, v, 0.8, causal, seq)
        o, lse = O.prefill(q, k, v, 0.8, causal, seq)
        for b, L in enumerate(seq):
            np.testing.assert_allclose(P[b, :, :L].sum(-1), 1.0, atol=1e-13)
            assert np.all(P[b, :, L:] == 0) and np.all(P[b, :, :, L:] == 0)
            for h in range(4):
                kv = h // 2
                for i in range(L):
                    n = (i + 1) if causal else L
                    vv = v[b, kv, :n]
                    assert np.all(o[b, h, i] >= vv.min(0) - 1e-12) and np.all(o[b, h, i] <= vv.max(0) + 1e-12)
                    s = O.scale64(0.8) * (k[b, kv, :n] @ q[b, h, i])
                    assert s.max() - 1e-12 <= lse[b, h, i] <= s.max() + math.log(n) + 1e-12
                    if causal:
                        assert np.all(P[b, h, i, n:] == 0)


def test_key_value_permutation_invariance():
    """P-8: jointly permuting (k_j, v_j) pairs changes nothing without a mask."""
    q, k, v = _rand(1, 2, 10, 8), _rand(1, 2, 30, 8), _rand(1, 2, 30, 8)
    perm = RNG.permutation(30)
    o1, l1 = O.prefill(q, k, v, 0.4)
    o2, l2 = O.prefill(q, k[:, :, perm], v[:, :, perm], 0.4)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_key_shift_invariance():
    """P-9: k_j <- k_j + u leaves O unchanged and adds scale*(q.u) to lse."""
    q, k, v = _rand(1, 1, 16, 8), _rand(1, 1, 16, 8), _rand(1, 1, 16, 8)
    u = 3.0 * _rand(8)
    for causal in (False, True):
        o1, l1 = O.prefill(q, k, v, 0.6, causal)
        o2, l2 = O.prefill(q, k + u, v, 0.6, causal)
        np.testing.assert_allclose(o1, o2, atol=1e-11)
        np.testing.assert_allclose((l2 - l1)[0, 0], O.scale64(0.6) * (q[0, 0] @ u), atol=1e-11)


def test_gqa_equals_expanded_mha_and_ragged_equals_unpadded():
    """P-10: GQA = MHA on repeat_interleave'd K/V; ragged sequence b = unpadded run; NaN padding inert."""
    q, k, v = _rand(2, 6, 20, 4), _rand(2, 2, 20, 4), _rand(2, 2, 20, 4)
    o1, l1 = O.prefill(q, k, v, 0.5, True)
    o2, l2 = O.prefill(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), 0.5, True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    seq = np.array([20, 9])
    qn, kn, vn = q.copy(), k.copy(), v.copy()
    qn[1, :, 9:] = kn[1, :, 9:] = vn[1, :, 9:] = np.nan
    for causal in (False, True):
        o, lse = O.prefill(qn, kn, vn, 0.5, causal, seq)
        assert np.isfinite(o).all()
        ou, lu = O.prefill(q[1:, :, :9], k[1:, :, :9], v[1:, :, :9], 0.5, causal)
        np.testing.assert_allclose(o[1, :, :9], ou[0], atol=1e-13)
        np.testing.assert_allclose(lse[1, :, :9], lu[0], atol=1e-13)


def test_paged_equals_contiguous_and_decode_is_last_causal_row():
    """P-11: paged decode = the same cache gathered contiguously = last row of causal prefill."""
    case = W.DecodeCase("p11", B=4, Hq=6, Hkv=2, D=16, dtype="bf16", ctx_lo=1, ctx_hi=70, seed=3)
    x = W.decode_inputs(case, nan_fill=True)
    o, lse = O.decode_paged(x["q"], x["k_cache"], x["v_cache"], x["block_table"], x["ctx_lens"], case.scale)
    for b in range(case.B):
        L = int(x["ctx_lens"][b])
        K = np.stack([O.gather_paged(x["k_cache"], x["v_cache"], x["block_table"], L, b, h)[0] for h in range(2)])
        V = np.stack([O.gather_paged(x["k_cache"], x["v_cache"], x["block_table"], L, b, h)[1] for h in range(2)])
        assert np.isfinite(K).all() and np.isfinite(V).all()
        # a causal prefill whose last query is this decode query
        qp = np.zeros((1, 6, L, 16))
        qp[0, :, L - 1] = x["q"][b]
        op, lp = O.prefill(qp, K[None], V[None], case.scale, causal=True)
        np.testing.assert_allclose(o[b], op[0, :, L - 1], atol=1e-13)
        np.testing.assert_allclose(lse[b], lp[0, :, L - 1], atol=1e-13)


def test_split_combine_identity():
    """P-12: attention over A u B = lse-weighted merge of attention over A and over B."""
    q, k, v = _rand(1, 2, 7, 8), _rand(1, 2, 50, 8), _rand(1, 2, 50, 8)
    o, lse = O.prefill(q, k, v, 0.9)
    cuts = [0, 13, 13, 31, 50]  # includes an empty part
    parts = [O.prefill(q, k[:, :, a:b], v[:, :, a:b], 0.9) for a, b in zip(cuts[:-1], cuts[1:])]
    om, lm = O.combine([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(om, o, atol=1e-13)
    np.testing.assert_allclose(lm, lse, atol=1e-13)


def test_peaked_scores_one_hot():
    """P-13: a score ahead by >= 50 makes the row equal that value row; sharp rescaling across blocks."""
    T, D = 300, 8
    q = np.zeros((1, 1, 1, D)); q[..., 0] = 1.0
    k = _rand(1, 1, T, D); k[..., 0] = np.clip(k[..., 0], -1, 1)
    k[0, 0, 211, 0] = 60.0
    v = _rand(1, 1, T, D)
    o, lse = O.prefill(q, k, v, 1.0)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 211], atol=1e-18 + 1e-12)
    np.testing.assert_allclose(lse[0, 0, 0], 60.0, atol=1e-12)
    # scores of std ~8: result unchanged when keys are reversed (stable rescaling)
    q2 = 8 * _rand(1, 1, 4, D)
    o1, l1 = O.prefill(q2, k, v, 1.0)
    o2, l2 = O.prefill(q2, k[:, :, ::-1], v[:, :, ::-1], 1.0)
    np.testing.assert_allclose(o1, o2, atol=1e-12)


# ---------------------------------------------------------------- the workload generator
def test_workload_generator_shapes_and_rounding():
    x = W.prefill_inputs(W.BERT, nan_padding=True)
    assert x["q"].shape == (8, 12, 512, 64)
    assert x["seq_lens"].min() >= 64 and x["seq_lens"].max() <= 512
    b = int(np.argmin(x["seq_lens"]))
    assert np.isnan(x["k"][b, :, x["seq_lens"][b]:]).all()
    fin = x["q"][np.isfinite(x["q"])]
    assert np.array_equal(fin, fin.astype(np.float16).astype(np.float32))
    d = W.decode_inputs(W.QWEN)
    ctx, tab = d["ctx_lens"], d["block_table"]
    assert ctx.min() >= 512 and ctx.max() <= 4096
    nblk = (ctx + 15) // 16
    used = np.concatenate([tab[b, :n] for b, n in enumerate(nblk)])
    assert sorted(used.tolist()) == list(range(int(nblk.sum())))  # a permutation of the used blocks
    assert all((tab[b, n:] == -1).all() for b, n in enumerate(nblk))
    bf = d["k_cache"].view(np.uint32)
    assert np.all((bf & 0xFFFF) == 0)  # bf16 values
    assert W.prefill_flops(2, 32, 512, 512, 128, True) == 4 * 128 * 2 * 32 * 512 * 513 / 2


# ---------------------------------------------------------------- planted mistakes
def _mutants():
    """Plausible oracle bugs: (attribute of the oracle module to replace, replacement)."""
    real_rows = O.head_rows

    def vis_no_diag(i, Lq, Lk, causal):        # causal mask that hides the diagonal
        j = np.arange(Lk)[None, :]
        vis = np.ones((i.shape[0], Lk), dtype=bool)
        if causal:
            vis &= j < (i[:, None] + (Lk - Lq))
        return vis

    def vis_top_left(i, Lq, Lk, causal):       # top-left causal alignment
        j = np.arange(Lk)[None, :]
        vis = np.ones((i.shape[0], Lk), dtype=bool)
        if causal:
            vis &= j <= i[:, None]
        return vis

    def no_scale(qh, kh, vh, scale, causal, Lq, Lk, rows):      # forgets the scale
        return real_rows(qh, kh, vh, 1.0, causal, Lq, Lk, rows)

    def k_for_v(qh, kh, vh, scale, causal, Lq, Lk, rows):       # wrong operand in the PV product
        return real_rows(qh, kh, kh, scale, causal, Lq, Lk, rows)

    def log2_lse(qh, kh, vh, scale, causal, Lq, Lk, rows):      # base-2 logsumexp
        o, lse, p = real_rows(qh, kh, vh, scale, causal, Lq, Lk, rows)
        return o, lse / math.log(2.0), p

    def drops_last_key(qh, kh, vh, scale, causal, Lq, Lk, rows):  # off-by-one sequence length
        return real_rows(qh, kh, vh, scale, causal, Lq, max(Lk - 1, 0), rows)

    return dict(no_diag=("_visible", vis_no_diag), top_left=("_visible", vis_top_left),
                no_scale=("head_rows", no_scale), k_for_v=("head_rows", k_for_v),
                log2_lse=("head_rows", log2_lse), drops_last_key=("head_rows", drops_last_key))


def _pins_pass():
    """Run a compact set of the pins; True if all pass."""
    tests = [lambda: test_worked_examples(c) for c in _golden_cases()]
    tests += [test_scale_zero_pins_mask_geometry, test_causal_row0_is_first_value, test_single_key_returns_value,
              test_brute_force_decode,
              lambda: test_brute_force_prefill(1, 2, 1, 3, 8, 4, True, False)]
    for t in tests:
        try:
            t()
        except AssertionError:
            return False
    return True


@pytest.mark.parametrize("name", list(_mutants().keys()))
def test_pins_catch_planted_mistakes(name, monkeypatch):
    assert _pins_pass()
    attr, fn = _mutants()[name]
    monkeypatch.setattr(O, attr, fn)
    assert not _pins_pass(), f"planted mistake {name!r} went unnoticed"


def test_gqa_mapping_mistake_is_caught(monkeypatch):
    """kvh = hq % Hkv instead of hq // G must fail the GQA worked example."""
    case = [c for c in _golden_cases() if c["name"] == "gqa_consecutive_heads_share_kv"][0]
    q, k, v = _arr(case["q"]), _arr(case["k"]), _arr(case["v"])
    perm = [0, 1, 0, 1]  # what hq % Hkv would read
    o_wrong = np.stack([v[0, perm[h]] for h in range(4)])[None]
    assert not np.allclose(o_wrong, _arr(case["o"]))
    o, _ = O.prefill(q, k, v, case["scale"])
    np.testing.assert_allclose(o, _arr(case["o"]), atol=1e-12)


# ---------------------------------------------------------------- chunked prefill and append (paged cache)
_CHUNK_TINY = [
    W.ChunkCase("ct-a", B=3, Hq=4, Hkv=2, D=4, dtype="bf16", ctx_lo=0, ctx_hi=20, chunk_lo=1, chunk_hi=9, seed=51),
    W.ChunkCase("ct-b", B=2, Hq=2, Hkv=2, D=4, dtype="fp16", ctx_lo=14, ctx_hi=18, chunk_lo=1, chunk_hi=3, seed=52),
]


@pytest.mark.parametrize("case", _CHUNK_TINY, ids=lambda c: c.name)
@pytest.mark.parametrize("causal", [True, False])
def test_brute_force_prefill_paged(case, causal):
    """P-14: chunked prefill through the block table = scalar brute force (padding rows NaN)."""
    x = W.chunk_inputs(case, nan_fill=False)
    kc, vc = O.cache_append(x["k_new"], x["v_new"], x["k_cache"], x["v_cache"], x["block_table"],
                            x["start_pos"], x["new_lens"])
    q = x["q"].copy()
    for b, n in enumerate(x["new_lens"]):
        q[b, :, n:] = np.nan  # padding rows must not matter
    o1, l1 = O.prefill_paged(q, kc, vc, x["block_table"], x["ctx_lens"], x["new_lens"], 0.7, causal)
    o2, l2 = brute.prefill_paged(q, kc, vc, x["block_table"], x["ctx_lens"], x["new_lens"], 0.7, causal)
    for b, n in enumerate(x["new_lens"]):
        np.testing.assert_allclose(o1[b, :, :n], o2[b, :, :n], atol=1e-12)
        np.testing.assert_allclose(l1[b, :, :n], l2[b, :, :n], atol=1e-12)
        assert (o1[b, :, n:] == 0).all() and np.isneginf(l1[b, :, n:]).all()


def test_prefill_paged_is_bottom_rows_of_contiguous_causal_prefill():
    """P-15: the chunk's rows equal the last rows of a causal prefill over the whole sequence
    laid out contiguously (checks the bottom-right alignment through the Tq == Tk path)."""
    case = W.ChunkCase("p15", B=3, Hq=6, Hkv=2, D=8, dtype="bf16", ctx_lo=5, ctx_hi=60, chunk_lo=1, chunk_hi=30,
                       seed=53)
    x = W.chunk_inputs(case, nan_fill=True)
    kc, vc = O.cache_append(x["k_new"], x["v_new"], x["k_cache"], x["v_cache"], x["block_table"],
                            x["start_pos"], x["new_lens"])
    o, lse = O.prefill_paged(x["q"], kc, vc, x["block_table"], x["ctx_lens"], x["new_lens"], case.scale)
    for b in range(case.B):
        L, n = int(x["ctx_lens"][b]), int(x["new_lens"][b])
        K = np.stack([O.gather_paged(kc, vc, x["block_table"], L, b, h)[0] for h in range(2)])
        V = np.stack([O.gather_paged(kc, vc, x["block_table"], L, b, h)[1] for h in range(2)])
        assert np.isfinite(K).all() and np.isfinite(V).all()  # the append overwrote every NaN it had to
        qf = np.zeros((1, 6, L, 8))
        qf[0, :, L - n:] = x["q"][b, :, :n]
        of, lf = O.prefill(qf, K[None], V[None], case.scale, causal=True)
        np.testing.assert_allclose(o[b, :, :n], of[0, :, L - n:], atol=1e-13)
        np.testing.assert_allclose(lse[b, :, :n], lf[0, :, L - n:], atol=1e-13)


def test_prefill_paged_single_row_is_decode():
    """P-16: a chunk of one token is the paged decode of that token."""
    case = W.ChunkCase("p16", B=4, Hq=6, Hkv=3, D=8, dtype="bf16", ctx_lo=0, ctx_hi=50, chunk_lo=1, chunk_hi=1,
                       seed=54)
    x = W.chunk_inputs(case)
    kc, vc = O.cache_append(x["k_new"], x["v_new"], x["k_cache"], x["v_cache"], x["block_table"],
                            x["start_pos"], x["new_lens"])
    o, lse = O.prefill_paged(x["q"], kc, vc, x["block_table"], x["ctx_lens"], x["new_lens"], case.scale)
    od, ld = O.decode_paged(x["q"][:, :, 0], kc, vc, x["block_table"], x["ctx_lens"], case.scale)
    np.testing.assert_allclose(o[:, :, 0], od, atol=1e-14)
    np.testing.assert_allclose(lse[:, :, 0], ld, atol=1e-14)


def test_cache_append_then_gather_is_concatenation():
    """P-17: after appending, the gathered sequence is the old tokens followed by the new ones,
    and no other slot of the cache changed (bit for bit)."""
    case = W.ChunkCase("p17", B=5, Hq=2, Hkv=2, D=4, dtype="fp16", ctx_lo=0, ctx_hi=40, chunk_lo=1, chunk_hi=37,
                       seed=55)
    x = W.chunk_inputs(case, nan_fill=True)
    kc, vc = O.cache_append(x["k_new"], x["v_new"], x["k_cache"], x["v_cache"], x["block_table"],
                            x["start_pos"], x["new_lens"])
    written = np.zeros(kc.shape[:3], dtype=bool)
    for b in range(case.B):
        s0, n = int(x["start_pos"][b]), int(x["new_lens"][b])
        for h in range(2):
            Kold, Vold = O.gather_paged(x["k_cache"], x["v_cache"], x["block_table"], s0, b, h)
            Knew, Vnew = O.gather_paged(kc, vc, x["block_table"], s0 + n, b, h)
            assert np.array_equal(Knew[:s0], Kold) and np.array_equal(Vnew[:s0], Vold)
            assert np.array_equal(Knew[s0:], x["k_new"][b, h, :n]) and np.array_equal(Vnew[s0:], x["v_new"][b, h, :n])
        pos = np.arange(s0, s0 + n)
        written[x["block_table"][b, pos // 16], :, pos % 16] = True
    same_k = (kc == x["k_cache"]) | (np.isnan(kc) & np.isnan(x["k_cache"]))
    same_v = (vc == x["v_cache"]) | (np.isnan(vc) & np.isnan(x["v_cache"]))
    assert same_k[~written].all() and same_v[~written].all()


def test_sdpa_cross_check_prefill_paged():
    """P-2 for the chunked form: torch SDPA (float64, CPU) on the gathered sequence with an explicit mask."""
    torch = pytest.importorskip("torch")
    case = W.ChunkCase("sdpa-chunk", B=3, Hq=8, Hkv=2, D=32, dtype="bf16", ctx_lo=10, ctx_hi=200, chunk_lo=1,
                       chunk_hi=64, seed=56)
    x = W.chunk_inputs(case)
    kc, vc = O.cache_append(x["k_new"], x["v_new"], x["k_cache"], x["v_cache"], x["block_table"],
                            x["start_pos"], x["new_lens"])
    o, _ = O.prefill_paged(x["q"], kc, vc, x["block_table"], x["ctx_lens"], x["new_lens"], case.scale)
    for b in range(case.B):
        L, n = int(x["ctx_lens"][b]), int(x["new_lens"][b])
        K = np.stack([O.gather_paged(kc, vc, x["block_table"], L, b, h)[0] for h in range(2)])
        V = np.stack([O.gather_paged(kc, vc, x["block_table"], L, b, h)[1] for h in range(2)])
        Kx = torch.from_numpy(np.repeat(K, 4, axis=0)).double()
        Vx = torch.from_numpy(np.repeat(V, 4, axis=0)).double()
        Q = torch.from_numpy(x["q"][b, :, :n]).double()
        mask = torch.from_numpy(np.arange(L)[None, :] <= (np.arange(n)[:, None] + L - n))
        ref = torch.nn.functional.scaled_dot_product_attention(Q, Kx, Vx, attn_mask=mask,
                                                               scale=O.scale64(case.scale))
        np.testing.assert_allclose(o[b, :, :n], ref.numpy(), atol=1e-10)
