"""Pins of the error budgets (oracle/bounds.py) against the arithmetic they claim to cover.

A float32 model of each form's arithmetic, written here from the library's stated numerics (not from
the budget formula), is run on random and on adversarial inputs:
  * 16-bit form: fp32 scores (products summed one at a time), p = 2^(x - m) in fp32 with a running max
    that lags (the 16-bit kernels move it only when a tile exceeds it by more than 8, and tolerate p up to
    2^15), P rounded to bf16 / fp16, O = sum r v / sum r in fp32 (each 64-key tile's sums formed one term
    at a time, then added to the running sums), one rounding to the output type;
  * FP8 form: tile max first, the max moving once a tile exceeds it by more than 1 (here also to any point
    up to 1 below the tile max: every lag the stated arithmetic allows), p 2^7 rounded to E4M3 (the oracle's
    codec), O = sum q v / sum p in fp32.
The model must stay inside the budget everywhere (adversarial inputs put P at rounding midpoints with the
values aligned to the rounding direction, so the budget is approached, not just met), and planted
deviations must exceed it on at least one input: a coarser rounding of P (6 significant bits for bf16, two
mantissa bits for E4M3), normalising the 16-bit form by the unrounded sum, scaling the FP8 P by 2^8, and a
dropped key tile (also on a 16384-key causal head, the long prefill's shape: through O up to 4096 keys,
through lse at every length).
"""
import numpy as np
import pytest

import workloads as W
from oracle import bounds as BD
from oracle import fp8 as F8
from oracle import gemm as G
from oracle import oracle as O

LOG2E = np.float32(np.log2(np.e))


def _round_bits(x, bits):
    """Round float32 values to `bits` significant bits, nearest even (no exponent limits)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)  # x = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 2.0 ** bits) / 2.0 ** bits, e).astype(np.float32)


def _round16(x, dtype):
    return W.round_to(np.asarray(x, dtype=np.float32), dtype)


def _dot32(q, K):
    """fp32 scores q . k_j with the products summed one dimension at a time (a bad order)."""
    acc = np.zeros(K.shape[0], dtype=np.float32)
    for e in range(K.shape[1]):
        acc = (acc + np.float32(q[e]) * K[:, e].astype(np.float32)).astype(np.float32)
    return acc


def _sum32(x):
    acc = np.float32(0.0)
    for v in np.asarray(x, dtype=np.float32):
        acc = np.float32(acc + v)
    return acc


def sim16(q, K, V, scale, dtype, tile=64, p_round=None, norm="rounded", out_round=None, drop=None, lazy=8.0):
    """One query row through the 16-bit kernels' arithmetic, in float32. Returns O (float32, output dtype)."""
    p_round = p_round or (lambda p: _round16(p, dtype))
    c = np.float32(abs(np.float32(scale)) * LOG2E)
    qs = np.asarray(q, dtype=np.float32) * (np.float32(-1.0) if scale < 0 else np.float32(1.0))
    s = _dot32(qs, K) if scale != 0 else np.zeros(K.shape[0], dtype=np.float32)
    m = np.float32(-np.inf)
    l = np.float32(0.0)
    lr = np.float32(0.0)
    acc = np.zeros(V.shape[1], dtype=np.float32)
    for t0 in range(0, K.shape[0], tile):
        if drop is not None and t0 // tile == drop:
            continue
        x = (s[t0:t0 + tile] * c).astype(np.float32)
        p = np.exp2((x - m).astype(np.float32)).astype(np.float32) if np.isfinite(m) else None
        if p is None or not (_sum32(p) <= 32768.0):
            mt = np.float32(x.max())
            if mt > m + lazy:
                alpha = np.float32(0.0) if not np.isfinite(m) else np.float32(np.exp2(np.float32(m - mt)))
                m = mt
                l, lr = np.float32(l * alpha), np.float32(lr * alpha)
                acc = (acc * alpha).astype(np.float32)
            p = np.exp2((x - m).astype(np.float32)).astype(np.float32)
        r = p_round(p)
        l = np.float32(l + _sum32(p))
        lr = np.float32(lr + _sum32(r))
        part = np.zeros(V.shape[1], dtype=np.float32)  # the tile's P.V, then added to the accumulator
        for j in range(len(r)):
            part = (part + r[j] * V[t0 + j].astype(np.float32)).astype(np.float32)
        acc = (acc + part).astype(np.float32)
    den = lr if norm == "rounded" else l
    o = (acc * np.float32(np.float32(1.0) / den)).astype(np.float32)
    return (out_round or (lambda y: _round16(y, dtype)))(o)


def sim_fp8(q, K, V, scale, dtype, tile=64, rng=None, code=None, pscale=7, drop=None, dot_err=BD.F8_DOT, seed=0):
    """One query row through the FP8 prefill's arithmetic in float32 (inputs already dequantized). The fp8
    matrix instruction's dot products (scores, each tile's P.V) carry an error of up to dot_err times the
    sum of the magnitudes of their products, drawn at random here."""
    code = code or (lambda y: F8.e4m3_to_float(F8.float_to_e4m3(y)).astype(np.float32))
    noise = np.random.default_rng(seed)
    c = np.float32(abs(np.float32(scale)) * LOG2E)
    qf = np.asarray(q, dtype=np.float32)
    s = (_dot32(qf, K) + noise.uniform(-1, 1, K.shape[0]) * dot_err * (np.abs(K) @ np.abs(qf))).astype(np.float32)
    m = np.float32(-np.inf)
    l = np.float32(0.0)
    acc = np.zeros(V.shape[1], dtype=np.float32)
    for t0 in range(0, K.shape[0], tile):
        if drop is not None and t0 // tile == drop:
            continue
        x = (s[t0:t0 + tile] * c).astype(np.float32)
        mt = np.float32(x.max())
        if mt > m + 1.0:
            lag = np.float32(rng.random()) if rng is not None else np.float32(0.0)  # any lag in [0, 1)
            m_new = np.float32(mt - lag)
            alpha = np.float32(0.0) if not np.isfinite(m) else np.float32(np.exp2(np.float32(m - m_new)))
            m = m_new
            l = np.float32(l * alpha)
            acc = (acc * alpha).astype(np.float32)
        p = np.exp2((x - m + np.float32(pscale)).astype(np.float32)).astype(np.float32)
        qp = code(p)
        l = np.float32(l + _sum32(p))
        part = np.zeros(V.shape[1], dtype=np.float32)
        for j in range(len(qp)):
            part = (part + np.float32(qp[j]) * V[t0 + j].astype(np.float32)).astype(np.float32)
        part += (noise.uniform(-1, 1, V.shape[1]) * dot_err * (qp @ np.abs(V[t0:t0 + len(qp)]))).astype(np.float32)
        acc = (acc + part).astype(np.float32)
    return _round16((acc * np.float32(np.float32(1.0) / l)).astype(np.float32), dtype)


def _rows_exact(q, K, V, scale, causal, Lq):
    """Exact outputs and budgets for every row of one head (Tq = Lq, Tk = K rows)."""
    Lk = K.shape[0]
    rows = np.arange(q.shape[0])
    o, _, _ = O.head_rows(q, K, V, scale, causal, Lq, Lk, rows)
    return o


def _visible(i, Lq, Lk, causal):
    return Lk if not causal else min(Lk, i + (Lk - Lq) + 1)


def _check16(q, K, V, scale, causal, dtype, sim_kw=None, expect_ok=True, what=""):
    Lq, Lk = q.shape[0], K.shape[0]
    o = _rows_exact(q, K, V, scale, causal, Lq)
    bud = BD.prefill(q[None, None], K[None, None], V[None, None], scale, causal, None, dtype)[0, 0]
    worst = 0.0
    for i in range(Lq):
        n = _visible(i, Lq, Lk, causal)
        if n <= 0:
            continue
        og = sim16(q[i], K[:n], V[:n], scale, dtype, **(sim_kw or {}))
        worst = max(worst, float((np.abs(og - o[i]) / bud[i]).max()))
    print(f"{what}: max err/budget = {worst:.3f}")
    if expect_ok:
        assert worst <= 1.0, f"{what}: the model exceeds the budget ({worst:.3f})"
    return worst


# ---------------------------------------------------------------- 16-bit form
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal,T,D,qmul,seed", [(True, 300, 64, 1.0, 1), (False, 200, 128, 1.0, 2),
                                                  (True, 260, 32, 8.0, 3), (False, 150, 16, 3.0, 4)])
def test_budget16_holds_for_the_model_on_random_inputs(dtype, causal, T, D, qmul, seed):
    rng = np.random.default_rng(seed)
    q = _round16(rng.standard_normal((T, D)) * qmul, dtype)
    K = _round16(rng.standard_normal((T, D)), dtype)
    V = _round16(rng.standard_normal((T, D)) * 3.0 + 2.0, dtype)
    _check16(q.astype(np.float64), K.astype(np.float64), V.astype(np.float64), 1.0 / np.sqrt(D), causal, dtype,
             what=f"random {dtype} causal={causal} qx{qmul}")


def _midpoint_case(dtype, bits, n_adv=128, vbig=1.0, offset=0.0):
    """D = 1, q = 1, scale = 1: scores are the keys. 64 keys at score 0 (p = 1 once the max settles on 0),
    then n_adv keys whose p sits just below (values +vbig) or just above (values -vbig) the rounding
    midpoint of [1, 2) for a format with `bits` significant bits, so every rounding error pushes O the
    same way. offset is added to every value."""
    mid = 1.0 + 2.0 ** -bits
    d = 2.0 ** -(bits + 6)
    pA, pB = mid - d, mid + d
    k = np.concatenate([np.zeros(64), np.tile([np.log(pA), np.log(pB)], n_adv // 2)])
    v = np.concatenate([np.zeros(64), np.tile([vbig, -vbig], n_adv // 2)]) + offset
    K = np.asarray(k, dtype=np.float32).astype(np.float64)[:, None]
    V = _round16(v, dtype).astype(np.float64)[:, None]
    q = np.ones((1, 1))
    return q, K, V


@pytest.mark.parametrize("dtype,bits", [("bf16", 8), ("fp16", 11)])
def test_budget16_is_approached_at_rounding_midpoints(dtype, bits):
    q, K, V = _midpoint_case(dtype, bits)
    worst = _check16(q, K, V, 1.0, False, dtype, what=f"midpoints {dtype}")
    assert worst >= 0.3, "the adversarial input should come close to the budget"


def test_budget16_rejects_coarser_rounding_of_p():
    # P rounded to 6 significant bits (two fewer than bf16), at that format's midpoints
    q, K, V = _midpoint_case("bf16", 6)
    _check16(q, K, V, 1.0, False, "bf16", what="bf16 with 8-bit P (correct)")
    worst = _check16(q, K, V, 1.0, False, "bf16", sim_kw=dict(p_round=lambda p: _round_bits(p, 6)),
                     expect_ok=False, what="P rounded to 6 bits")
    assert worst > 1.0


def test_budget16_rejects_normalising_by_the_unrounded_sum():
    # every adversarial p rounds down; all values equal 2 - 2^-6 (so O does too, exactly, when O divides by
    # the sum of the weights it applies)
    dtype = "bf16"
    mid = 1.0 + 2.0 ** -8
    k = np.concatenate([np.zeros(64), np.full(1000, np.log(mid - 2.0 ** -14))])
    K = np.asarray(k, dtype=np.float32).astype(np.float64)[:, None]
    V = np.full((K.shape[0], 1), 2.0 - 2.0 ** -6)
    q = np.ones((1, 1))
    _check16(q, K, V, 1.0, False, dtype, what="normalised by the rounded sum (correct)")
    worst = _check16(q, K, V, 1.0, False, dtype, sim_kw=dict(norm="unrounded"), expect_ok=False,
                     what="normalised by the unrounded sum")
    assert worst > 1.0


def test_budget16_rejects_a_dropped_key_tile():
    rng = np.random.default_rng(11)
    T, D = 200, 64
    q = _round16(rng.standard_normal((T, D)), "bf16").astype(np.float64)
    K = _round16(rng.standard_normal((T, D)), "bf16").astype(np.float64)
    V = _round16(rng.standard_normal((T, D)), "bf16").astype(np.float64)
    worst = _check16(q[-4:], K, V, 0.125, False, "bf16", sim_kw=dict(drop=1), expect_ok=False,
                     what="one 64-key tile dropped")
    assert worst > 1.0


def test_budget16_rejects_a_coarser_output_rounding():
    rng = np.random.default_rng(12)
    T, D = 100, 64
    q = _round16(rng.standard_normal((4, D)), "bf16").astype(np.float64)
    K = _round16(rng.standard_normal((T, D)), "bf16").astype(np.float64)
    V = _round16(rng.standard_normal((T, D)) * 4.0, "bf16").astype(np.float64)
    worst = _check16(q, K, V, 0.125, False, "bf16", sim_kw=dict(out_round=lambda y: _round_bits(y, 5)),
                     expect_ok=False, what="output rounded to 5 bits")
    assert worst > 1.0


def test_budget16_decode_and_paged_forms_match_the_prefill_budget():
    """The decode / chunked budgets are the prefill budget of the same rows (plus the merge's weight term
    for the decode, which only widens it)."""
    case = W.DecodeCase("b", B=3, Hq=4, Hkv=2, D=64, dtype="bf16", ctx_lo=20, ctx_hi=300, seed=13)
    x = W.decode_inputs(case)
    bd = BD.decode_paged(x["q"], x["k_cache"], x["v_cache"], x["block_table"], x["ctx_lens"], case.scale, "bf16")
    for b in range(case.B):
        L = int(x["ctx_lens"][b])
        for kvh in range(2):
            K, V = O.gather_paged(x["k_cache"], x["v_cache"], x["block_table"], L, b, kvh)
            for g in range(2):
                hq = kvh * 2 + g
                bp = BD.prefill(x["q"][b, hq][None, None, None], K[None, None], V[None, None], case.scale, False,
                                None, "bf16")[0, 0, 0]
                assert np.all(bd[b, hq] >= bp) and np.all(bd[b, hq] <= bp * 1.01 + 1e-12)


# ---------------------------------------------------------------- FP8 form
def _check_fp8(q, K, V, scale, causal, dtype, sim_kw=None, expect_ok=True, what="", lags=3):
    Lq, Lk = q.shape[0], K.shape[0]
    o = _rows_exact(q, K, V, scale, causal, Lq)
    bud = BD.prefill_fp8(q[None, None], K[None, None], V[None, None], scale, causal, None, dtype)[0, 0]
    worst = 0.0
    rng = np.random.default_rng(5)
    for i in range(Lq):
        n = _visible(i, Lq, Lk, causal)
        for rep in range(lags):  # the kernel's lag (0) and random lags in [0, 1)
            og = sim_fp8(q[i], K[:n], V[:n], scale, dtype, rng=None if rep == 0 else rng, **(sim_kw or {}))
            worst = max(worst, float((np.abs(og - o[i]) / bud[i]).max()))
    print(f"{what}: max err/budget = {worst:.3f}")
    if expect_ok:
        assert worst <= 1.0, f"{what}: the model exceeds the budget ({worst:.3f})"
    return worst


@pytest.mark.parametrize("causal,T,seed", [(True, 260, 21), (False, 150, 22)])
def test_budget_fp8_holds_for_the_model_on_random_inputs(causal, T, seed):
    rng = np.random.default_rng(seed)
    D = 64
    q = F8.dequantize(W.e4m3_codes(rng, (T, D)), 0.5)
    K = F8.dequantize(W.e4m3_codes(rng, (T, D)), 0.25)
    V = F8.dequantize(W.e4m3_codes(rng, (T, D)), 0.5)
    _check_fp8(q, K, V, 1.0 / np.sqrt(D), causal, "bf16", what=f"fp8 random causal={causal}")


def _fp8_midpoint_case(p_mid, n_adv=1000):
    """64 keys at score 0 (p = 1), then n_adv keys with p just below p_mid (they round down); all values 1."""
    k = np.concatenate([np.zeros(64), np.full(n_adv, np.log(p_mid * (1.0 - 2.0 ** -12)))])
    K = np.asarray(k, dtype=np.float32).astype(np.float64)[:, None]
    V = np.ones((K.shape[0], 1))
    return np.ones((1, 1)), K, V


def test_budget_fp8_is_approached_at_e4m3_midpoints():
    q, K, V = _fp8_midpoint_case(136.0 / 128.0)  # midpoint of 128 and 144, the E4M3 values around 2^7 p
    worst = _check_fp8(q, K, V, 1.0, False, "bf16", what="fp8 midpoints", lags=1)
    assert worst >= 0.5


def test_budget_fp8_rejects_two_mantissa_bits():
    q, K, V = _fp8_midpoint_case(144.0 / 128.0)  # midpoint of 128 and 160 (two mantissa bits)
    _check_fp8(q, K, V, 1.0, False, "bf16", what="fp8 with E4M3 (correct)", lags=1)
    worst = _check_fp8(q, K, V, 1.0, False, "bf16", sim_kw=dict(code=lambda y: _round_bits(y, 3)),
                       expect_ok=False, what="fp8 P with two mantissa bits", lags=1)
    assert worst > 1.0


def test_budget_fp8_rejects_scaling_p_by_2_8():
    # keys 0.99 above the settled max (no move: the lag is below 1), so p = 1.99: 2^8 p = 508 saturates at 448
    k = np.concatenate([np.zeros(64), np.full(200, 0.99 / np.log2(np.e))])
    K = np.asarray(k, dtype=np.float32).astype(np.float64)[:, None]
    V = np.concatenate([np.zeros(64), np.ones(200)])[:, None]
    q = np.ones((1, 1))
    _check_fp8(q, K, V, 1.0, False, "bf16", what="fp8 P scaled by 2^7 (correct)", lags=1)
    worst = _check_fp8(q, K, V, 1.0, False, "bf16", sim_kw=dict(pscale=8), expect_ok=False, what="P scaled by 2^8",
                       lags=1)
    assert worst > 1.0


def _long_head(seed=23, nrows=None):
    """One head of the 16384-token causal prefill with E4M3 codes drawn as the FP8 bench draws them."""
    rng = np.random.default_rng(seed)
    T, D = 16384, 128
    rows = np.array([70, 130, 200, 400, 700, 1000, 2047, 4000, 8191, 12000, 16383])[:nrows]
    q = F8.dequantize(W.e4m3_codes(rng, (len(rows), D)), 0.25)
    K = F8.dequantize(W.e4m3_codes(rng, (T, D)), 0.25)
    V = F8.dequantize(W.e4m3_codes(rng, (T, D)), 0.5)
    return rows, q, K, V, 1.0 / np.sqrt(D)


def test_budget_fp8_worst_case_catches_a_dropped_tile_on_early_rows():
    """The worst-case budget (against the exact definition) exposes one dropped 64-key tile on the rows
    that see up to a few hundred keys; for longer rows the lse check and the model check below do."""
    rows, q, K, V, scale = _long_head(nrows=4)
    for r, i in enumerate(rows):
        L = i + 1
        o, _, _ = O.head_rows(q[r][None], K[:L], V[:L], scale, False, 1, L, np.array([0]))
        bud = BD.prefill_fp8(q[r][None, None, None], K[None, None, :L], V[None, None, :L], scale, False, None,
                             "bf16")[0, 0, 0]
        ok = sim_fp8(q[r], K[:L], V[:L], scale, "bf16")
        assert (np.abs(ok - o[0]) <= bud).all(), f"row {i}: the model exceeds the budget"
        bad = sim_fp8(q[r], K[:L], V[:L], scale, "bf16", drop=0)
        assert (np.abs(bad - o[0]) > bud).any(), f"row {i}: dropped tile not caught"


def test_fp8_model_holds_the_float32_arithmetic_and_a_dropped_tile_is_caught_at_every_length():
    """The float64 model of the FP8 arithmetic (oracle/bounds.fp8_model_row) against the float32
    simulation on one head of the 16384-token causal shape, rows up to the last: the simulation stays
    inside the model's tight budget, and the model inside the worst-case budget of the exact result.
    Dropping one 64-key tile (the first, a middle one, the last full one) leaves the tight O budget on
    every row with up to 4096 keys; on longer rows the change of O is within what the fp8 instruction's
    dot-product accuracy admits, and the lse check (1e-4 relative, taken as 2e-4 to cover the kernel's own
    lse error) catches it on every row."""
    rows, q, K, V, scale = _long_head()
    for r, i in enumerate(rows):
        L = i + 1
        mo, mb, amb = BD.fp8_model_row(q[r], K[:L], V[:L], scale)
        tight = mb + 0.5 * G.ulp16(np.abs(mo) + mb, "bf16")
        sim = sim_fp8(q[r], K[:L], V[:L], scale, "bf16")
        ratio = float((np.abs(sim - mo) / tight).max())
        o, lse, _ = O.head_rows(q[r][None], K[:L], V[:L], scale, False, 1, L, np.array([0]))
        wc = BD.prefill_fp8(q[r][None, None, None], K[None, None, :L], V[None, None, :L], scale, False, None,
                            "bf16")[0, 0, 0]
        drops = sorted({0, L // 128, max(L // 64 - 1, 0)})
        worst_drop = min(float((np.abs(sim_fp8(q[r], K[:L], V[:L], scale, "bf16", drop=t) - mo) / tight).max())
                         for t in drops)
        lse_caught = True
        for t in drops:
            keep = np.ones(L, dtype=bool)
            keep[64 * t:64 * t + 64] = False
            _, l2, _ = O.head_rows(q[r][None], K[:L][keep], V[:L][keep], scale, False, 1, int(keep.sum()),
                                   np.array([0]))
            lse_caught &= bool(abs(l2[0] - lse[0]) > 2e-4 * max(1.0, abs(lse[0])))
        print(f"row {i}: ambiguous={amb} sim/tight={ratio:.3f} model vs exact / worst case="
              f"{float((np.abs(mo - o[0]) / wc).max()):.3f} weakest dropped-tile O ratio={worst_drop:.2f} "
              f"lse catches it={lse_caught}")
        assert ratio <= 1.0
        assert (np.abs(mo - o[0]) <= wc).all()
        if L <= 4096:
            assert worst_drop > 1.0
        assert lse_caught


def test_fp8_model_rejects_two_mantissa_bits_in_the_arithmetic():
    rows, q, K, V, scale = _long_head(nrows=3)
    for r, i in enumerate(rows):
        L = i + 1
        mo, mb, _ = BD.fp8_model_row(q[r], K[:L], V[:L], scale)
        tight = mb + 0.5 * G.ulp16(np.abs(mo) + mb, "bf16")
        bad = sim_fp8(q[r], K[:L], V[:L], scale, "bf16", code=lambda y: _round_bits(y, 3))
        assert (np.abs(bad - mo) > tight).any()
