"""Pins of the rotary-embedding oracle (oracle/rope.py) against what the mathematics fixes.

* round16 against numpy's correctly rounded float16 conversion and against a
  brute-force nearest-bf16 search with ties to even;
* the rotation against an independent complex-number form (x[i] + i x[i+D/2]
  times e^{i p theta}), norm preservation per pair, identity at position 0,
  and the relative-position property (q at m and k at n give a dot product
  that depends only on m - n);
* planted mistakes (sine sign flipped, interleaved pairing, cosine only)
  each fail one of the pins;
* the fused forms equal the plain definitions applied to pre-rotated inputs.
"""
import numpy as np
import pytest

import workloads as W
from oracle import oracle as O
from oracle import rope as R


def _table64(max_pos, D, base=10000.0):
    i = np.arange(D // 2)
    ang = np.arange(max_pos)[:, None] * base ** (-2.0 * i / D)[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


# ---------------------------------------------------------------- rounding to the 16-bit types
def test_round16_fp16_matches_numpy():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10, rng.standard_normal(2000) * 1e-5,
                        np.array([0.0, -0.0, 1.0, 65504.0, 2.0 ** -24, 3 * 2.0 ** -25])])
    assert np.array_equal(R.round16(x, "fp16"), x.astype(np.float16).astype(np.float64))


def _bf16_brute(x):
    out = np.empty_like(x)
    for k, v in enumerate(x):
        b = np.array([v], dtype=np.float32).view(np.uint32)[0] & 0xFFFF0000
        cands = [np.array([c], dtype=np.uint32).view(np.float32)[0].astype(np.float64)
                 for c in (b - 0x10000, b, b + 0x10000)]
        d = [abs(c - v) for c in cands]
        best = min(d)
        ties = [c for c, dd in zip(cands, d) if dd == best]
        if len(ties) > 1:  # even last mantissa bit
            ties = [c for c in ties if (np.array([c], dtype=np.float32).view(np.uint32)[0] >> 16) % 2 == 0]
        out[k] = ties[0]
    return out


def test_round16_bf16_brute_force():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(3000) * 3
    # exact midpoints between bf16 neighbours, and values just beside them
    base = np.array([1.0, 1.0078125, -2.5, 3.140625], dtype=np.float64)
    mids = base + np.exp2(np.floor(np.log2(np.abs(base))) - 8)  # half a bf16 step above each
    x = np.concatenate([x, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf)])
    assert np.array_equal(R.round16(x, "bf16"), _bf16_brute(x))


# ---------------------------------------------------------------- the rotation
def pin_complex_form(rot):
    rng = np.random.default_rng(3)
    D, P = 16, 40
    tab = _table64(P, D)
    x = rng.standard_normal((P, D))
    pos = np.arange(P)
    z = (x[:, : D // 2] + 1j * x[:, D // 2:]) * np.exp(1j * pos[:, None] * 10000.0 ** (-2.0 * np.arange(D // 2) / D))
    ref = np.concatenate([z.real, z.imag], axis=1)
    assert np.allclose(rot(x, pos, tab), ref, rtol=0, atol=1e-12)


def pin_relative_position(rot):
    rng = np.random.default_rng(4)
    D = 32
    tab = _table64(200, D)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    dots = [rot(q, m, tab) @ rot(k, m - 7, tab) for m in (7, 20, 55, 150)]
    assert np.allclose(dots, dots[0], rtol=1e-12, atol=1e-12)


def pin_norm_and_identity(rot):
    rng = np.random.default_rng(5)
    D = 64
    tab = _table64(100, D)
    x = rng.standard_normal((100, D))
    y = rot(x, np.arange(100), tab)
    n0 = x[:, : D // 2] ** 2 + x[:, D // 2:] ** 2
    n1 = y[:, : D // 2] ** 2 + y[:, D // 2:] ** 2
    assert np.allclose(n0, n1, rtol=1e-12)
    assert np.array_equal(y[0], x[0])


def _all_rot_pins(rot):
    pin_complex_form(rot)
    pin_relative_position(rot)
    pin_norm_and_identity(rot)


def test_rotation_pins():
    _all_rot_pins(R.rotate)


def _rot_sin_flipped(x, pos, tab):
    t = np.array(tab, copy=True)
    t[:, t.shape[1] // 2:] *= -1
    return R.rotate(x, pos, t)


def _rot_interleaved(x, pos, tab):
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    perm = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])
    inv = np.argsort(perm)
    return R.rotate(x[..., perm], pos, tab)[..., inv]


def _rot_cos_only(x, pos, tab):
    t = np.array(tab, copy=True)
    t[:, t.shape[1] // 2:] = 0
    return R.rotate(x, pos, t)


@pytest.mark.parametrize("rot", [_rot_sin_flipped, _rot_interleaved, _rot_cos_only])
def test_rotation_pins_catch_planted_mistakes(rot):
    with pytest.raises(AssertionError):
        _all_rot_pins(rot)


def test_workload_table_is_cos_sin_of_llama3_frequencies():
    tab = W.rope_table(64, 16)
    ref = _table64(64, 16, base=500000.0).astype(np.float32)
    assert np.array_equal(tab, ref)


# ---------------------------------------------------------------- fused forms = definitions on rotated inputs
def test_decode_rope_is_decode_of_rotated_query():
    case = W.DecodeCase("rope", B=3, Hq=4, Hkv=2, D=16, dtype="bf16", ctx_lo=1, ctx_hi=60, seed=6)
    x = W.decode_inputs(case)
    tab = W.rope_table(64, 16)
    o1, l1 = R.decode_paged_rope(x["q"], x["k_cache"], x["v_cache"], x["block_table"], x["ctx_lens"], tab,
                                 case.scale, "bf16")
    pos = x["ctx_lens"] - 1
    qr = np.stack([R.rotate(x["q"][b], np.full(case.Hq, pos[b]), tab) for b in range(case.B)])
    o2, l2 = O.decode_paged(R.round16(qr, "bf16"), x["k_cache"], x["v_cache"], x["block_table"], x["ctx_lens"],
                            case.scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_single_row_chunk_rope_is_decode_rope():
    case = W.ChunkCase("rope1", B=4, Hq=6, Hkv=3, D=16, dtype="bf16", ctx_lo=0, ctx_hi=50, chunk_lo=1, chunk_hi=1,
                       seed=7)
    x = W.chunk_inputs(case)
    tab = W.rope_table(64, 16)
    kc, vc = R.cache_append_rope(x["k_new"], x["v_new"], x["k_cache"], x["v_cache"], x["block_table"],
                                 x["start_pos"], tab, "bf16")
    o1, l1 = R.prefill_paged_rope(x["q"], kc, vc, x["block_table"], x["ctx_lens"], None, tab, case.scale, "bf16")
    o2, l2 = R.decode_paged_rope(x["q"][:, :, 0], kc, vc, x["block_table"], x["ctx_lens"], tab, case.scale, "bf16")
    np.testing.assert_allclose(o1[:, :, 0], o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1[:, :, 0], l2, rtol=0, atol=1e-12)


def test_append_rope_rotates_keys_at_their_positions():
    case = W.ChunkCase("rope-app", B=2, Hq=2, Hkv=2, D=8, dtype="bf16", ctx_lo=3, ctx_hi=30, chunk_lo=1,
                       chunk_hi=9, seed=8)
    x = W.chunk_inputs(case)
    tab = W.rope_table(64, 8)
    kc, vc = R.cache_append_rope(x["k_new"], x["v_new"], x["k_cache"], x["v_cache"], x["block_table"],
                                 x["start_pos"], tab, "bf16", x["new_lens"])
    for b in range(case.B):
        for i in range(int(x["new_lens"][b])):
            p = int(x["start_pos"][b]) + i
            blk, slot = x["block_table"][b, p // 16], p % 16
            for h in range(case.Hkv):
                want = R.round16(R.rotate(x["k_new"][b, h, i], p, tab), "bf16")
                assert np.array_equal(kc[blk, h, slot], want)
                assert np.array_equal(vc[blk, h, slot], x["v_new"][b, h, i])
