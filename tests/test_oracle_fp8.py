"""Pins of the E4M3 (FP8) oracle against what the format and the mathematics fix.

The codec is pinned by values the OCP 8-bit floating point specification
states for E4M3 (bias 7, subnormals m * 2^-9, largest finite 448, NaN at
S.1111.111, no infinities), by monotonicity and symmetry of the code order,
by a brute-force nearest-value search (ties to the even code) and by the
saturation rule. Planted mistakes in copies of the codec (wrong bias, ties
away from zero, no saturation, wrong subnormal step, swapped scales) must
each fail one of the pins. The attention over an FP8 cache is pinned by exact
identities of the definition under power-of-two scales.
"""
import math

import numpy as np
import pytest

import workloads as W
from oracle import fp8 as F8
from oracle import oracle as O

FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
ALL_VALUES = np.unique(F8.e4m3_to_float(FINITE))  # the 253 distinct finite values (+0 and -0 coincide)


# ---------------------------------------------------------------- pins, parameterised by the codec under test
def pin_spec_values(dec):
    spec = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
            0x30: 0.5, 0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0x48: 4.0, 0x77: 240.0, 0x78: 256.0, 0x7E: 448.0,
            0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in spec.items():
        assert float(dec(np.array([c], dtype=np.uint8))[0]) == v, hex(c)
    assert math.isnan(dec(np.array([0x7F], dtype=np.uint8))[0]) and math.isnan(dec(np.array([0xFF], dtype=np.uint8))[0])
    assert np.isfinite(dec(FINITE)).all()


def pin_order(dec):
    pos = dec(np.arange(0, 127, dtype=np.uint8))
    assert (np.diff(pos) > 0).all()
    assert np.array_equal(dec(np.arange(128, 255, dtype=np.uint8)), -pos)


def pin_roundtrip(enc, dec):
    assert np.array_equal(enc(dec(FINITE).astype(np.float32)), FINITE)


def pin_nearest(enc, dec):
    rng = np.random.default_rng(7)
    vals = np.unique(dec(FINITE))
    mids = 0.5 * (vals[1:] + vals[:-1])
    x = np.concatenate([rng.standard_normal(3000) * 40, rng.standard_normal(1000) * 0.01, mids,
                        np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf)]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    codes = enc(x)
    got = dec(codes)
    xd = x.astype(np.float64)
    d = np.abs(vals[None, :] - xd[:, None])
    best = d.min(axis=1)
    assert np.array_equal(np.abs(got - xd), best), "not the nearest value"
    tie = (d == best[:, None]).sum(axis=1) > 1
    assert np.all(codes[tie & (got != 0)] % 2 == 0), "ties must go to the even code"


def pin_saturation(enc):
    x = np.array([448.0, 449.0, 464.0, 465.0, 1e6, 3e38, -449.0, -1e6, np.inf, -np.inf], dtype=np.float32)
    assert enc(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7E, 0xFE]


def _all_pins(enc, dec):
    pin_spec_values(dec)
    pin_order(dec)
    pin_roundtrip(enc, dec)
    pin_nearest(enc, dec)
    pin_saturation(enc)


def test_codec_pins():
    _all_pins(F8.float_to_e4m3, F8.e4m3_to_float)


# ---------------------------------------------------------------- planted mistakes
def _dec_bias8(codes):
    c = np.asarray(codes).astype(np.int64)
    v = F8.e4m3_to_float(codes)
    return np.where((c >> 3) & 0xF, v / 2.0, v)


def _dec_sub_step(codes):
    c = np.asarray(codes).astype(np.int64)
    v = F8.e4m3_to_float(codes)
    return np.where(((c >> 3) & 0xF) == 0, v * 2.0, v)


def _enc_ties_away(x):
    x = np.asarray(x, dtype=np.float32)
    c = F8.float_to_e4m3(x)
    # round half away from zero: move ties up one code
    vals = F8.e4m3_to_float(c)
    up = F8.float_to_e4m3(np.nextafter(x, np.where(x >= 0, np.inf, -np.inf)).astype(np.float32))
    tie = np.abs(np.abs(x.astype(np.float64)) - np.abs(vals)) == np.abs(np.abs(F8.e4m3_to_float(up)) - np.abs(x))
    return np.where(tie & (up != c), up, c).astype(np.uint8)


def _enc_no_saturation(x):
    x = np.asarray(x, dtype=np.float32)
    c = F8.float_to_e4m3(x)
    return np.where(np.abs(x) > 464, c | 0x7F, c).astype(np.uint8)


def _enc_truncate(x):
    x = np.asarray(x, dtype=np.float32)
    c = F8.float_to_e4m3(x)
    over = np.abs(F8.e4m3_to_float(c)) > np.abs(x.astype(np.float64))
    return np.where(over & (c & 0x7F != 0), c - 1, c).astype(np.uint8)


@pytest.mark.parametrize("enc,dec,name", [
    (F8.float_to_e4m3, _dec_bias8, "bias 8"),
    (F8.float_to_e4m3, _dec_sub_step, "subnormal step 2^-8"),
    (_enc_ties_away, F8.e4m3_to_float, "ties away from zero"),
    (_enc_no_saturation, F8.e4m3_to_float, "overflow to NaN"),
    (_enc_truncate, F8.e4m3_to_float, "truncation"),
])
def test_codec_pins_catch_planted_mistakes(enc, dec, name):
    with pytest.raises(AssertionError):
        _all_pins(enc, dec)


# ---------------------------------------------------------------- quantisation with a scale
def test_quantize_saturates_quotients_that_overflow():
    # x / scale beyond float32's range is infinite before the conversion: it saturates like any magnitude
    # above 448
    x = np.array([3e38, -3e38, 65504.0, 1.0], dtype=np.float32)
    assert F8.quantize(x, 1e-35).tolist() == [0x7E, 0xFE, 0x7E, 0x7E]


def test_quantize_error_within_half_step():
    rng = np.random.default_rng(3)
    for s in (1.0, 0.25, 0.0078125, 3.0, 0.1):
        x = (rng.standard_normal(5000) * 50 * s).astype(np.float32)
        x = x[np.abs(x) / s <= 448]
        back = F8.dequantize(F8.quantize(x, s), s)
        # half the spacing of the format at |x| / s (2^-3 relative for normals, 2^-10 absolute below 2^-6)
        a = np.abs(x.astype(np.float64)) / float(np.float32(s))
        k = np.floor(np.log2(np.maximum(a, 2.0 ** -30)))
        half = 0.5 * np.exp2(np.maximum(k, -6) - 3) * float(np.float32(s))
        assert (np.abs(back - x) <= half * (1 + 1e-12)).all()


def test_quantize_power_of_two_scale_is_exact_shift():
    """With s = 2^k, x / s is exact, so the codes are those of the scaled values."""
    x = np.array([0.3, -1.7, 100.0, 3e-4], dtype=np.float32)
    assert np.array_equal(F8.quantize(x, 0.5), F8.float_to_e4m3(x * 2))


# ---------------------------------------------------------------- attention over an FP8 cache
def _fp8_case(seed=71, B=3, Hq=6, Hkv=2, D=16):
    case = W.DecodeCase("fp8", B=B, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16", ctx_lo=1, ctx_hi=70, seed=seed)
    x = W.decode_inputs(case)
    rng = np.random.default_rng(seed)
    x["k8"] = rng.integers(0, 256, x["k_cache"].shape).astype(np.uint8)
    x["v8"] = rng.integers(0, 256, x["v_cache"].shape).astype(np.uint8)
    # NaN codes only where the cache is unused (the oracle must never read them)
    for a in (x["k8"], x["v8"]):
        a[(a & 0x7F) == 0x7F] = 0x3C
    return case, x


def test_decode_fp8_scale_identities():
    """O(ks, vs, scale) = vs * O(1, 1, scale * ks) and lse(ks, vs, scale) = lse(1, 1, scale * ks)."""
    case, x = _fp8_case()
    args = (x["block_table"], x["ctx_lens"])
    o1, l1 = F8.decode_paged_fp8(x["q"], x["k8"], x["v8"], 0.25, 8.0, *args, scale=0.5)
    o2, l2 = F8.decode_paged_fp8(x["q"], x["k8"], x["v8"], 1.0, 1.0, *args, scale=0.125)
    np.testing.assert_allclose(o1, 8.0 * o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-12)


def test_decode_fp8_swapped_scales_are_caught():
    """A planted mistake (k_scale applied to V and v_scale to K) breaks the identity above."""
    case, x = _fp8_case()
    args = (x["block_table"], x["ctx_lens"])
    o1, _ = F8.decode_paged_fp8(x["q"], x["k8"], x["v8"], 8.0, 0.25, *args, scale=0.5)  # swapped
    o2, _ = F8.decode_paged_fp8(x["q"], x["k8"], x["v8"], 1.0, 1.0, *args, scale=0.125)
    assert not np.allclose(o1, 8.0 * o2, rtol=1e-6)


def test_decode_fp8_single_token_returns_its_value():
    """ctx = 1: O is the one value row, dequantized; lse = scale * q . k."""
    case, x = _fp8_case(B=2)
    ctx = np.array([1, 1], dtype=np.int32)
    o, lse = F8.decode_paged_fp8(x["q"], x["k8"], x["v8"], 0.5, 2.0, x["block_table"], ctx, 0.25)
    for b in range(2):
        blk = x["block_table"][b, 0]
        for hq in range(case.Hq):
            kvh = hq // (case.Hq // case.Hkv)
            v = F8.e4m3_to_float(x["v8"][blk, kvh, 0]) * 2.0
            k = F8.e4m3_to_float(x["k8"][blk, kvh, 0]) * 0.5
            assert np.array_equal(o[b, hq], v)
            assert abs(lse[b, hq] - 0.25 * float(x["q"][b, hq].astype(np.float64) @ k)) < 1e-12


def test_append_fp8_writes_codes_and_nothing_else():
    case = W.ChunkCase("fp8-append", B=3, Hq=4, Hkv=2, D=8, dtype="bf16", ctx_lo=0, ctx_hi=40, chunk_lo=0,
                       chunk_hi=21, seed=72)
    x = W.chunk_inputs(case)
    rng = np.random.default_rng(72)
    k8 = rng.integers(0, 126, x["k_cache"].shape).astype(np.uint8)
    v8 = rng.integers(0, 126, x["v_cache"].shape).astype(np.uint8)
    kc, vc = F8.cache_append_fp8(x["k_new"], x["v_new"], k8, v8, x["block_table"], x["start_pos"], 0.5, 0.125,
                                 x["new_lens"])
    touched = np.zeros(k8.shape, dtype=bool)
    for b in range(case.B):
        for i in range(int(x["new_lens"][b])):
            pos = int(x["start_pos"][b]) + i
            blk, slot = x["block_table"][b, pos // 16], pos % 16
            touched[blk, :, slot] = True
            for h in range(case.Hkv):
                assert np.array_equal(kc[blk, h, slot], F8.float_to_e4m3(x["k_new"][b, h, i] * 2))
                assert np.array_equal(vc[blk, h, slot], F8.float_to_e4m3(x["v_new"][b, h, i] * 8))
    assert np.array_equal(kc[~touched], k8[~touched]) and np.array_equal(vc[~touched], v8[~touched])


def test_prefill_fp8_scale_identity():
    """O(qs, ks, vs, scale) = vs * O(1, 1, 1, scale * qs * ks); lse likewise (scale-only dependence). The
    error budget of the FP8 arithmetic is pinned in test_oracle_bounds.py."""
    case = W.PrefillCase("fp8p", B=2, Hq=4, Hkv=2, T=40, D=16, dtype="bf16", causal=True, ragged=True, seed=73)
    x = W.prefill_inputs_fp8(case)
    o1, l1 = F8.prefill_fp8(x["q"], x["k"], x["v"], 0.5, 0.25, 4.0, 0.5, True, x["seq_lens"])
    o2, l2 = F8.prefill_fp8(x["q"], x["k"], x["v"], 1.0, 1.0, 1.0, 0.0625, True, x["seq_lens"])
    np.testing.assert_allclose(o1, 4.0 * o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-12)
