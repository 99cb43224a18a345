"""Pins of the linear-layer oracle (oracle/gemm.py) against what the mathematics fixes.

* y = x w^T against a pure-Python triple loop on small integer matrices (exact);
* closed forms: a one-hot activation row selects a column of the weight, one-hot
  weight rows permute the activation columns, ones times w[n, k] = n + 2k sums
  to K n + K (K - 1);
* planted mistakes (the weight used untransposed, the last k term dropped, k
  read one place off) each fail one of the pins;
* ulp16 against numpy's float16 spacing and the bf16 bit step; error_bound
  holds a float32 accumulation in a bad order, and a 16-bit accumulation breaks it.
"""
import numpy as np
import pytest

import workloads as W
from oracle import gemm as G
from oracle import rope as R


def _brute(x, w):
    M, K = len(x), len(x[0])
    N = len(w)
    return [[sum(x[m][k] * w[n][k] for k in range(K)) for n in range(N)] for m in range(M)]


def _pin_brute(f):
    rng = np.random.default_rng(3)
    x = rng.integers(-9, 10, (3, 7))
    w = rng.integers(-9, 10, (5, 7))
    return np.array_equal(f(x, w), np.array(_brute(x.tolist(), w.tolist()), dtype=np.float64))


def _pin_square_brute(f):
    rng = np.random.default_rng(4)
    x = rng.integers(-9, 10, (6, 6))
    w = rng.integers(-9, 10, (6, 6))
    return np.array_equal(f(x, w), np.array(_brute(x.tolist(), w.tolist()), dtype=np.float64))


def _pin_one_hot_row(f):
    rng = np.random.default_rng(5)
    w = rng.integers(-50, 50, (8, 8)).astype(np.float64)
    ok = True
    for i in range(8):
        x = np.zeros((1, 8))
        x[0, i] = 1.0
        ok &= np.array_equal(f(x, w)[0], w[:, i])
    return ok


def _pin_permutation(f):
    rng = np.random.default_rng(6)
    perm = rng.permutation(9)
    w = np.eye(9)[perm]  # row n is e_{perm[n]}
    x = rng.integers(-50, 50, (4, 9)).astype(np.float64)
    return np.array_equal(f(x, w), x[:, perm])


def _pin_closed_form(f):
    K, N = 37, 11
    n = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    w = (n + 2 * k).astype(np.float64)
    y = f(np.ones((1, K)), w)
    return np.array_equal(y[0], K * np.arange(N) + K * (K - 1.0))


PINS = [_pin_brute, _pin_square_brute, _pin_one_hot_row, _pin_permutation, _pin_closed_form]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_meets_pin(pin):
    assert pin(G.linear)


def _untransposed(x, w):
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return x @ w  # only defined for square w


def _drop_last_term(x, w):
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return x[:, :-1] @ w[:, :-1].T


def _shifted_k(x, w):
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return x @ np.roll(w, 1, axis=1).T


@pytest.mark.parametrize("mistake", [_untransposed, _drop_last_term, _shifted_k], ids=lambda f: f.__name__)
def test_planted_mistake_fails_a_pin(mistake):
    def safe(pin):
        try:
            return pin(mistake)
        except ValueError:
            return False
    assert not all(safe(p) for p in PINS)


def test_shape_mismatch_rejected():
    with pytest.raises(ValueError):
        G.linear(np.ones((2, 3)), np.ones((3, 2)))


# ---------------------------------------------------------------- units in the last place
def test_ulp16_fp16_matches_numpy_spacing():
    rng = np.random.default_rng(7)
    y = np.concatenate([rng.standard_normal(5000) * 100, rng.standard_normal(500) * 1e-6, [1.0, 2.0, 32768.0]])
    h = y.astype(np.float16)
    # numpy's spacing steps toward +inf; at |h| that is the step of |h|'s binade (zero included)
    assert np.array_equal(G.ulp16(h.astype(np.float64), "fp16"), np.spacing(np.abs(h)).astype(np.float64))


def test_ulp16_bf16_is_the_bit_step():
    rng = np.random.default_rng(8)
    y = W.round_to(rng.standard_normal(4000).astype(np.float32) * 50, "bf16")
    mag = y.view(np.uint32) & np.uint32(0x7FFF0000)
    up = (mag + np.uint32(0x10000)).view(np.float32).astype(np.float64)
    step = up - mag.view(np.float32).astype(np.float64)
    assert np.array_equal(G.ulp16(y, "bf16"), step)


# ---------------------------------------------------------------- the error bound
def _f32_accumulate(x, w, order):
    """float32 products, float32 running sum over k in the given order."""
    x32 = x.astype(np.float32)
    w32 = w.astype(np.float32)
    M, N = x.shape[0], w.shape[0]
    acc = np.zeros((M, N), dtype=np.float32)
    for k in order:
        acc = (acc + np.outer(x32[:, k], w32[:, k]).astype(np.float32)).astype(np.float32)
    return acc


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_error_bound_holds_for_float32_accumulation(dtype):
    M, N, K = 2, 64, 4096
    x = W.gemm_inputs(M, N, K, dtype, seed=9)
    y = G.linear(x["x"], x["w"])
    # a bad order: largest products first, so the small ones are lost against a large running sum
    order = np.argsort(-np.abs(x["x"][0]) * np.abs(x["w"]).max(axis=0))
    acc = _f32_accumulate(x["x"], x["w"], order).astype(np.float64)
    got = R.round16(acc, dtype)
    bound = G.error_bound(x["x"], x["w"], dtype)
    assert (np.abs(got - y) <= bound).all()


def test_error_bound_rejects_16bit_accumulation():
    M, N, K = 1, 64, 4096
    x = W.gemm_inputs(M, N, K, "fp16", seed=10)
    y = G.linear(x["x"], x["w"])
    acc = np.zeros((M, N))
    for k in range(K):  # running sum rounded to fp16 after every term
        acc = R.round16(acc + np.outer(x["x"][:, k], x["w"][:, k]), "fp16")
    assert (np.abs(acc - y) > G.error_bound(x["x"], x["w"], "fp16")).any()
