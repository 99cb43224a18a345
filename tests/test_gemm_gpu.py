"""GPU parity of the split-K linear-layer product (attn_gemm_splitk, through the C ABI).

Reference: y = x w^T in float64 (oracle/gemm.py). Tolerance per element: oracle/gemm.error_bound, one
unit in the last place of the output type at |y| plus gamma_K * sum_k |x_mk w_nk| (float32 products and
sums, u = 2^-24), which any float32 summation order meets. The largest error / bound ratio is printed.
Cases: the Llama3-8B / Granite-8B linear layers at decode batch 1 and 2 (every element), ragged M, N and
K around the tile sizes (16 weight rows, 16 activation rows, k-steps of 32, one launch per 64 rows of
x), every configuration on one ragged shape, K = 0, and determinism.
"""
import numpy as np
import pytest

import workloads as W
from oracle import gemm as G
from test_parity_gpu import _note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta(gpu):
    import torch  # noqa: F401
    import tiled_attention_02_amd as ta
    ta.lib()
    return ta


def _dev(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16 if dtype == "bf16" else torch.float16).cuda()


def _run(ta, x, w, dtype, config=None):
    import torch
    y = ta.attn_gemm_splitk(_dev(x, dtype), _dev(w, dtype), config=config)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def _check(ta, M, N, K, dtype, seed, config=None, what=""):
    d = W.gemm_inputs(M, N, K, dtype, seed)
    _note(f"[case] gemm {what} M={M} N={N} K={K} {dtype} config={config}")
    y = _run(ta, d["x"], d["w"], dtype, config)
    ref = G.linear(d["x"], d["w"])
    bound = G.error_bound(d["x"], d["w"], dtype)
    err = np.abs(y - ref)
    ratio = float((err / bound).max()) if err.size else 0.0
    _note(f"[parity] gemm {what}: max|dy|={err.max() if err.size else 0:.3e} max err/bound={ratio:.3f}")
    assert np.isfinite(y).all()
    assert ratio <= 1.0, f"{what}: error exceeds the bound (ratio {ratio})"
    return y


@pytest.mark.parametrize("layer", list(W.LINEAR_SHAPES))
@pytest.mark.parametrize("M", [1, 2])
def test_llama_linear_layers(ta, layer, M):
    N, K = W.LINEAR_SHAPES[layer]
    _check(ta, M, N, K, "bf16", seed=60 + M, what=layer)


@pytest.mark.parametrize("layer", ["qkv_proj", "down_proj"])
def test_llama_linear_layers_fp16(ta, layer):
    N, K = W.LINEAR_SHAPES[layer]
    _check(ta, 2, N, K, "fp16", seed=63, what=layer)


@pytest.mark.parametrize("M", [1, 3, 16, 17, 32, 33, 44, 63, 64, 65, 130])
@pytest.mark.parametrize("N,K", [(1, 8), (15, 24), (17, 40), (100, 328), (257, 1000)])
def test_ragged_shapes(ta, M, N, K):
    _check(ta, M, N, K, "bf16" if (M + N) % 2 else "fp16", seed=M * 1000 + N, what="ragged")


CONFIGS = [(r, wv, u) for r in (16, 32) for wv in (1, 2, 3, 5, 8, 16) for u in (1, 2, 4, 8)]


@pytest.mark.parametrize("config", CONFIGS, ids=lambda c: f"r{c[0]}w{c[1]}u{c[2]}")
def test_every_configuration(ta, config):
    _check(ta, 19, 83, 2056, "bf16", seed=70, config=config, what="config")


@pytest.mark.parametrize("config", [(32, 16, 8), (32, 16, 1), (16, 16, 4)])
def test_largest_reduction_tiles(ta, config):
    """64 activation rows with 32 weight rows and 16 waves: 128 KiB of partial tiles in LDS."""
    _check(ta, 64, 200, 4096, "bf16", seed=73, config=config, what="64 rows")


def test_zero_k_gives_zero(ta):
    import torch
    x = torch.empty((3, 0), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((40, 0), dtype=torch.bfloat16, device="cuda")
    y = ta.attn_gemm_splitk(x, w)
    torch.cuda.synchronize()
    assert y.shape == (3, 40) and bool((y == 0).all())


def test_empty_m_or_n(ta):
    import torch
    x = torch.zeros((0, 64), dtype=torch.float16, device="cuda")
    w = torch.zeros((16, 64), dtype=torch.float16, device="cuda")
    assert ta.attn_gemm_splitk(x, w).shape == (0, 16)
    assert ta.attn_gemm_splitk(torch.zeros((2, 64), dtype=torch.float16, device="cuda"),
                               torch.zeros((0, 64), dtype=torch.float16, device="cuda")).shape == (2, 0)


def test_deterministic(ta):
    N, K = W.LINEAR_SHAPES["o_proj"]
    d = W.gemm_inputs(2, N, K, "bf16", seed=71)
    y1 = _run(ta, d["x"], d["w"], "bf16")
    y2 = _run(ta, d["x"], d["w"], "bf16")
    assert np.array_equal(y1, y2)


def test_rows_beyond_m_do_not_leak(ta):
    """y rows past M are never written: a larger output buffer keeps its sentinel."""
    import torch
    d = W.gemm_inputs(5, 48, 64, "bf16", seed=72)
    x = _dev(d["x"], "bf16")
    w = _dev(d["w"], "bf16")
    big = torch.full((8, 48), 7.0, dtype=torch.bfloat16, device="cuda")
    ta.attn_gemm_splitk(x, w, out=big[:5])
    torch.cuda.synchronize()
    assert bool((big[5:] == 7.0).all())
    ref = G.linear(d["x"], d["w"])
    assert (np.abs(big[:5].float().cpu().numpy() - ref) <= G.error_bound(d["x"], d["w"], "bf16")).all()
