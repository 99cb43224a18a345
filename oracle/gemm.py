"""CPU oracle for the linear-layer matrix product (test infrastructure).

This module is test infrastructure. Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import or run it; the library never does.
It shares no code with the HIP path.

Source: comemg.com, "天下苦英偉達久矣！PyTorch免CUDA加速推理，Triton時代要來？",
section "Triton SplitK GEMM 內核": the linear layers of the Llama3-8B and
Granite-8B inference runs are FP16 matrix products computed by a GEMM kernel
that splits the reduction (K) dimension across workers; section "GEMM 內核調優"
tunes that kernel per weight shape (the shapes are that section's figure 4).
Splitting K only reorders the sum, so what the kernel computes has the plain
definition written out here, in float64 on the exact input values:

    y[m, n] = sum_k x[m, k] * w[n, k]

with x the activations [M, K] (one row per token) and w the layer's weight
[N, K] (out_features x in_features, the linear-layer convention y = x w^T).

Readings where the page is silent (listed in the design notes): no bias; the
output has the inputs' 16-bit type and is the exact sum rounded once, the
products and the running sums in between being float32 on the GPU; the error
that allows is `error_bound` below.
"""
from __future__ import annotations

import numpy as np

__all__ = ["linear", "ulp16", "error_bound"]

# significant bits and the exponent of the smallest normal number (frexp convention) of the 16-bit types
_FMT = {"bf16": (8, -125), "fp16": (11, -13)}


def linear(x, w) -> np.ndarray:
    """y = x w^T in float64: x [M, K], w [N, K] -> y [M, N]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError(f"shapes x {x.shape}, w {w.shape}: need [M, K] and [N, K]")
    return x @ w.T


def ulp16(y, dtype) -> np.ndarray:
    """Spacing of the 16-bit type at |y| (the subnormal spacing below its smallest normal)."""
    bits, emin = _FMT[dtype]
    a = np.abs(np.asarray(y, dtype=np.float64))
    _, e = np.frexp(a)
    e = np.where(a == 0, emin, np.maximum(e, emin))  # frexp(0) has exponent 0; zero lies in the subnormal range
    return np.exp2(e.astype(np.float64) - bits)


def error_bound(x, w, dtype) -> np.ndarray:
    """Per-element bound on |y_gpu - y| for a computation that forms the K products exactly in float32
    (16-bit by 16-bit products need at most 22 significant bits), adds them in float32 in any order
    (at most K - 1 roundings on the path of each product: |error| <= gamma_K * sum_k |x_mk w_nk| with
    gamma_K = K u / (1 - K u), u = 2^-24) and rounds the sum once to the 16-bit type (half a unit in the
    last place, taken here as one unit at |y| to cover the sum's own error moving it across a binade)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    K = x.shape[1]
    u = 2.0 ** -24
    gamma = K * u / (1.0 - K * u)
    return ulp16(linear(x, w), dtype) + gamma * (np.abs(x) @ np.abs(w).T)
