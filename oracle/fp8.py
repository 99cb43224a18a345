"""CPU oracle for the 8-bit floating-point (E4M3) KV cache (test infrastructure).

This module is test infrastructure. Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import or run it; the library never does.
It shares no code with the HIP path.

Sources. The pages name end-to-end FP8 inference as the next step for LLM
serving (comemg.com, "天下苦英偉達久矣！PyTorch免CUDA加速推理，Triton時代要來？",
section "未來工作"), quantized kernels that cut memory use (ai-stack.site,
kernels update commentary, section "关键技术点", item on quantization kernels),
and folding dequantisation into the consuming product as a standard fusion
(the-ai.news, "Snelle attention-kernels en operatorfusie versnellen
AI-modellen", section on operator fusion). The pages fix no format; the
format here is E4M3 of the OCP 8-bit floating point specification (the one
gfx950 converts natively): sign, 4 exponent bits with bias 7, 3 mantissa bits;
exponent field 0 holds subnormals m * 2^-9; S.1111.111 is NaN; there are no
infinities, so the largest finite magnitude is 1.75 * 2^8 = 448.

Readings (listed in the design notes):
  * one float32 scale per cache (k_scale, v_scale); a stored code is
    e4m3(x / scale) with x / scale a float32 division of the float32 value of
    x (bf16 / fp16 inputs are exact in float32), rounded to nearest with ties
    to the even code, magnitudes beyond 448 saturating to 448;
  * the cache entry means code_value * scale; attention over an FP8 cache is
    the definition of oracle.py applied to those dequantized values.
"""
from __future__ import annotations

import numpy as np

from . import oracle as O

__all__ = ["E4M3_MAX", "e4m3_to_float", "float_to_e4m3", "quantize", "dequantize", "cache_append_fp8",
           "decode_paged_fp8", "prefill_paged_fp8", "prefill_fp8"]

E4M3_MAX = 448.0


def e4m3_to_float(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8 array) as float64; NaN for S.1111.111."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def float_to_e4m3(x) -> np.ndarray:
    """E4M3 code (uint8) of float32 values: round to nearest, ties to even, saturating at +-448.

    For |x| in [2^k, 2^(k+1)) the representable step is 2^(k-3) (normal
    numbers, k >= -6) and 2^-9 below 2^-6 (subnormals): |x| is rounded to a
    multiple of that step (np.rint: ties to even, which is the even code since
    the code's last bit is the multiple's last bit), then clamped to 448.
    Infinities saturate like every other magnitude above 448. NaN maps to a NaN code with x's sign.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    nan = np.isnan(a)
    # saturation first: every magnitude above 448, infinity included, becomes 448 (the rounding below
    # would also take (448, 464] to 448, but has no step for infinity)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    k = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = np.exp2(np.maximum(k, -6.0) - 3.0)
    r = np.minimum(np.rint(a / step) * step, E4M3_MAX)
    # code fields of the rounded magnitude (it may have moved up a binade)
    sub = r < 2.0 ** -6
    e = np.where(sub, 0.0, np.floor(np.log2(np.where(r > 0, r, 1.0))) + 7.0)
    m = np.where(sub, r / 2.0 ** -9, (r / np.exp2(e - 7.0) - 1.0) * 8.0)
    code = (e.astype(np.int64) << 3) | np.rint(m).astype(np.int64)
    code = np.where(nan, 0x7F, code)
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)


def quantize(x, scale) -> np.ndarray:
    """Codes of x / scale (float32 division), as stored in an FP8 cache."""
    s = np.float32(scale)
    with np.errstate(over="ignore"):  # a quotient beyond float32's range is infinite, then saturates
        return float_to_e4m3(np.asarray(x, dtype=np.float32) / s)


def dequantize(codes, scale) -> np.ndarray:
    """What a stored code means: its value times the cache's scale (float64)."""
    return e4m3_to_float(codes) * float(np.float32(scale))


def cache_append_fp8(k_new, v_new, k_cache, v_cache, block_table, start_pos, k_scale, v_scale, new_lens=None):
    """Quantize new K/V ([B,Hkv,Tnew,D], float) and write the codes into copies of uint8 caches.

    Token i < new_lens[b] becomes position start_pos[b] + i of sequence b:
    block block_table[b, pos // block], slot pos % block. Nothing else changes.
    """
    kq = quantize(k_new, k_scale)
    vq = quantize(v_new, v_scale)
    return O.cache_append(kq, vq, k_cache, v_cache, block_table, start_pos, new_lens)


def decode_paged_fp8(q, k_cache, v_cache, k_scale, v_scale, block_table, ctx_lens, scale):
    """One-token decode over E4M3 caches (uint8 codes): the decode definition on the dequantized cache."""
    return O.decode_paged(q, dequantize(k_cache, k_scale), dequantize(v_cache, v_scale), block_table, ctx_lens,
                          scale)


def prefill_paged_fp8(q, k_cache, v_cache, k_scale, v_scale, block_table, ctx_lens, q_lens, scale, causal=True):
    """Chunked prefill over E4M3 caches: the chunked-prefill definition on the dequantized cache."""
    return O.prefill_paged(q, dequantize(k_cache, k_scale), dequantize(v_cache, v_scale), block_table, ctx_lens,
                           q_lens, scale, causal)


def prefill_fp8(q8, k8, v8, q_scale, k_scale, v_scale, scale, causal=False, seq_lens=None):
    """Prefill attention on E4M3 inputs: the prefill definition on the dequantized q, k, v."""
    return O.prefill(dequantize(q8, q_scale), dequantize(k8, k_scale), dequantize(v8, v_scale), scale, causal,
                     seq_lens)
