"""CPU oracle for rotary position embedding fused into attention (test infrastructure).

This module is test infrastructure. Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import or run it; the library never does.
It shares no code with the HIP path.

Source: the Llama3-8B inference trace of comemg.com, "天下苦英偉達久矣！PyTorch
免CUDA加速推理，Triton時代要來？", section "模型推理", lists RoPE among the small
kernels that run between the matrix products and attention; the-ai.news page
("Snelle attention-kernels en operatorfusie versnellen AI-modellen", operator
fusion section) gives the reason to fuse such a step into its neighbour: it
saves a round trip of the tensor through memory. The pages do not define the
rotation; the oracle takes the rotary embedding in the half-split layout of
the Llama family (readings in the design notes):

    for a row x of D values at position p and i < D/2, with c = C[p, i] and
    s = S[p, i] from the caller's table (cos / sin of p * theta_i):
        x'[i]       = x[i] * c - x[i + D/2] * s
        x'[i + D/2] = x[i + D/2] * c + x[i] * s

The table is an input (float32 [max_pos, D]: cosines in columns 0 .. D/2-1,
sines in D/2 .. D-1), as a serving engine computes it once; the rotation is
applied in float64 to the exact input values. A rotated row then enters a
16-bit tensor (the key cache, the query operand of the products), so it is
rounded once to that type, to nearest with ties to even.
"""
from __future__ import annotations

import numpy as np

from . import oracle as O

__all__ = ["round16", "rotate", "rope_rows", "cache_append_rope", "prefill_paged_rope", "decode_paged_rope"]

# significant bits and smallest normal exponent (frexp convention) of the two 16-bit types
_FMT = {"bf16": (8, -125), "fp16": (11, -13)}


def round16(x, dtype) -> np.ndarray:
    """float64 values rounded once to bf16 / fp16 (nearest, ties to even; subnormal steps below the
    smallest normal), returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    bits, emin = _FMT[dtype]
    _, e = np.frexp(x)
    step = np.exp2(np.maximum(e, emin).astype(np.float64) - bits)
    return np.rint(x / step) * step


def rotate(x, pos, table) -> np.ndarray:
    """Rotate rows x [..., D] at positions pos (broadcast to x's leading shape) with table [max_pos, D]."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    h = D // 2
    t = np.asarray(table, dtype=np.float64)[np.asarray(pos)]
    c, s = t[..., :h], t[..., h:]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_rows(x, first_pos, table) -> np.ndarray:
    """x [B, H, T, D]: row t of sequence b sits at position first_pos[b] + t."""
    B, H, T, D = x.shape
    pos = np.asarray(first_pos, dtype=np.int64)[:, None, None] + np.arange(T)[None, None, :]
    pos = np.broadcast_to(pos, (B, H, T))
    # rows past the table (padding only) read its ends; they never reach a result
    return rotate(x, np.clip(pos, 0, len(table) - 1), table)


def cache_append_rope(k_new, v_new, k_cache, v_cache, block_table, start_pos, table, dtype, new_lens=None):
    """Append with K rotated at its position (start_pos[b] + i) and rounded to the cache's 16-bit type;
    V as given. Returns float64 caches."""
    k_rot = round16(rope_rows(k_new, start_pos, table), dtype)
    return O.cache_append(k_rot, np.asarray(v_new, dtype=np.float64), np.asarray(k_cache, dtype=np.float64),
                          np.asarray(v_cache, dtype=np.float64), block_table, start_pos, new_lens)


def prefill_paged_rope(q, k_cache, v_cache, block_table, ctx_lens, q_lens, table, scale, dtype, causal=True):
    """Chunked prefill whose query rows are rotated at their positions (ctx - q_len + i) and rounded to
    the 16-bit type first; the cache holds already-rotated keys."""
    B, Hq, Tq, _ = q.shape
    ql = np.full(B, Tq) if q_lens is None else np.asarray(q_lens)
    first = np.asarray(ctx_lens) - ql
    qr = round16(rope_rows(q, first, table), dtype)
    return O.prefill_paged(qr, k_cache, v_cache, block_table, ctx_lens, q_lens, scale, causal)


def decode_paged_rope(q, k_cache, v_cache, block_table, ctx_lens, table, scale, dtype):
    """One-token decode whose query is rotated at position ctx - 1 (and rounded to the 16-bit type)
    first; the cache holds rotated keys."""
    pos = np.asarray(ctx_lens, dtype=np.int64) - 1
    qr = round16(rotate(q, np.broadcast_to(pos[:, None], q.shape[:2]), table), dtype)
    return O.decode_paged(qr, k_cache, v_cache, block_table, ctx_lens, scale)
