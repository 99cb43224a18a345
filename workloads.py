"""Seeded synthetic inputs for the attention workloads (shared by tests, bench and smoke).

This module only draws random numbers, rounds them to the storage dtype and lays
them out (padding, paged cache, block table). It holds none of the attention
arithmetic: the CPU oracle and the HIP library both receive what it returns.

Workload shapes are those of the five attention cases this library is measured
on: a tiny 128x128 head, a BERT-base-shaped ragged encoder batch, a
Llama3-8B-shaped causal prefill (batch 2, 512 tokens, 32/8 heads), a
Qwen2.5-1.5B-shaped paged decode batch (64 sequences, 12/2 heads, 16-token
blocks) and a 16384-token causal prefill. Values are N(0,1) as the pages'
micro-benchmarks use random activations; the paged cache is laid out with a
seeded random permutation of physical blocks, as in a vLLM-style block pool.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BLOCK = 16  # tokens per KV-cache block (vLLM example uses block_size=16)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to bf16/fp16 (round to nearest even); return float32 holding them."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp16":
        return x.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        lsb = (u >> 16) & 1
        u = (u + 0x7FFF + lsb) & 0xFFFF0000
        out = u.astype(np.uint32).view(np.float32)
        # keep NaN payloads NaN (inputs are finite except planted sentinels)
        out = np.where(np.isnan(x), np.float32("nan"), out)
        return out
    if dtype == "fp32":
        return x
    raise ValueError(dtype)


@dataclass
class PrefillCase:
    name: str
    B: int
    Hq: int
    Hkv: int
    T: int
    D: int
    dtype: str
    causal: bool
    ragged: bool
    seed: int
    scale: float = field(default=0.0)

    def __post_init__(self):
        if self.scale == 0.0:
            self.scale = 1.0 / math.sqrt(self.D)


@dataclass
class DecodeCase:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    dtype: str
    ctx_lo: int
    ctx_hi: int
    seed: int
    spare_blocks: int = 8
    scale: float = field(default=0.0)

    def __post_init__(self):
        if self.scale == 0.0:
            self.scale = 1.0 / math.sqrt(self.D)


@dataclass
class ChunkCase:
    """A chunked-prefill batch through the paged cache: each sequence already
    holds ctx tokens (uniform in [ctx_lo, ctx_hi]) and receives a chunk of n new
    tokens (uniform in [chunk_lo, chunk_hi]); queries are padded to Tq = chunk_hi."""
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    dtype: str
    ctx_lo: int
    ctx_hi: int
    chunk_lo: int
    chunk_hi: int
    seed: int
    spare_blocks: int = 8
    scale: float = field(default=0.0)

    def __post_init__(self):
        if self.scale == 0.0:
            self.scale = 1.0 / math.sqrt(self.D)


# The five measured cases.
TINY = PrefillCase("tiny fp16 1x1x128x64", B=1, Hq=1, Hkv=1, T=128, D=64, dtype="fp16",
                   causal=False, ragged=False, seed=1)
BERT = PrefillCase("bert-base ragged fp16 B=8 H=12 Tmax=512 D=64", B=8, Hq=12, Hkv=12, T=512, D=64,
                   dtype="fp16", causal=False, ragged=True, seed=2)
LLAMA = PrefillCase("llama3-8b causal bf16 B=2 Hq=32 Hkv=8 T=512 D=128", B=2, Hq=32, Hkv=8, T=512, D=128,
                    dtype="bf16", causal=True, ragged=False, seed=3)
QWEN = DecodeCase("qwen2.5-1.5b paged decode bf16 B=64 Hq=12 Hkv=2 D=128 ctx~U[512,4096]", B=64, Hq=12,
                  Hkv=2, D=128, dtype="bf16", ctx_lo=512, ctx_hi=4096, seed=4)
LONG = PrefillCase("long causal bf16 B=1 Hq=32 Hkv=8 T=16384 D=128", B=1, Hq=32, Hkv=8, T=16384, D=128,
                   dtype="bf16", causal=True, ragged=False, seed=5)

ALL_PREFILL = [TINY, BERT, LLAMA, LONG]

# Chunked prefill of a long prompt against its cached prefix (llama3-8b heads).
CHUNK = ChunkCase("chunked prefill llama3-8b bf16 B=4 Hq=32 Hkv=8 D=128 prefix~U[2048,8192] chunk=1024", B=4,
                  Hq=32, Hkv=8, D=128, dtype="bf16", ctx_lo=2048, ctx_hi=8192, chunk_lo=1024, chunk_hi=1024,
                  seed=6)


def prefill_inputs(case: PrefillCase, nan_padding: bool = False, Tq: int | None = None,
                   Tk: int | None = None):
    """Return dict(q, k, v, seq_lens) as float32 numpy arrays holding dtype-rounded values.

    Draw order: q, k, v (N(0,1), float32) then the ragged lengths. Lengths are
    uniform integers in [64, T] (both ends included). With ``nan_padding`` the
    padded rows (position >= length) of q, k and v are set to NaN.
    """
    rng = np.random.default_rng(case.seed)
    Tq = case.T if Tq is None else Tq
    Tk = case.T if Tk is None else Tk
    q = rng.standard_normal((case.B, case.Hq, Tq, case.D), dtype=np.float32)
    k = rng.standard_normal((case.B, case.Hkv, Tk, case.D), dtype=np.float32)
    v = rng.standard_normal((case.B, case.Hkv, Tk, case.D), dtype=np.float32)
    q, k, v = (round_to(a, case.dtype) for a in (q, k, v))
    seq_lens = None
    if case.ragged:
        lo = min(64, case.T)
        seq_lens = rng.integers(lo, case.T + 1, case.B).astype(np.int32)
        if nan_padding:
            for b, L in enumerate(seq_lens):
                q[b, :, L:, :] = np.nan
                k[b, :, L:, :] = np.nan
                v[b, :, L:, :] = np.nan
    return dict(q=q, k=k, v=v, seq_lens=seq_lens)


def decode_inputs(case: DecodeCase, nan_fill: bool = False, ctx_lens=None):
    """Return dict(q, k_cache, v_cache, block_table, ctx_lens) for a paged decode batch.

    Draw order: context lengths (uniform integers in [ctx_lo, ctx_hi]), then a
    permutation of the physical blocks, then q, k_cache, v_cache (N(0,1)).
    Logical block i of sequence b maps to physical block perm[off_b + i];
    unused table entries are -1. ``spare_blocks`` extra physical blocks are never
    referenced. With ``nan_fill`` unused slots (tail of the last block and the
    spare blocks) hold NaN.
    """
    rng = np.random.default_rng(case.seed)
    if ctx_lens is None:
        ctx = rng.integers(case.ctx_lo, case.ctx_hi + 1, case.B).astype(np.int32)
    else:
        ctx = np.asarray(ctx_lens, dtype=np.int32)
    nblk = (ctx + BLOCK - 1) // BLOCK
    used = int(nblk.sum())
    NB = used + case.spare_blocks
    perm = rng.permutation(used).astype(np.int32)
    max_blocks = int(-(-case.ctx_hi // BLOCK))
    max_blocks = max(max_blocks, int(nblk.max()))
    table = np.full((case.B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(case.B):
        table[b, : nblk[b]] = perm[off: off + nblk[b]]
        off += nblk[b]
    q = rng.standard_normal((case.B, case.Hq, case.D), dtype=np.float32)
    kc = rng.standard_normal((NB, case.Hkv, BLOCK, case.D), dtype=np.float32)
    vc = rng.standard_normal((NB, case.Hkv, BLOCK, case.D), dtype=np.float32)
    q, kc, vc = (round_to(a, case.dtype) for a in (q, kc, vc))
    if nan_fill:
        for b in range(case.B):
            tail = int(ctx[b]) % BLOCK
            if tail:
                last = table[b, nblk[b] - 1]
                kc[last, :, tail:, :] = np.nan
                vc[last, :, tail:, :] = np.nan
        kc[used:] = np.nan
        vc[used:] = np.nan
    return dict(q=q, k_cache=kc, v_cache=vc, block_table=table, ctx_lens=ctx)


E4M3_NAN = 0x7F  # an E4M3 NaN code (S.1111.111)


def e4m3_codes(rng, shape, exp_lo=4, exp_hi=9, p_zero=0.02, p_sub=0.02):
    """Random E4M3 codes (uint8) drawn field by field: random sign and mantissa,
    exponent field uniform in [exp_lo, exp_hi] (values of magnitude 2^-3 ..
    1.875 * 2^2 by default), a fraction p_zero of zeros and p_sub of subnormals
    (exponent field 0). No arithmetic on values: the codes are the inputs."""
    sign = rng.integers(0, 2, shape).astype(np.uint8) << 7
    exp = rng.integers(exp_lo, exp_hi + 1, shape).astype(np.uint8)
    mant = rng.integers(0, 8, shape).astype(np.uint8)
    u = rng.random(shape)
    exp = np.where(u < p_zero + p_sub, 0, exp).astype(np.uint8)
    mant = np.where(u < p_zero, 0, mant).astype(np.uint8)
    return (sign | (exp << 3) | mant).astype(np.uint8)


def decode_inputs_fp8(case: DecodeCase, nan_fill: bool = False, ctx_lens=None):
    """decode_inputs with E4M3 caches: q, block_table and ctx_lens as there;
    k_cache / v_cache are uint8 codes from e4m3_codes (generator seeded with
    seed + 1000). With ``nan_fill`` every unused slot holds the NaN code."""
    x = decode_inputs(case, nan_fill=True, ctx_lens=ctx_lens)
    rng = np.random.default_rng(case.seed + 1000)
    k8 = e4m3_codes(rng, x["k_cache"].shape)
    v8 = e4m3_codes(rng, x["v_cache"].shape)
    if nan_fill:
        k8[np.isnan(x["k_cache"])] = E4M3_NAN
        v8[np.isnan(x["v_cache"])] = E4M3_NAN
    return dict(q=x["q"], k_cache=k8, v_cache=v8, block_table=x["block_table"], ctx_lens=x["ctx_lens"])


def rope_table(max_pos: int, D: int, base: float = 500000.0) -> np.ndarray:
    """Input table of a rotary embedding, float32 [max_pos, D]: cos(p * theta_i) in column i and
    sin(p * theta_i) in column D/2 + i, theta_i = base^(-2i/D) (the Llama-3 frequencies), computed in
    float64 and rounded to float32. An input like a weight: the kernels and the oracle only read it."""
    i = np.arange(D // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / D)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * theta[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def prefill_inputs_fp8(case: PrefillCase, Tq: int | None = None, Tk: int | None = None):
    """prefill_inputs' shapes and ragged lengths with E4M3 codes for q, k, v (e4m3_codes, generator seeded
    with seed + 2000); padding positions (>= seq_lens[b]) hold the NaN code."""
    x = prefill_inputs(case, nan_padding=True, Tq=Tq, Tk=Tk)
    rng = np.random.default_rng(case.seed + 2000)
    out = {}
    for n in ("q", "k", "v"):
        c = e4m3_codes(rng, x[n].shape)
        c[np.isnan(x[n])] = E4M3_NAN
        out[n] = c
    out["seq_lens"] = x["seq_lens"]
    return out


def chunk_inputs(case: ChunkCase, nan_fill: bool = False, starts=None, lens=None):
    """Return dict(q, k_new, v_new, k_cache, v_cache, block_table, start_pos, new_lens, ctx_lens).

    Draw order: context lengths before the chunk, chunk lengths, a permutation
    of the physical blocks (enough for context + chunk), then q [B,Hq,Tq,D],
    k_new / v_new [B,Hkv,Tq,D] and the caches (N(0,1)). The caches hold
    values at every slot, the chunk's own positions included: appending the
    chunk overwrites them. ctx_lens = start_pos + new_lens. With ``nan_fill``
    the chunk's positions in the cache, the tail of each last block, the spare
    blocks and the padded rows of q / k_new / v_new hold NaN. ``starts`` /
    ``lens`` replace the drawn context / chunk lengths (the draws still happen,
    so the other arrays do not change).
    """
    rng = np.random.default_rng(case.seed)
    start = rng.integers(case.ctx_lo, case.ctx_hi + 1, case.B).astype(np.int32)
    n = rng.integers(case.chunk_lo, case.chunk_hi + 1, case.B).astype(np.int32)
    if starts is not None:
        start = np.asarray(starts, dtype=np.int32)
    if lens is not None:
        n = np.asarray(lens, dtype=np.int32)
    assert start.shape == (case.B,) and n.shape == (case.B,) and (n <= case.chunk_hi).all()
    total = start + n
    nblk = (total + BLOCK - 1) // BLOCK
    used = int(nblk.sum())
    NB = used + case.spare_blocks
    perm = rng.permutation(used).astype(np.int32)
    max_blocks = int(-(-max(case.ctx_hi + case.chunk_hi, int(total.max())) // BLOCK))
    table = np.full((case.B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(case.B):
        table[b, : nblk[b]] = perm[off: off + nblk[b]]
        off += nblk[b]
    Tq = case.chunk_hi
    q = rng.standard_normal((case.B, case.Hq, Tq, case.D), dtype=np.float32)
    kn = rng.standard_normal((case.B, case.Hkv, Tq, case.D), dtype=np.float32)
    vn = rng.standard_normal((case.B, case.Hkv, Tq, case.D), dtype=np.float32)
    kc = rng.standard_normal((NB, case.Hkv, BLOCK, case.D), dtype=np.float32)
    vc = rng.standard_normal((NB, case.Hkv, BLOCK, case.D), dtype=np.float32)
    q, kn, vn, kc, vc = (round_to(a, case.dtype) for a in (q, kn, vn, kc, vc))
    if nan_fill:
        for b in range(case.B):
            q[b, :, n[b]:] = np.nan
            kn[b, :, n[b]:] = np.nan
            vn[b, :, n[b]:] = np.nan
            pos = np.arange(start[b], total[b])
            kc[table[b, pos // BLOCK], :, pos % BLOCK] = np.nan
            vc[table[b, pos // BLOCK], :, pos % BLOCK] = np.nan
            tail = int(total[b]) % BLOCK
            if tail:
                last = table[b, nblk[b] - 1]
                kc[last, :, tail:, :] = np.nan
                vc[last, :, tail:, :] = np.nan
        kc[used:] = np.nan
        vc[used:] = np.nan
    return dict(q=q, k_new=kn, v_new=vn, k_cache=kc, v_cache=vc, block_table=table, start_pos=start,
                new_lens=n, ctx_lens=total)


def chunk_flops(ctx_lens, q_lens, Hq, D, causal=True):
    """Algorithmic flops of a chunked prefill: 4*D per visible (query, key) pair."""
    pairs = 0
    for L, n in zip(np.asarray(ctx_lens), np.asarray(q_lens)):
        L, n = int(L), int(n)
        pairs += sum(L - n + i + 1 for i in range(n)) if causal else n * L
    return 4.0 * D * Hq * pairs


def append_bytes(new_lens, Hkv, D, elem=2):
    """Algorithmic HBM bytes of an append: the new K and V read once and written once."""
    n = int(np.asarray(new_lens, dtype=np.int64).sum())
    return 2 * 2 * n * Hkv * D * elem


def prefill_flops(B, Hq, Tq, Tk, D, causal, seq_lens=None):
    """Algorithmic flops: 4*D per unmasked (query, key) pair (QK^T and PV, one multiply-add each)."""
    pairs = 0
    for b in range(B):
        Lq = Tq if seq_lens is None else int(seq_lens[b])
        Lk = Tk if seq_lens is None else int(seq_lens[b])
        if causal:
            off = Lk - Lq
            for_rows = 0
            # row i sees keys 0..min(Lk-1, i+off)
            for i in range(Lq):
                n = min(Lk, i + off + 1)
                for_rows += max(0, n)
            pairs += for_rows
        else:
            pairs += Lq * Lk
    return 4.0 * D * Hq * pairs


def prefill_bytes(B, Hq, Hkv, Tq, Tk, D, seq_lens=None, elem=2):
    """Algorithmic HBM bytes of one prefill call: q and o of the valid rows, k and v of the valid keys (once per
    kv head), and the lse of the valid rows (fp32)."""
    total = 0
    for b in range(B):
        Lq = Tq if seq_lens is None else int(seq_lens[b])
        Lk = Tk if seq_lens is None else int(seq_lens[b])
        total += 2 * Hq * Lq * D * elem + 2 * Hkv * Lk * D * elem + Hq * Lq * 4
    return total


def decode_bytes(ctx_lens, Hq, Hkv, D, elem=2, max_blocks=None, kv_elem=None):
    """Algorithmic HBM bytes of one paged decode call.

    K and V of every valid token, read once per kv head (kv_elem bytes per
    element, default elem; 1 for an E4M3 cache), plus q, o (elem bytes), lse
    (fp32), ctx_lens and the block-table entries actually read.
    """
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    B = ctx.shape[0]
    kv = int(ctx.sum()) * Hkv * D * (elem if kv_elem is None else kv_elem) * 2
    qo = 2 * B * Hq * D * elem
    lse = B * Hq * 4
    table = int(((ctx + BLOCK - 1) // BLOCK).sum()) * 4
    return kv + qo + lse + table + 4 * B


# Linear layers of a Llama3-8B / Granite-8B transformer block (hidden 4096, 32 query and 8 kv heads of
# 128, MLP width 14336), as weight shapes (N = out_features, K = in_features): fused q/k/v projection,
# output projection, fused gate/up projection, down projection. Decode runs them at M = batch tokens
# (the pages' end-to-end runs: batch 2; their decode micro-benchmark: batch 1).
LINEAR_SHAPES = {
    "qkv_proj": (6144, 4096),
    "o_proj": (4096, 4096),
    "gate_up_proj": (28672, 4096),
    "down_proj": (4096, 14336),
}
LINEAR_M = 2


def gemm_inputs(M: int, N: int, K: int, dtype: str, seed: int):
    """Activations x [M, K] ~ N(0, 1) and weights w [N, K] ~ N(0, 1/K), rounded to dtype (float32
    arrays holding the 16-bit values), so that y = x w^T has entries of order 1."""
    rng = np.random.default_rng(seed)
    x = round_to(rng.standard_normal((M, K), dtype=np.float32), dtype)
    w = round_to(rng.standard_normal((N, K), dtype=np.float32) / np.float32(math.sqrt(K)), dtype)
    return dict(x=x, w=w)


def gemm_bytes(M: int, N: int, K: int, elem: int = 2) -> int:
    """Algorithmic HBM bytes of y = x w^T: the weight, the activations and the output, each once."""
    return (N * K + M * K + M * N) * elem
