"""GPU parity on seeded random configurations (through the C ABI, against the float64 oracle).

Each case draws its configuration from its own seed (numpy default_rng), so a failure names a
reproducible case: prefill (batch, heads with GQA groups 1-8, Tq / Tk from 1 to 300 including
Tq != Tk, D 64 / 128, bf16 / fp16, causal or not, ragged or not, scale drawn from a wide range),
paged decode (context lengths 1 to 2000 mixed within a batch, head layouts, scale), chunked prefill
(prefixes 0 to 1500, chunks 0 to 200), decode over E4M3 caches (contexts 1 to 2000, scales drawn
over four decades), chunked prefill with the rotary embedding fused and over E4M3 caches, and the
split-K GEMM (M 1 to 40, N 1 to 700, K a multiple of 8
up to 3000, a random configuration). Tolerances are those of the hand-picked parity tests: per element
max(stated bound, the budget of the stated arithmetic, oracle/bounds.py); the rotary cases, whose
queries the kernel rounds after its own fp32 rotation, use max(stated bound, half an ulp).
"""
import numpy as np
import pytest

import workloads as W
from oracle import bounds as BD
from oracle import fp8 as F8
from oracle import gemm as G
from oracle import oracle as O
from oracle import rope as R
from test_chunked_gpu import _chunk_check
from test_fp8_gpu import _decode_fp8_check, _fp8_chunk_inputs
from test_parity_gpu import _compare, _decode_check, _dev, _note, _run_prefill
from test_rope_gpu import _append as _rope_append, _check_append, _table

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta(gpu):
    import torch  # noqa: F401
    import tiled_attention_02_amd as ta
    ta.lib()
    return ta


def _heads(rng):
    hkv = int(rng.integers(1, 5))
    g = int(rng.choice([1, 2, 3, 4, 6, 8]))
    return hkv * g, hkv


@pytest.mark.parametrize("seed", range(1000, 1048))
def test_random_prefill(ta, seed):
    rng = np.random.default_rng(seed)
    hq, hkv = _heads(rng)
    D = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "fp16"]))
    causal = bool(rng.integers(0, 2))
    ragged = bool(rng.integers(0, 4) == 0)
    T = int(rng.integers(1, 301))
    Tq, Tk = T, T
    if not ragged and rng.integers(0, 2):
        Tq, Tk = int(rng.integers(1, 301)), int(rng.integers(1, 301))
    scale = float(rng.choice([1.0 / np.sqrt(D), 0.0, -0.2, 0.01, 1.0]))
    B = int(rng.integers(1, 4))
    # the scale is passed explicitly below (0.0 is valid: uniform weights)
    case = W.PrefillCase(f"random prefill {seed}", B=B, Hq=hq, Hkv=hkv, T=T, D=D, dtype=dtype, causal=causal,
                         ragged=ragged and T >= 2, seed=seed)
    x = W.prefill_inputs(case, nan_padding=True, Tq=Tq, Tk=Tk)
    _note(f"[case] random prefill seed={seed} B={B} Hq={hq} Hkv={hkv} Tq={Tq} Tk={Tk} D={D} {dtype} "
          f"causal={causal} ragged={x['seq_lens'] is not None} scale={scale}")
    o, lse = _run_prefill(ta, x, case, causal, scale)
    o_ref, lse_ref = O.prefill(x["q"], x["k"], x["v"], scale, causal, x["seq_lens"])
    bound = BD.prefill(x["q"], x["k"], x["v"], scale, causal, x["seq_lens"], dtype)
    _compare(o, lse, o_ref, lse_ref, dtype, what=f"random prefill {seed}", bound=bound)


@pytest.mark.parametrize("seed", range(2000, 2036))
def test_random_decode(ta, seed):
    rng = np.random.default_rng(seed)
    hq, hkv = _heads(rng)
    D = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "fp16"]))
    B = int(rng.integers(1, 9))
    ctx = rng.integers(1, 2001, B)
    ctx[rng.integers(0, B)] = int(rng.choice([1, 16, 256, 257, 2000]))
    scale = float(rng.choice([1.0 / np.sqrt(D), -0.1, 0.3]))
    case = W.DecodeCase(f"random decode {seed}", B=B, Hq=hq, Hkv=hkv, D=D, dtype=dtype, ctx_lo=1,
                        ctx_hi=int(ctx.max()), seed=seed, scale=scale)
    _decode_check(ta, case, ctx_lens=ctx, scale=scale, what=f"random decode {seed} Hq={hq} Hkv={hkv} D={D} {dtype}")


@pytest.mark.parametrize("seed", range(5000, 5024))
def test_random_fp8_decode(ta, seed):
    rng = np.random.default_rng(seed)
    hq, hkv = _heads(rng)
    D = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "fp16"]))
    B = int(rng.integers(1, 9))
    ctx = rng.integers(1, 2001, B)
    ctx[rng.integers(0, B)] = int(rng.choice([1, 63, 64, 65, 256, 2000]))
    ks, vs = (float(10.0 ** rng.uniform(-3, 1)) for _ in range(2))
    case = W.DecodeCase(f"random fp8 decode {seed}", B=B, Hq=hq, Hkv=hkv, D=D, dtype=dtype, ctx_lo=1,
                        ctx_hi=int(ctx.max()), seed=seed)
    _decode_fp8_check(ta, case, ks, vs, ctx_lens=ctx,
                      what=f"random fp8 decode {seed} Hq={hq} Hkv={hkv} D={D} {dtype} ks={ks:.3g} vs={vs:.3g}")


@pytest.mark.parametrize("seed", range(3000, 3024))
def test_random_chunked_prefill(ta, seed):
    rng = np.random.default_rng(seed)
    hq, hkv = _heads(rng)
    D = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "fp16"]))
    B = int(rng.integers(1, 6))
    starts = [int(v) for v in rng.integers(0, 1501, B)]
    lens = [int(v) for v in rng.integers(0, 201, B)]
    lens[0] = max(lens[0], 1)
    causal = bool(rng.integers(0, 4) != 0)
    case = W.ChunkCase(f"random chunk {seed}", B=B, Hq=hq, Hkv=hkv, D=D, dtype=dtype, ctx_lo=0, ctx_hi=1500,
                       chunk_lo=0, chunk_hi=max(lens), seed=seed)
    _chunk_check(ta, case, causal=causal, starts=starts, lens=lens,
                 what=f"random chunk {seed} Hq={hq} Hkv={hkv} D={D} {dtype} causal={causal}")


@pytest.mark.parametrize("seed", range(4000, 4024))
def test_random_gemm(ta, seed):
    import torch
    rng = np.random.default_rng(seed)
    M = int(rng.integers(1, 41))
    N = int(rng.integers(1, 701))
    K = 8 * int(rng.integers(1, 376))
    dtype = str(rng.choice(["bf16", "fp16"]))
    config = (int(rng.choice([16, 32])), int(rng.integers(1, 17)), int(rng.choice([1, 2, 4, 8])))
    d = W.gemm_inputs(M, N, K, dtype, seed)
    _note(f"[case] random gemm seed={seed} M={M} N={N} K={K} {dtype} config={config}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    y = ta.attn_gemm_splitk(torch.from_numpy(d["x"]).to(tdt).cuda(), torch.from_numpy(d["w"]).to(tdt).cuda(),
                            config=config)
    torch.cuda.synchronize()
    err = np.abs(y.float().cpu().numpy() - G.linear(d["x"], d["w"]))
    ratio = float((err / G.error_bound(d["x"], d["w"], dtype)).max())
    _note(f"[parity] random gemm {seed}: max err/bound={ratio:.3f}")
    assert ratio <= 1.0


def _chunk_case(rng, seed, name):
    hq, hkv = _heads(rng)
    D = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "fp16"]))
    B = int(rng.integers(1, 5))
    starts = [int(v) for v in rng.integers(0, 1501, B)]
    lens = [int(v) for v in rng.integers(1, 201, B)]
    causal = bool(rng.integers(0, 4) != 0)
    case = W.ChunkCase(f"{name} {seed}", B=B, Hq=hq, Hkv=hkv, D=D, dtype=dtype, ctx_lo=0, ctx_hi=1500,
                       chunk_lo=1, chunk_hi=max(lens), seed=seed)
    return case, starts, lens, causal


@pytest.mark.parametrize("seed", range(6000, 6012))
def test_random_rope_chunked_prefill(ta, seed):
    import torch
    rng = np.random.default_rng(seed)
    case, starts, lens, causal = _chunk_case(rng, seed, "random rope chunk")
    x = W.chunk_inputs(case, nan_fill=True, starts=starts, lens=lens)
    tab, tab_d = _table(case.D)
    what = f"random rope chunk {seed} Hq={case.Hq} Hkv={case.Hkv} D={case.D} {case.dtype} causal={causal}"
    _note(f"[case] {what} start={starts} n={lens}")
    kc, vc = _rope_append(ta, x, case.dtype, tab_d)
    kref, vref = R.cache_append_rope(x["k_new"], x["v_new"], x["k_cache"], x["v_cache"], x["block_table"],
                                     x["start_pos"], tab, case.dtype, x["new_lens"])
    _check_append(kc, vc, kref, vref, case.dtype, what)
    o, lse = ta.attn_fwd_paged(_dev(x["q"], case.dtype), kc, vc, _i32(x["block_table"]), _i32(x["ctx_lens"]),
                               _i32(x["new_lens"]), scale=case.scale, causal=causal, rope=tab_d)
    torch.cuda.synchronize()
    o_ref, lse_ref = R.prefill_paged_rope(x["q"], kref, vref, x["block_table"], x["ctx_lens"], x["new_lens"], tab,
                                          case.scale, case.dtype, causal)
    _compare(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, case.dtype, what=what)


@pytest.mark.parametrize("seed", range(7000, 7012))
def test_random_fp8_chunked_prefill(ta, seed):
    import torch
    rng = np.random.default_rng(seed)
    case, starts, lens, causal = _chunk_case(rng, seed, "random fp8 chunk")
    case = W.ChunkCase(case.name, B=case.B, Hq=case.Hq, Hkv=case.Hkv, D=case.D, dtype=case.dtype, ctx_lo=0,
                       ctx_hi=1500, chunk_lo=1, chunk_hi=200, seed=seed)
    x, k8, v8 = _fp8_chunk_inputs(case, seed + 1)
    # scales over four decades each: values up to 75 in magnitude, whose P-rounding error the budget
    # scales with (the stated absolute bound alone cannot hold there)
    ks, vs = float(10.0 ** rng.uniform(-3, 1)), float(10.0 ** rng.uniform(-3, 1))
    what = f"random fp8 chunk {seed} Hq={case.Hq} Hkv={case.Hkv} D={case.D} {case.dtype} causal={causal}"
    _note(f"[case] {what} ctx={x['ctx_lens'].tolist()} n={x['new_lens'].tolist()} ks={ks:.3g} vs={vs:.3g}")
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    o, lse = ta.attn_fwd_paged_fp8(_dev(x["q"], case.dtype), u8(k8), u8(v8), ks, vs, _i32(x["block_table"]),
                                   _i32(x["ctx_lens"]), _i32(x["new_lens"]), scale=case.scale, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = F8.prefill_paged_fp8(x["q"], k8, v8, ks, vs, x["block_table"], x["ctx_lens"], x["new_lens"],
                                          case.scale, causal)
    bound = BD.prefill_paged(x["q"], F8.dequantize(k8, ks), F8.dequantize(v8, vs), x["block_table"],
                             x["ctx_lens"], x["new_lens"], case.scale, causal, case.dtype)
    _compare(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, case.dtype, what=what, bound=bound)


def _i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
