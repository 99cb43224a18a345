"""GPU parity of the E4M3 (FP8) KV cache: quantizing append and decode over it.

Both entry points are called through the C ABI and compared with the float64
oracle (oracle/fp8.py) on the same seeded inputs:
  - attn_cache_append_fp8 must produce the oracle's codes bit for bit (the
    float32 division and the rounding decide an integer code; both sides
    take that decision in float32), slots it must not touch unchanged;
  - attn_decode_paged_fp8 must match the decode definition over the
    dequantized cache to the library's tolerance (bf16 1e-2, fp16 2e-3 on O,
    1e-4 relative on lse): E4M3 values are exact in both 16-bit types, so the
    dequantization adds no error of its own;
  - with power-of-two scales the FP8 decode equals, bit for bit, the 16-bit
    decode of a cache that holds the dequantized values (the scales fold out
    of the products exactly).
Unused cache slots hold the E4M3 NaN code, so any read of them into a result
shows up.
"""
import numpy as np
import pytest

import workloads as W
from oracle import bounds as BD
from oracle import fp8 as F8
from test_parity_gpu import _compare, _dev, _note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta(gpu):
    import torch  # noqa: F401
    import tiled_attention_02_amd as ta
    ta.lib()
    return ta


def _u8(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).cuda()


def _i32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def _run_decode_fp8(ta, x, case, ks, vs, scale=None):
    import torch
    scale = case.scale if scale is None else scale
    o, lse = ta.attn_decode_paged_fp8(_dev(x["q"], case.dtype), _u8(x["k_cache"]), _u8(x["v_cache"]), ks, vs,
                                      _i32(x["block_table"]), _i32(x["ctx_lens"]), scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def _decode_fp8_check(ta, case, ks, vs, ctx_lens=None, what=None):
    x = W.decode_inputs_fp8(case, nan_fill=True, ctx_lens=ctx_lens)
    what = what or case.name
    _note(f"[case] fp8 decode {what} ks={ks} vs={vs} ctx[min,max]=({x['ctx_lens'].min()},{x['ctx_lens'].max()})")
    o, lse = _run_decode_fp8(ta, x, case, ks, vs)
    o_ref, lse_ref = F8.decode_paged_fp8(x["q"], x["k_cache"], x["v_cache"], ks, vs, x["block_table"],
                                         x["ctx_lens"], case.scale)
    bound = BD.decode_paged(x["q"], F8.dequantize(x["k_cache"], ks), F8.dequantize(x["v_cache"], vs),
                            x["block_table"], x["ctx_lens"], case.scale, case.dtype)
    _compare(o, lse, o_ref, lse_ref, case.dtype, what=f"fp8 decode {what}", bound=bound)
    return x, o, lse


# ---------------------------------------------------------------- decode over an E4M3 cache vs the oracle
def test_fp8_decode_qwen_shape(ta):
    case = W.DecodeCase("fp8 qwen", B=64, Hq=12, Hkv=2, D=128, dtype="bf16", ctx_lo=512, ctx_hi=4096, seed=81)
    _decode_fp8_check(ta, case, 0.25, 0.0625)


@pytest.mark.parametrize("Hq,Hkv,D,dtype,ks,vs", [(8, 8, 128, "bf16", 0.5, 2.0), (16, 1, 128, "fp16", 0.0173, 0.031),
                                                 (12, 2, 64, "fp16", 0.125, 0.125), (5, 1, 64, "bf16", 1.0, 0.3),
                                                 (32, 8, 128, "bf16", 0.09, 0.011)])
def test_fp8_decode_head_layouts(ta, Hq, Hkv, D, dtype, ks, vs):
    case = W.DecodeCase("fp8 heads", B=5, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, ctx_lo=1, ctx_hi=1500, seed=82)
    _decode_fp8_check(ta, case, ks, vs, what=f"Hq={Hq} Hkv={Hkv} D={D} {dtype}")


@pytest.mark.parametrize("ctx", [[1, 2, 15, 16, 17, 31, 32, 33], [48, 63, 64, 65, 127, 128, 129, 192],
                                 [255, 256, 257, 511, 512, 513, 1000, 4096], [33000, 20481, 4097, 12800]])
def test_fp8_decode_context_edges(ta, ctx):
    case = W.DecodeCase("fp8 edges", B=len(ctx), Hq=12, Hkv=2, D=128, dtype="bf16", ctx_lo=1, ctx_hi=4096, seed=83)
    _decode_fp8_check(ta, case, 0.3, 0.7, ctx_lens=ctx, what=f"ctx={ctx}")


def test_fp8_decode_extreme_codes(ta):
    """Codes across the whole finite range (exponent fields 0..15): large scores, subnormal values."""
    import torch
    case = W.DecodeCase("fp8 wide", B=4, Hq=8, Hkv=2, D=128, dtype="bf16", ctx_lo=100, ctx_hi=900, seed=84)
    x = W.decode_inputs_fp8(case, nan_fill=True)
    rng = np.random.default_rng(85)
    live = x["k_cache"] != W.E4M3_NAN
    wide = W.e4m3_codes(rng, x["k_cache"].shape, exp_lo=0, exp_hi=15)
    wide[(wide & 0x7F) == 0x7F] = 0x7E
    x["k_cache"] = np.where(live, wide, x["k_cache"]).astype(np.uint8)
    x["v_cache"] = np.where(live, W.e4m3_codes(rng, x["v_cache"].shape, exp_lo=0, exp_hi=14), x["v_cache"]).astype(np.uint8)
    ks, vs = 2.0 ** -9, 2.0 ** -4
    o, lse = _run_decode_fp8(ta, x, case, ks, vs)
    o_ref, lse_ref = F8.decode_paged_fp8(x["q"], x["k_cache"], x["v_cache"], ks, vs, x["block_table"],
                                         x["ctx_lens"], case.scale)
    bound = BD.decode_paged(x["q"], F8.dequantize(x["k_cache"], ks), F8.dequantize(x["v_cache"], vs),
                            x["block_table"], x["ctx_lens"], case.scale, "bf16")
    _compare(o, lse, o_ref, lse_ref, "bf16", what="fp8 decode wide codes", bound=bound)
    del torch


def test_fp8_decode_matches_16bit_decode_of_dequantized_cache(ta):
    """Power-of-two scales: the FP8 decode and the 16-bit decode over the dequantized values (exact in bf16)
    compute the same scores (the scales fold out exactly); the E4M3 kernel takes 64-token steps and the
    16-bit one 32-token steps, so their running maxima, and with them the bf16 roundings of the
    probabilities, can differ: each O is within 2^-8 max|v| of the exact weighted mean from that rounding,
    so the two agree within 2^-7 max|v| plus one unit in the last place; lse (fp32 sums of the unrounded
    probabilities) within 1e-6 relative."""
    import torch
    case = W.DecodeCase("fp8 vs bf16", B=16, Hq=12, Hkv=2, D=128, dtype="bf16", ctx_lo=1, ctx_hi=3000, seed=86)
    x = W.decode_inputs_fp8(case, nan_fill=False)
    ks, vs = 0.125, 0.5
    o8, l8 = _run_decode_fp8(ta, x, case, ks, vs)
    kd = F8.dequantize(x["k_cache"], ks).astype(np.float32)  # exact in bf16
    vd = F8.dequantize(x["v_cache"], vs).astype(np.float32)
    assert np.array_equal(W.round_to(kd, "bf16"), kd) and np.array_equal(W.round_to(vd, "bf16"), vd)
    o16, l16 = ta.attn_decode_paged(_dev(x["q"], "bf16"), _dev(kd, "bf16"), _dev(vd, "bf16"),
                                    _i32(x["block_table"]), _i32(x["ctx_lens"]), scale=case.scale)
    torch.cuda.synchronize()
    o16 = o16.float().cpu().numpy()
    l16 = l16.cpu().numpy()
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(o16), 2.0 ** -126))) - 7)
    same = float((o8 == o16).mean())
    _note(f"[parity] fp8 vs 16-bit decode: max |dO| = {float(np.abs(o8 - o16).max()):.2e}, "
          f"{100 * same:.2f} % identical, max rel dlse = {float((np.abs(l8 - l16) / np.abs(l16)).max()):.2e}")
    assert (np.abs(o8 - o16) <= 2.0 ** -7 * float(np.abs(vd).max()) + ulp).all()
    assert (np.abs(l8 - l16) <= 1e-6 * np.maximum(1.0, np.abs(l16))).all()


# ---------------------------------------------------------------- quantizing append vs the oracle
@pytest.mark.parametrize("D,dtype,ks,vs", [(128, "bf16", 0.0173, 0.0625), (64, "fp16", 0.5, 0.003),
                                         (128, "fp16", 1.0, 1.0), (64, "bf16", 0.25, 0.11)])
def test_fp8_append_codes_bit_exact(ta, D, dtype, ks, vs):
    import torch
    case = W.ChunkCase("fp8 append", B=3, Hq=8, Hkv=2, D=D, dtype=dtype, ctx_lo=0, ctx_hi=700, chunk_lo=0,
                       chunk_hi=300, seed=87)
    x = W.chunk_inputs(case, nan_fill=True)
    rng = np.random.default_rng(88)
    k8 = W.e4m3_codes(rng, x["k_cache"].shape)
    v8 = W.e4m3_codes(rng, x["v_cache"].shape)
    # some inputs beyond the format's range after scaling (saturation), some in the subnormal range
    kn = x["k_new"].copy()
    kn[:, :, ::7] *= 300.0
    kn[:, :, 3::11] *= 1e-3
    kn = W.round_to(kn, dtype)
    _note(f"[case] fp8 append D={D} {dtype} ks={ks} vs={vs} n={x['new_lens'].tolist()}")
    kc, vc = _u8(k8), _u8(v8)
    ta.attn_cache_append_fp8(_dev(kn, dtype), _dev(x["v_new"], dtype), kc, vc, ks, vs, _i32(x["block_table"]),
                             _i32(x["start_pos"]), _i32(x["new_lens"]))
    torch.cuda.synchronize()
    kref, vref = F8.cache_append_fp8(kn, x["v_new"], k8, v8, x["block_table"], x["start_pos"], ks, vs,
                                     x["new_lens"])
    assert np.array_equal(kc.cpu().numpy(), kref), "K codes differ"
    assert np.array_equal(vc.cpu().numpy(), vref), "V codes differ"


def _every_16bit_value(dtype):
    """Every finite 16-bit value of dtype and both infinities, as float32."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    if dtype == "bf16":
        v = (bits << 16).view(np.float32)
    else:
        v = bits.astype(np.uint16).view(np.float16).astype(np.float32)
    return v[~np.isnan(v)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("ks", [0.1, 1.0 / 3.0, 0.37, 0.0123, 1.0, 2.0 ** -100, 2.0 ** -101, 2.0 ** 100, 1e-35, 3e35])
def test_fp8_append_every_16bit_value(ta, dtype, ks):
    """Every finite 16-bit value (and +-inf) through the quantizing append, codes bit for bit against the
    oracle's float32 division and rounding: covers the multiply-and-correct division (scales in
    [2^-100, 2^100]) and the plain division (scales outside), saturation and the subnormal codes."""
    import torch
    vals = _every_16bit_value(dtype)
    D = 128
    n = -(-len(vals) // (16 * D)) * 16 * D  # whole cache blocks
    flat = np.zeros(n, dtype=np.float32)
    flat[:len(vals)] = vals
    T = n // D
    kn = flat.reshape(1, 1, T, D)
    vn = kn[:, :, ::-1].copy()
    nblk = T // 16
    table = np.arange(nblk, dtype=np.int32).reshape(1, nblk)
    k8 = np.full((nblk, 1, 16, D), W.E4M3_NAN, dtype=np.uint8)
    v8 = k8.copy()
    vs = 0.37 if ks != 0.37 else 0.1
    _note(f"[case] fp8 append every {dtype} value ks={ks} vs={vs} rows={T}")
    kc, vc = _u8(k8), _u8(v8)
    start = np.zeros(1, dtype=np.int32)
    ta.attn_cache_append_fp8(_dev(kn, dtype), _dev(vn, dtype), kc, vc, ks, vs, _i32(table), _i32(start), None)
    torch.cuda.synchronize()
    kref, vref = F8.cache_append_fp8(kn, vn, k8, v8, table, start, ks, vs)
    kg, vg = kc.cpu().numpy(), vc.cpu().numpy()
    for name, got, ref, src in (("K", kg, kref, kn), ("V", vg, vref, vn)):
        bad = np.nonzero(got.reshape(-1) != ref.reshape(-1))[0]
        if bad.size:
            xs = src.reshape(-1)[bad[:8]]
            _note(f"[mismatch] {name}: x={xs.tolist()} bits={[hex(int(b)) for b in xs.view(np.uint32)]} "
                  f"gpu={got.reshape(-1)[bad[:8]].tolist()} oracle={ref.reshape(-1)[bad[:8]].tolist()}")
    assert np.array_equal(kg, kref), f"K codes differ at {int((kg != kref).sum())} values"
    assert np.array_equal(vg, vref), f"V codes differ at {int((vg != vref).sum())} values"


def test_fp8_append_then_decode(ta):
    """A decode step as a server runs it: the new token's K/V quantized into the cache, then the decode."""
    import torch
    case = W.ChunkCase("fp8 step", B=6, Hq=12, Hkv=2, D=128, dtype="bf16", ctx_lo=0, ctx_hi=2000, chunk_lo=1,
                       chunk_hi=1, seed=89)
    x = W.chunk_inputs(case, nan_fill=True)
    rng = np.random.default_rng(90)
    k8 = W.e4m3_codes(rng, x["k_cache"].shape)
    v8 = W.e4m3_codes(rng, x["v_cache"].shape)
    ks, vs = 0.02, 0.013
    kc, vc = _u8(k8), _u8(v8)
    ta.attn_cache_append_fp8(_dev(x["k_new"], "bf16"), _dev(x["v_new"], "bf16"), kc, vc, ks, vs,
                             _i32(x["block_table"]), _i32(x["start_pos"]), None)
    o, lse = ta.attn_decode_paged_fp8(_dev(x["q"][:, :, 0], "bf16"), kc, vc, ks, vs, _i32(x["block_table"]),
                                      _i32(x["ctx_lens"]), scale=case.scale)
    torch.cuda.synchronize()
    kref, vref = F8.cache_append_fp8(x["k_new"], x["v_new"], k8, v8, x["block_table"], x["start_pos"], ks, vs)
    o_ref, lse_ref = F8.decode_paged_fp8(x["q"][:, :, 0], kref, vref, ks, vs, x["block_table"], x["ctx_lens"],
                                         case.scale)
    _compare(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "bf16", what="fp8 append + decode")


def test_fp8_rejects_bad_scales(ta):
    import torch
    q = torch.zeros((2, 4, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((4, 2, 16, 128), dtype=torch.uint8, device="cuda")
    bt, cl = _i32(np.zeros((2, 2))), _i32([1, 1])
    for ks, vs in ((0.0, 1.0), (1.0, -1.0), (float("nan"), 1.0), (1.0, float("inf"))):
        with pytest.raises(ta.AttnError, match="k_scale and v_scale"):
            ta.attn_decode_paged_fp8(q, kc, kc, ks, vs, bt, cl)


# ---------------------------------------------------------------- chunked prefill over an E4M3 cache
def _fp8_chunk_inputs(case, seed):
    """chunk_inputs' q, table and lengths over E4M3 caches whose slots at or past each sequence's context
    (and the spare blocks) hold the NaN code; every position < ctx holds a finite code."""
    x = W.chunk_inputs(case)
    rng = np.random.default_rng(seed)
    shape = x["k_cache"].shape
    k8 = W.e4m3_codes(rng, shape)
    v8 = W.e4m3_codes(rng, shape)
    used = np.zeros(shape[0] * 16, dtype=bool)
    for b in range(case.B):
        pos = np.arange(int(x["ctx_lens"][b]))
        used[x["block_table"][b, pos // 16] * 16 + pos % 16] = True
    unused = ~used.reshape(shape[0], 16)
    for a in (k8, v8):
        a.transpose(0, 2, 1, 3)[unused] = W.E4M3_NAN
    return x, k8, v8


@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "fp16"), (128, "fp16"), (64, "bf16")])
@pytest.mark.parametrize("causal", [True, False])
def test_fp8_chunked_prefill(ta, D, dtype, causal):
    import torch
    case = W.ChunkCase("fp8 chunk", B=3, Hq=8, Hkv=2, D=D, dtype=dtype, ctx_lo=0, ctx_hi=900, chunk_lo=1,
                       chunk_hi=300, seed=94)
    x, k8, v8 = _fp8_chunk_inputs(case, 95)
    ks, vs = 0.0625, 0.11
    what = f"fp8 chunked prefill D={D} {dtype} causal={causal}"
    _note(f"[case] {what} ctx={x['ctx_lens'].tolist()} n={x['new_lens'].tolist()}")
    o, lse = ta.attn_fwd_paged_fp8(_dev(x["q"], dtype), _u8(k8), _u8(v8), ks, vs, _i32(x["block_table"]),
                                   _i32(x["ctx_lens"]), _i32(x["new_lens"]), scale=case.scale, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = F8.prefill_paged_fp8(x["q"], k8, v8, ks, vs, x["block_table"], x["ctx_lens"], x["new_lens"],
                                          case.scale, causal)
    bound = BD.prefill_paged(x["q"], F8.dequantize(k8, ks), F8.dequantize(v8, vs), x["block_table"], x["ctx_lens"],
                             x["new_lens"], case.scale, causal, dtype)
    _compare(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, dtype, what=what, bound=bound)


def test_fp8_append_then_chunked_prefill_with_rope(ta):
    """The FP8 serving path for a prompt chunk: the chunk's K/V quantized into the cache, then the chunk's
    attention over the E4M3 cache with rotated queries."""
    import torch
    from oracle import rope as R
    case = W.ChunkCase("fp8 chunk+rope", B=3, Hq=12, Hkv=2, D=128, dtype="bf16", ctx_lo=0, ctx_hi=1200, chunk_lo=1,
                       chunk_hi=260, seed=96)
    x = W.chunk_inputs(case, nan_fill=True)
    rng = np.random.default_rng(97)
    k8 = W.e4m3_codes(rng, x["k_cache"].shape)
    v8 = W.e4m3_codes(rng, x["v_cache"].shape)
    ks, vs = 0.02, 0.03
    tab = W.rope_table(2048, case.D)
    kc, vc = _u8(k8), _u8(v8)
    ta.attn_cache_append_fp8(_dev(x["k_new"], "bf16"), _dev(x["v_new"], "bf16"), kc, vc, ks, vs,
                             _i32(x["block_table"]), _i32(x["start_pos"]), _i32(x["new_lens"]))
    o, lse = ta.attn_fwd_paged_fp8(_dev(x["q"], "bf16"), kc, vc, ks, vs, _i32(x["block_table"]), _i32(x["ctx_lens"]),
                                   _i32(x["new_lens"]), scale=case.scale, causal=True,
                                   rope=torch.from_numpy(tab).cuda())
    torch.cuda.synchronize()
    kref, vref = F8.cache_append_fp8(x["k_new"], x["v_new"], k8, v8, x["block_table"], x["start_pos"], ks, vs,
                                     x["new_lens"])
    assert np.array_equal(kc.cpu().numpy(), kref) and np.array_equal(vc.cpu().numpy(), vref)
    o_ref, lse_ref = R.prefill_paged_rope(x["q"], F8.dequantize(kref, ks), F8.dequantize(vref, vs),
                                          x["block_table"], x["ctx_lens"], x["new_lens"], tab, case.scale, "bf16")
    _compare(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "bf16", what="fp8 append + chunk + rope")


def test_fp8_chunked_prefill_long_prefix_sampled(ta):
    """A 20,000-token prefix over an E4M3 cache plus a 512-row chunk; oracle on sampled rows."""
    import torch
    case = W.ChunkCase("fp8 long", B=1, Hq=8, Hkv=2, D=128, dtype="bf16", ctx_lo=20000, ctx_hi=20000, chunk_lo=512,
                       chunk_hi=512, seed=98)
    x, k8, v8 = _fp8_chunk_inputs(case, 99)
    ks, vs = 0.125, 0.25
    o, lse = ta.attn_fwd_paged_fp8(_dev(x["q"], "bf16"), _u8(k8), _u8(v8), ks, vs, _i32(x["block_table"]),
                                   _i32(x["ctx_lens"]), _i32(x["new_lens"]), scale=case.scale, causal=True)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    from oracle import oracle as O
    L = int(x["ctx_lens"][0])
    kd, vd = F8.dequantize(k8, ks), F8.dequantize(v8, vs)
    K = np.stack([O.gather_paged(kd, vd, x["block_table"], L, 0, h)[0] for h in range(case.Hkv)])[None]
    V = np.stack([O.gather_paged(kd, vd, x["block_table"], L, 0, h)[1] for h in range(case.Hkv)])[None]
    rows = np.array([0, 1, 63, 64, 127, 128, 255, 256, 300, 511])
    picks = np.array([(0, hq, i) for hq in range(case.Hq) for i in rows])
    o_ref, lse_ref = O.prefill_rows(x["q"], K, V, case.scale, True, None, picks)
    bound = BD.prefill_rows(x["q"], K, V, case.scale, True, None, picks, "bf16")
    _compare(o[0][picks[:, 1], picks[:, 2]], lse[0][picks[:, 1], picks[:, 2]], o_ref, lse_ref, "bf16",
             what="fp8 long prefix sampled", bound=bound)
