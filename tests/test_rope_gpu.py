"""GPU parity of the rotary embedding fused into the paged path.

attn_cache_append_rope, attn_fwd_paged_rope and attn_decode_paged_rope are
called through the C ABI and compared with oracle/rope.py on the same seeded
inputs and the same cos/sin table (workloads.rope_table, an input):
  - the appended keys: the rotation is computed in fp32 on the GPU and
    rounded once to the 16-bit type, the oracle rounds the exact rotation;
    the two may differ by one unit in the last place where the fp32 result
    lies next to a rounding boundary, so the test requires every element
    within one ulp and at least 99.9 % of them identical; values and untouched
    slots must match exactly;
  - the attention with rotated queries: the library's tolerance (bf16 1e-2,
    fp16 2e-3 on O, 1e-4 relative on lse) against the oracle run on the
    oracle's own appended cache.
"""
import numpy as np
import pytest

import workloads as W
from oracle import oracle as O
from oracle import rope as R
from test_parity_gpu import _compare, _dev, _note

pytestmark = pytest.mark.gpu

MAX_POS = 4096


@pytest.fixture(scope="module")
def ta(gpu):
    import torch  # noqa: F401
    import tiled_attention_02_amd as ta
    ta.lib()
    return ta


def _i32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def _table(D):
    import torch
    t = W.rope_table(MAX_POS, D)
    return t, torch.from_numpy(t).cuda()


def _ulps(a, b, dtype):
    """|a - b| in units of the 16-bit type's spacing at b (b exact in that type)."""
    bits = 8 if dtype == "bf16" else 11
    _, e = np.frexp(np.where(b == 0, 1.0, b))
    return np.abs(a - b) / np.exp2(e.astype(np.float64) - bits)


def _append(ta, x, dtype, tab_d, use_lens=True):
    import torch
    kc = _dev(x["k_cache"], dtype)
    vc = _dev(x["v_cache"], dtype)
    ta.attn_cache_append(_dev(x["k_new"], dtype), _dev(x["v_new"], dtype), kc, vc, _i32(x["block_table"]),
                         _i32(x["start_pos"]), _i32(x["new_lens"]) if use_lens else None, rope=tab_d)
    torch.cuda.synchronize()
    return kc, vc


def _check_append(kc, vc, kref, vref, dtype, what):
    k = kc.float().cpu().numpy().astype(np.float64)
    v = vc.float().cpu().numpy().astype(np.float64)
    nan = np.isnan(kref)
    assert np.array_equal(np.isnan(k), nan)
    u = _ulps(k[~nan], kref[~nan], dtype)
    same = float((u == 0).mean())
    _note(f"[parity] {what}: rotated keys max {u.max():.2f} ulp, {100 * same:.4f} % identical")
    assert u.max() <= 1.0 and same >= 0.999
    assert np.array_equal(np.isnan(v), np.isnan(vref)) and np.array_equal(v[~np.isnan(v)], vref[~np.isnan(vref)])


@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "fp16"), (128, "fp16"), (64, "bf16")])
@pytest.mark.parametrize("causal", [True, False])
def test_rope_append_then_chunked_prefill(ta, D, dtype, causal):
    import torch
    case = W.ChunkCase("rope chunk", B=3, Hq=8, Hkv=2, D=D, dtype=dtype, ctx_lo=0, ctx_hi=1500, chunk_lo=1,
                       chunk_hi=300, seed=91)
    x = W.chunk_inputs(case, nan_fill=True)
    tab, tab_d = _table(D)
    what = f"rope chunk D={D} {dtype} causal={causal}"
    _note(f"[case] {what} start={x['start_pos'].tolist()} n={x['new_lens'].tolist()}")
    kc, vc = _append(ta, x, dtype, tab_d)
    kref, vref = R.cache_append_rope(x["k_new"], x["v_new"], x["k_cache"], x["v_cache"], x["block_table"],
                                     x["start_pos"], tab, dtype, x["new_lens"])
    _check_append(kc, vc, kref, vref, dtype, what)
    o, lse = ta.attn_fwd_paged(_dev(x["q"], dtype), kc, vc, _i32(x["block_table"]), _i32(x["ctx_lens"]),
                               _i32(x["new_lens"]), scale=case.scale, causal=causal, rope=tab_d)
    torch.cuda.synchronize()
    o_ref, lse_ref = R.prefill_paged_rope(x["q"], kref, vref, x["block_table"], x["ctx_lens"], x["new_lens"], tab,
                                          case.scale, dtype, causal)
    _compare(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, dtype, what=what)


@pytest.mark.parametrize("Hq,Hkv,D,dtype", [(12, 2, 128, "bf16"), (8, 8, 64, "fp16"), (16, 1, 128, "fp16")])
def test_rope_decode_step(ta, Hq, Hkv, D, dtype):
    """A decode step with rotary embedding: the new token's K rotated into the cache, then the decode."""
    import torch
    case = W.ChunkCase("rope step", B=8, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, ctx_lo=0, ctx_hi=3000, chunk_lo=1,
                       chunk_hi=1, seed=92)
    x = W.chunk_inputs(case, nan_fill=True)
    tab, tab_d = _table(D)
    what = f"rope decode Hq={Hq} Hkv={Hkv} D={D} {dtype}"
    kc, vc = _append(ta, x, dtype, tab_d, use_lens=False)
    kref, vref = R.cache_append_rope(x["k_new"], x["v_new"], x["k_cache"], x["v_cache"], x["block_table"],
                                     x["start_pos"], tab, dtype)
    _check_append(kc, vc, kref, vref, dtype, what)
    o, lse = ta.attn_decode_paged(_dev(x["q"][:, :, 0], dtype), kc, vc, _i32(x["block_table"]), _i32(x["ctx_lens"]),
                                  scale=case.scale, rope=tab_d)
    torch.cuda.synchronize()
    o_ref, lse_ref = R.decode_paged_rope(x["q"][:, :, 0], kref, vref, x["block_table"], x["ctx_lens"], tab,
                                         case.scale, dtype)
    _compare(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, dtype, what=what)


def test_rope_prompt_in_chunks_equals_rotated_prefill(ta):
    """A prompt processed as three chunks with rotary embedding equals, row for row, the causal prefill of
    the whole prompt over rotated queries and keys (oracle)."""
    import torch
    T, Hq, Hkv, D = 900, 4, 2, 128
    full = W.PrefillCase("rope prompt", B=1, Hq=Hq, Hkv=Hkv, T=T, D=D, dtype="bf16", causal=True, ragged=False,
                         seed=93)
    x = W.prefill_inputs(full)
    tab, tab_d = _table(D)
    qr = R.round16(R.rope_rows(x["q"], [0], tab), "bf16")
    kr = R.round16(R.rope_rows(x["k"], [0], tab), "bf16")
    o_ref, lse_ref = O.prefill(qr, kr, x["v"], full.scale, True, None)
    nb = (T + 15) // 16
    table = np.random.default_rng(93).permutation(nb + 3)[:nb].astype(np.int32)[None]
    kc = torch.zeros((nb + 3, Hkv, 16, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    bt = _i32(table)
    for s, e in ((0, 333), (333, 334), (334, T)):
        ta.attn_cache_append(_dev(x["k"][:, :, s:e], "bf16"), _dev(x["v"][:, :, s:e], "bf16"), kc, vc, bt,
                             _i32([s]), None, rope=tab_d)
        o, lse = ta.attn_fwd_paged(_dev(x["q"][:, :, s:e], "bf16"), kc, vc, bt, _i32([e]), None, scale=full.scale,
                                   causal=True, rope=tab_d)
        torch.cuda.synchronize()
        _compare(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref[:, :, s:e], lse_ref[:, :, s:e], "bf16",
                 what=f"rope prompt chunk [{s},{e})")


def test_rope_rejects_bad_tables(ta):
    import torch
    q = torch.zeros((2, 4, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((4, 2, 16, 128), dtype=torch.bfloat16, device="cuda")
    bt, cl = _i32(np.zeros((2, 2))), _i32([1, 1])
    with pytest.raises(ValueError, match="rope must be"):
        ta.attn_decode_paged(q, kc, kc, bt, cl, rope=torch.zeros((16, 64), dtype=torch.float32, device="cuda"))
    L = ta.lib()
    import ctypes
    st = L.attn_decode_paged_rope(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kc.data_ptr()),
                                  ctypes.c_void_p(kc.data_ptr()), None, 16, ctypes.c_void_p(bt.data_ptr()),
                                  ctypes.c_void_p(cl.data_ptr()), ctypes.c_void_p(q.data_ptr()), None, 2, 4, 2, 128,
                                  16, 2, 4, ctypes.c_float(0.1), 1, None, 0, None)
    assert st == 1 and "rotary table" in ta.attn_last_error()
