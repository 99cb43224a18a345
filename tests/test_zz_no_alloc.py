"""The decode entry point that allocates nothing (attn_decode_paged_noalloc) against attn_decode_paged.

Both are called through the C ABI (ctypes, raw pointers and sizes) on the same inputs. The no-allocation
call keeps its split partials in the library's static per-GPU scratch array; its kernels are the ones
attn_decode_paged launches with a caller's workspace, so O and lse must agree bit for bit, and both must
match the float64 oracle to the stated bounds. Two calls in a row, the second on a smaller batch (fewer
sequences, shorter contexts, another head layout) so that it runs over what the first left in the
scratch; a third call repeats the first and must reproduce it exactly. Every output buffer is allocated
before the calls (the no-allocation call itself allocates nothing).
"""
import ctypes

import numpy as np
import pytest

import workloads as W
from oracle import oracle as O
from test_parity_gpu import _compare, _dev, _note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta(gpu):
    import torch  # noqa: F401
    import tiled_attention_02_amd as ta
    ta.lib()
    return ta


def _inputs(case, ctx=None):
    import torch
    x = W.decode_inputs(case, nan_fill=True, ctx_lens=ctx)
    d = dict(q=_dev(x["q"], case.dtype), kc=_dev(x["k_cache"], case.dtype), vc=_dev(x["v_cache"], case.dtype),
             bt=torch.from_numpy(x["block_table"]).cuda(), cl=torch.from_numpy(x["ctx_lens"]).cuda())
    return x, d


def _raw_noalloc(ta, d, case, o, lse):
    """attn_decode_paged_noalloc through the C ABI with raw pointers."""
    import torch
    L = ta.lib()
    B, Hq, D = d["q"].shape
    NB, Hkv = d["kc"].shape[:2]
    dt = 1 if case.dtype == "bf16" else 0
    st = L.attn_decode_paged_noalloc(
        ctypes.c_void_p(d["q"].data_ptr()), ctypes.c_void_p(d["kc"].data_ptr()), ctypes.c_void_p(d["vc"].data_ptr()),
        ctypes.c_void_p(d["bt"].data_ptr()), ctypes.c_void_p(d["cl"].data_ptr()), ctypes.c_void_p(o.data_ptr()),
        ctypes.c_void_p(lse.data_ptr()), B, Hq, Hkv, D, 16, d["bt"].shape[1], NB, ctypes.c_float(case.scale), dt,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, ta.attn_last_error()


def test_noalloc_decode_equals_workspace_decode(ta):
    import torch
    big = W.DecodeCase("noalloc big", B=64, Hq=12, Hkv=2, D=128, dtype="bf16", ctx_lo=512, ctx_hi=4096, seed=301)
    small = W.DecodeCase("noalloc small", B=5, Hq=8, Hkv=4, D=64, dtype="fp16", ctx_lo=1, ctx_hi=700, seed=302)
    cases = [(big, None), (small, [1, 17, 300, 699, 256])]
    prepared = []
    for case, ctx in cases:
        x, d = _inputs(case, ctx)
        o_na = torch.empty_like(d["q"])
        l_na = torch.empty(d["q"].shape[:2], dtype=torch.float32, device="cuda")
        o_ws = torch.empty_like(d["q"])
        l_ws = torch.empty_like(l_na)
        prepared.append((case, x, d, o_na, l_na, o_ws, l_ws))
    torch.cuda.synchronize()
    for case, x, d, o_na, l_na, o_ws, l_ws in prepared:
        _note(f"[case] no-allocation decode {case.name} B={case.B} Hq={case.Hq} Hkv={case.Hkv} D={case.D} "
              f"maxb={d['bt'].shape[1]}")
        _raw_noalloc(ta, d, case, o_na, l_na)
        torch.cuda.synchronize()
        ta.attn_decode_paged(d["q"], d["kc"], d["vc"], d["bt"], d["cl"], scale=case.scale, out=o_ws, lse=l_ws)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ws) and torch.equal(l_na.view(torch.int32), l_ws.view(torch.int32)), \
            f"{case.name}: the no-allocation call differs from attn_decode_paged"
        o_ref, lse_ref = O.decode_paged(x["q"], x["k_cache"], x["v_cache"], x["block_table"], x["ctx_lens"],
                                        case.scale)
        _compare(o_na.float().cpu().numpy(), l_na.cpu().numpy(), o_ref, lse_ref, case.dtype,
                 what=f"no-allocation decode {case.name}", strict=True)
    # the first batch again, after the smaller one has overwritten part of the scratch
    case, x, d, o_na, l_na, o_ws, l_ws = prepared[0]
    o2 = torch.empty_like(o_na)
    l2 = torch.empty_like(l_na)
    _raw_noalloc(ta, d, case, o2, l2)
    torch.cuda.synchronize()
    assert torch.equal(o2, o_ws) and torch.equal(l2.view(torch.int32), l_ws.view(torch.int32))


def test_noalloc_decode_refuses_partials_beyond_the_scratch(ta):
    import torch
    case = W.DecodeCase("too big", B=2, Hq=12, Hkv=2, D=128, dtype="bf16", ctx_lo=1, ctx_hi=100, seed=303)
    x, d = _inputs(case)
    bt = torch.full((4096, 256), -1, dtype=torch.int32, device="cuda")
    cl = torch.ones(4096, dtype=torch.int32, device="cuda")
    q = torch.zeros((4096, 64, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    L = ta.lib()
    st = L.attn_decode_paged_noalloc(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(d["kc"].data_ptr()),
                                     ctypes.c_void_p(d["vc"].data_ptr()), ctypes.c_void_p(bt.data_ptr()),
                                     ctypes.c_void_p(cl.data_ptr()), ctypes.c_void_p(o.data_ptr()), None, 4096, 64, 8,
                                     128, 16, 256, d["kc"].shape[0], ctypes.c_float(0.1), 1, None)
    assert st == 2 and "scratch" in ta.attn_last_error()
