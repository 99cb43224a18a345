"""Race check of the prefill's K/V staging: the pipelined kernel (libattn.so) against the same code built
with its debug key loop (libattn_single.so: one K and one V buffer, each tile loaded, waited for and
consumed before the next load, nothing overlapped). The pipelined kernel has two forms: double buffering
(K two tiles ahead, V one ahead, every load awaited at the end of its step) and, in the FP8 prefill, the
P.V product lagged by one tile over four-deep rings (K four tiles ahead of its scores, V three ahead of its
product, loads left in flight across barriers, waits counted per tile). Both forms run the same arithmetic in the same order
as the debug loop, so every output and lse must agree bit for bit; a wavefront that overwrote a buffer
another wavefront was still reading, or read one before its loads landed, would show as a difference.
Every prefill form is covered (contiguous causal / non-causal / ragged, Tq != Tk, chunked through the
block table over 16-bit, rotary and E4M3 caches, and the FP8 prefill), at sizes of one, two, three and
many key tiles (three is the first that reuses a double buffer, five the first that reuses a ring
buffer), and a grid larger than the chip.
"""
import numpy as np
import pytest

import workloads as W
from test_parity_gpu import _dev, _note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ta(gpu):
    import torch  # noqa: F401
    import tiled_attention_02_amd as ta
    ta.lib()
    return ta


def _i32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def _u8(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).cuda()


def _both(ta, call, what):
    """call() -> (o, lse) device tensors; run it on both libraries, then twice more on the pipelined one."""
    import torch
    outs = []
    for single in (False, True, False):
        if single:
            with ta.single_buffer_library():
                o, lse = call()
        else:
            o, lse = call()
        torch.cuda.synchronize()
        outs.append((o.clone(), lse.clone()))
    (o1, l1), (o2, l2), (o3, l3) = outs
    same = torch.equal(o1.view(torch.int16) if o1.dtype != torch.uint8 else o1,
                       o2.view(torch.int16) if o2.dtype != torch.uint8 else o2)
    lsame = torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    rep = torch.equal(o1, o3) and torch.equal(l1.view(torch.int32), l3.view(torch.int32))
    ndiff = int((o1.view(torch.int16) != o2.view(torch.int16)).sum().item())
    _note(f"[single-buffer] {what}: O bitwise equal={same} ({ndiff} elements differ) lse equal={lsame} "
          f"pipelined repeat equal={rep}")
    assert same and lsame, f"{what}: pipelined and single-buffer results differ"
    assert rep, f"{what}: the pipelined kernel is not deterministic"


@pytest.mark.parametrize("T", [60, 128, 190, 700])
@pytest.mark.parametrize("D,dtype,causal", [(128, "bf16", True), (64, "fp16", False), (128, "fp16", False),
                                            (64, "bf16", True)])
def test_contiguous(ta, T, D, dtype, causal):
    case = W.PrefillCase("sb", B=2, Hq=4, Hkv=2, T=T, D=D, dtype=dtype, causal=causal, ragged=False, seed=500 + T)
    x = W.prefill_inputs(case)
    q, k, v = (_dev(x[n], dtype) for n in ("q", "k", "v"))
    _both(ta, lambda: ta.attn_fwd(q, k, v, scale=case.scale, causal=causal),
          f"T={T} D={D} {dtype} causal={causal}")


def test_ragged_and_tq_ne_tk(ta):
    import torch
    case = W.BERT
    x = W.prefill_inputs(case, nan_padding=True)
    q, k, v = (_dev(x[n], case.dtype) for n in ("q", "k", "v"))
    sl = torch.from_numpy(x["seq_lens"]).cuda()
    _both(ta, lambda: ta.attn_fwd(q, k, v, scale=case.scale, seq_lens=sl), "BERT ragged fp16")
    c2 = W.PrefillCase("tq!=tk", B=2, Hq=8, Hkv=2, T=0, D=128, dtype="bf16", causal=True, ragged=False, seed=510)
    x = W.prefill_inputs(c2, Tq=300, Tk=900)
    q, k, v = (_dev(x[n], "bf16") for n in ("q", "k", "v"))
    _both(ta, lambda: ta.attn_fwd(q, k, v, scale=c2.scale, causal=True), "Tq=300 Tk=900 causal")


def test_long_causal(ta):
    case = W.PrefillCase("sb-long", B=1, Hq=8, Hkv=2, T=4096, D=128, dtype="bf16", causal=True, ragged=False,
                         seed=511)
    x = W.prefill_inputs(case)
    q, k, v = (_dev(x[n], "bf16") for n in ("q", "k", "v"))
    _both(ta, lambda: ta.attn_fwd(q, k, v, scale=case.scale, causal=True), "T=4096 causal bf16")


@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "fp16")])
def test_large_grid(ta, D, dtype):
    # B * Hq * ceil(T / 128) = 576 workgroups: more than the chip holds at once
    case = W.PrefillCase("sb-grid", B=2, Hq=32, Hkv=8, T=1100, D=D, dtype=dtype, causal=True, ragged=False,
                         seed=514)
    x = W.prefill_inputs(case)
    q, k, v = (_dev(x[n], dtype) for n in ("q", "k", "v"))
    _both(ta, lambda: ta.attn_fwd(q, k, v, scale=case.scale, causal=True), f"B=2 Hq=32 T=1100 D={D} causal")


# Grids of several workgroups per CU (workgroups that start in later rounds, reusing the CU's LDS):
# key tile counts of one to ten, ragged batches and Tq != Tk.
@pytest.mark.parametrize("T", [64, 200, 256, 320, 577])
@pytest.mark.parametrize("D,dtype,causal", [(128, "bf16", True), (64, "fp16", False), (128, "fp16", False),
                                            (64, "bf16", True)])
def test_many_workgroups(ta, T, D, dtype, causal):
    B, Hq = (8, 64) if T <= 256 else (4, 64)
    assert -(-T // 128) * Hq * B >= 512
    case = W.PrefillCase("sb-many", B=B, Hq=Hq, Hkv=8, T=T, D=D, dtype=dtype, causal=causal, ragged=False,
                         seed=520 + T)
    x = W.prefill_inputs(case)
    q, k, v = (_dev(x[n], dtype) for n in ("q", "k", "v"))
    _both(ta, lambda: ta.attn_fwd(q, k, v, scale=case.scale, causal=causal),
          f"many workgroups B={B} Hq={Hq} T={T} D={D} {dtype} causal={causal}")


def test_many_workgroups_ragged_and_tq_ne_tk(ta):
    import torch
    case = W.PrefillCase("sb-many-ragged", B=8, Hq=16, Hkv=4, T=600, D=128, dtype="bf16", causal=True, ragged=True,
                         seed=530)
    x = W.prefill_inputs(case, nan_padding=True)
    q, k, v = (_dev(x[n], "bf16") for n in ("q", "k", "v"))
    sl = torch.from_numpy(x["seq_lens"]).cuda()
    _both(ta, lambda: ta.attn_fwd(q, k, v, scale=case.scale, causal=True, seq_lens=sl),
          "many workgroups, ragged causal")
    c2 = W.PrefillCase("sb-many-tq", B=1, Hq=64, Hkv=16, T=0, D=64, dtype="fp16", causal=True, ragged=False, seed=531)
    x = W.prefill_inputs(c2, Tq=1000, Tk=1300)
    q, k, v = (_dev(x[n], "fp16") for n in ("q", "k", "v"))
    _both(ta, lambda: ta.attn_fwd(q, k, v, scale=c2.scale, causal=True), "many workgroups, Tq=1000 Tk=1300 causal")


@pytest.mark.parametrize("form", ["16-bit", "rotary", "E4M3"])
def test_chunked(ta, form):
    import torch
    case = W.ChunkCase("sb-chunk", B=3, Hq=8, Hkv=2, D=128, dtype="bf16", ctx_lo=0, ctx_hi=900, chunk_lo=1,
                       chunk_hi=300, seed=512)
    x = W.chunk_inputs(case, nan_fill=True)
    bt, cl, ql = _i32(x["block_table"]), _i32(x["ctx_lens"]), _i32(x["new_lens"])
    q = _dev(x["q"], "bf16")
    kn, vn = _dev(x["k_new"], "bf16"), _dev(x["v_new"], "bf16")
    sp = _i32(x["start_pos"])
    if form == "E4M3":
        kc = torch.zeros(x["k_cache"].shape, dtype=torch.uint8, device="cuda")
        vc = torch.zeros_like(kc)
        ta.attn_cache_append_fp8(kn, vn, kc, vc, 0.25, 0.125, bt, sp, ql)
        call = lambda: ta.attn_fwd_paged_fp8(q, kc, vc, 0.25, 0.125, bt, cl, ql, scale=case.scale)  # noqa: E731
    else:
        kc, vc = _dev(x["k_cache"], "bf16"), _dev(x["v_cache"], "bf16")
        rope = torch.from_numpy(W.rope_table(4096, 128)).cuda() if form == "rotary" else None
        ta.attn_cache_append(kn, vn, kc, vc, bt, sp, ql, rope=rope)
        call = lambda: ta.attn_fwd_paged(q, kc, vc, bt, cl, ql, scale=case.scale, rope=rope)  # noqa: E731
    torch.cuda.synchronize()
    _both(ta, call, f"chunked {form}")


@pytest.mark.parametrize("T,causal", [(64, True), (200, True), (320, False), (1000, False), (2048, True)])
def test_fp8_prefill(ta, T, causal):
    import torch
    case = W.PrefillCase("sb-fp8", B=1, Hq=8, Hkv=2, T=T, D=128, dtype="bf16", causal=causal, ragged=False,
                         seed=513)
    x = W.prefill_inputs_fp8(case)
    q, k, v = _u8(x["q"]), _u8(x["k"]), _u8(x["v"])
    _both(ta, lambda: ta.attn_fwd_fp8(q, k, v, 0.25, 0.25, 0.5, scale=case.scale, causal=causal,
                                      out_dtype=torch.bfloat16), f"fp8 prefill T={T} causal={causal}")
