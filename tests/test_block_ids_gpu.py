"""The block-id rule of the C ABI, on the GPU: an id outside [0, num_blocks) inside a sequence's context
marks an unmapped block, which the attention calls read as zero keys and values (and the appends never
write). Expected values come from the float64 oracle run on a copy of the cache with one extra, all-zero
physical block that those entries point to instead. Covered: the paged decode (16-bit and E4M3 caches)
and the chunked prefill (16-bit and E4M3 caches), with ids -1, -7, num_blocks and a large positive id.
"""
import numpy as np
import pytest

import workloads as W
from oracle import fp8 as F8
from oracle import oracle as O
from test_parity_gpu import _compare, _dev, _note

pytestmark = pytest.mark.gpu

BAD = (-1, -7, None, 1 << 30)  # None: num_blocks itself


@pytest.fixture(scope="module")
def ta(gpu):
    import torch  # noqa: F401
    import tiled_attention_02_amd as ta
    ta.lib()
    return ta


def _i32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def _unmap(table, ctx, NB, rng):
    """Replace some in-context entries by bad ids; return (gpu table, oracle table pointing at block NB)."""
    t_gpu = table.copy()
    t_ref = table.copy()
    nblk = (np.asarray(ctx) + 15) // 16
    for b in range(table.shape[0]):
        picks = rng.choice(int(nblk[b]), size=min(2, int(nblk[b])), replace=False)
        for n, i in enumerate(picks):
            bad = BAD[(b + n) % len(BAD)]
            t_gpu[b, i] = NB if bad is None else bad
            t_ref[b, i] = NB
    return t_gpu, t_ref


def _zero_block(cache):
    z = np.zeros((1,) + cache.shape[1:], dtype=cache.dtype)
    return np.concatenate([cache, z], axis=0)


@pytest.mark.parametrize("fp8", [False, True])
def test_decode_unmapped_blocks_read_as_zeros(ta, fp8):
    import torch
    case = W.DecodeCase("unmapped", B=6, Hq=12, Hkv=2, D=128, dtype="bf16", ctx_lo=20, ctx_hi=1500, seed=71)
    x = W.decode_inputs_fp8(case, nan_fill=True) if fp8 else W.decode_inputs(case, nan_fill=True)
    NB = x["k_cache"].shape[0]
    t_gpu, t_ref = _unmap(x["block_table"], x["ctx_lens"], NB, np.random.default_rng(72))
    _note(f"[case] decode unmapped ids fp8={fp8}")
    q = _dev(x["q"], "bf16")
    if fp8:
        kc = torch.from_numpy(x["k_cache"]).cuda()
        vc = torch.from_numpy(x["v_cache"]).cuda()
        o, lse = ta.attn_decode_paged_fp8(q, kc, vc, 0.5, 0.25, _i32(t_gpu), _i32(x["ctx_lens"]), scale=case.scale)
        o_ref, lse_ref = F8.decode_paged_fp8(x["q"], _zero_block(x["k_cache"]), _zero_block(x["v_cache"]), 0.5, 0.25,
                                             t_ref, x["ctx_lens"], case.scale)
    else:
        kc, vc = _dev(x["k_cache"], "bf16"), _dev(x["v_cache"], "bf16")
        o, lse = ta.attn_decode_paged(q, kc, vc, _i32(t_gpu), _i32(x["ctx_lens"]), scale=case.scale)
        o_ref, lse_ref = O.decode_paged(x["q"], _zero_block(x["k_cache"]), _zero_block(x["v_cache"]), t_ref,
                                        x["ctx_lens"], case.scale)
    torch.cuda.synchronize()
    _compare(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "bf16", what=f"decode unmapped fp8={fp8}")


@pytest.mark.parametrize("fp8", [False, True])
def test_chunked_prefill_unmapped_blocks_read_as_zeros(ta, fp8):
    import torch
    case = W.ChunkCase("unmapped-chunk", B=3, Hq=8, Hkv=2, D=128, dtype="bf16", ctx_lo=100, ctx_hi=700,
                       chunk_lo=30, chunk_hi=200, seed=73)
    x = W.chunk_inputs(case, nan_fill=False)
    NB = x["k_cache"].shape[0]
    # unmap only prefix blocks, never a block the chunk's own rows live in
    t_gpu = x["block_table"].copy()
    t_ref = x["block_table"].copy()
    rng = np.random.default_rng(74)
    for b in range(case.B):
        nfull = int(x["start_pos"][b]) // 16
        for n, i in enumerate(rng.choice(nfull, size=min(2, nfull), replace=False)):
            bad = BAD[(b + n) % len(BAD)]
            t_gpu[b, i] = NB if bad is None else bad
            t_ref[b, i] = NB
    ql = x["new_lens"]
    _note(f"[case] chunked prefill unmapped ids fp8={fp8}")
    q = _dev(x["q"], "bf16")
    if fp8:
        k8 = F8.quantize(x["k_cache"], 0.25)
        v8 = F8.quantize(x["v_cache"], 0.125)
        kc, vc = torch.from_numpy(k8).cuda(), torch.from_numpy(v8).cuda()
        o, lse = ta.attn_fwd_paged_fp8(q, kc, vc, 0.25, 0.125, _i32(t_gpu), _i32(x["ctx_lens"]), _i32(ql),
                                       scale=case.scale)
        o_ref, lse_ref = F8.prefill_paged_fp8(x["q"], _zero_block(k8), _zero_block(v8), 0.25, 0.125, t_ref,
                                              x["ctx_lens"], ql, case.scale, True)
    else:
        kc, vc = _dev(x["k_cache"], "bf16"), _dev(x["v_cache"], "bf16")
        o, lse = ta.attn_fwd_paged(q, kc, vc, _i32(t_gpu), _i32(x["ctx_lens"]), _i32(ql), scale=case.scale)
        o_ref, lse_ref = O.prefill_paged(x["q"], _zero_block(x["k_cache"]), _zero_block(x["v_cache"]), t_ref,
                                         x["ctx_lens"], ql, case.scale, True)
    torch.cuda.synchronize()
    _compare(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "bf16",
             what=f"chunked unmapped fp8={fp8}")
