"""Paged caches larger than 4 GiB (through the C ABI, against the float64 oracle).

A serving process sizes its caches to the device's memory, so physical blocks sit at byte offsets far
past 2^32. Here each cache holds 600,000 blocks of 16 tokens x 2 kv heads x 128 dims in bf16 (4.9 GB;
1,100,000 blocks, 4.5 GB, for the E4M3 form), and every block a sequence uses lies past byte 2^32 of
its cache (the last block of the cache included). The oracle works on compact caches that hold only
those blocks, with the block table renumbered; the GPU copies them to their high physical ids. Covered:
decode (16-bit and E4M3), append into the high blocks (16-bit and E4M3) and the chunked prefill over
them. The rest of each large cache is never written nor read. A last case runs the contiguous prefill
on K and V tensors of 2.3 GB each (rows past byte 2^31).
"""
import numpy as np
import pytest

import workloads as W
from oracle import bounds as BD
from oracle import fp8 as F8
from oracle import oracle as O
from test_parity_gpu import _compare, _dev, _note

pytestmark = pytest.mark.gpu

NB16 = 600_000     # blocks of a 16-bit cache: 8 KiB each (Hkv 2, D 128)
NB8 = 1_100_000    # blocks of an E4M3 cache: 4 KiB each


@pytest.fixture(scope="module")
def ta(gpu):
    import torch  # noqa: F401
    import tiled_attention_02_amd as ta
    ta.lib()
    return ta


def _i32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def _high_ids(n, nb, block_bytes, seed):
    """n distinct physical ids, all past byte 2^32 of the cache, the cache's last block among them."""
    lo = (1 << 32) // block_bytes + 1
    rng = np.random.default_rng(seed)
    ids = rng.choice(np.arange(lo, nb - 1), n - 1, replace=False)
    ids = np.concatenate([[nb - 1], ids]).astype(np.int64)
    rng.shuffle(ids)
    assert ids.min() * block_bytes >= (1 << 32) and ids.max() == nb - 1
    return ids


def _big(small, ids, nb, tdtype):
    """A cache of nb blocks (uninitialised) holding small's blocks at physical ids `ids`."""
    import torch
    big = torch.empty((nb,) + tuple(small.shape[1:]), dtype=tdtype, device="cuda")
    big.index_copy_(0, torch.from_numpy(ids).cuda(), small)
    return big


def _renumber(table, ids):
    return np.where(table >= 0, ids[np.maximum(table, 0)], -1).astype(np.int32)


def _free():
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_decode_over_caches_past_4_gib(ta):
    import torch
    case = W.DecodeCase("large cache", B=3, Hq=8, Hkv=2, D=128, dtype="bf16", ctx_lo=1, ctx_hi=1500, seed=91)
    x = W.decode_inputs(case, nan_fill=True, ctx_lens=[700, 1500, 33])
    ids = _high_ids(x["k_cache"].shape[0], NB16, 2 * 16 * 128 * 2, seed=92)
    _note(f"[case] decode, bf16 caches of {NB16} blocks, ids {ids.min()}..{ids.max()}")
    kc = _big(_dev(x["k_cache"], "bf16"), ids, NB16, torch.bfloat16)
    vc = _big(_dev(x["v_cache"], "bf16"), ids, NB16, torch.bfloat16)
    o, lse = ta.attn_decode_paged(_dev(x["q"], "bf16"), kc, vc, _i32(_renumber(x["block_table"], ids)),
                                  _i32(x["ctx_lens"]), scale=case.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = O.decode_paged(x["q"], x["k_cache"], x["v_cache"], x["block_table"], x["ctx_lens"], case.scale)
    bound = BD.decode_paged(x["q"], x["k_cache"], x["v_cache"], x["block_table"], x["ctx_lens"], case.scale, "bf16")
    _compare(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "bf16", what="decode past 4 GiB",
             bound=bound)
    del kc, vc
    _free()


def test_fp8_decode_over_caches_past_4_gib(ta):
    import torch
    case = W.DecodeCase("large fp8 cache", B=3, Hq=8, Hkv=2, D=128, dtype="bf16", ctx_lo=1, ctx_hi=1500, seed=93)
    x = W.decode_inputs_fp8(case, nan_fill=True, ctx_lens=[1200, 16, 817])
    ids = _high_ids(x["k_cache"].shape[0], NB8, 2 * 16 * 128, seed=94)
    _note(f"[case] decode, E4M3 caches of {NB8} blocks, ids {ids.min()}..{ids.max()}")
    ks, vs = 0.05, 0.03
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    kc = _big(u8(x["k_cache"]), ids, NB8, torch.uint8)
    vc = _big(u8(x["v_cache"]), ids, NB8, torch.uint8)
    o, lse = ta.attn_decode_paged_fp8(_dev(x["q"], "bf16"), kc, vc, ks, vs, _i32(_renumber(x["block_table"], ids)),
                                      _i32(x["ctx_lens"]), scale=case.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = F8.decode_paged_fp8(x["q"], x["k_cache"], x["v_cache"], ks, vs, x["block_table"],
                                         x["ctx_lens"], case.scale)
    bound = BD.decode_paged(x["q"], F8.dequantize(x["k_cache"], ks), F8.dequantize(x["v_cache"], vs),
                            x["block_table"], x["ctx_lens"], case.scale, "bf16")
    _compare(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "bf16", what="E4M3 decode past 4 GiB",
             bound=bound)
    del kc, vc
    _free()


def test_append_and_chunked_prefill_past_4_gib(ta):
    import torch
    case = W.ChunkCase("large cache chunk", B=2, Hq=8, Hkv=2, D=128, dtype="bf16", ctx_lo=0, ctx_hi=900,
                       chunk_lo=1, chunk_hi=130, seed=95)
    x = W.chunk_inputs(case, nan_fill=True, starts=[900, 37], lens=[130, 64])
    ids = _high_ids(x["k_cache"].shape[0], NB16, 2 * 16 * 128 * 2, seed=96)
    table = _i32(_renumber(x["block_table"], ids))
    start, lens, ctx = _i32(x["start_pos"]), _i32(x["new_lens"]), _i32(x["ctx_lens"])
    _note(f"[case] append + chunked prefill, bf16 caches of {NB16} blocks, ids {ids.min()}..{ids.max()}")
    kc = _big(_dev(x["k_cache"], "bf16"), ids, NB16, torch.bfloat16)
    vc = _big(_dev(x["v_cache"], "bf16"), ids, NB16, torch.bfloat16)
    ta.attn_cache_append(_dev(x["k_new"], "bf16"), _dev(x["v_new"], "bf16"), kc, vc, table, start, lens)
    o, lse = ta.attn_fwd_paged(_dev(x["q"], "bf16"), kc, vc, table, ctx, lens, scale=case.scale)
    torch.cuda.synchronize()
    kref, vref = O.cache_append(x["k_new"], x["v_new"], x["k_cache"], x["v_cache"], x["block_table"],
                                x["start_pos"], x["new_lens"])
    tid = torch.from_numpy(ids).cuda()
    for got, ref, n in ((kc, kref, "K"), (vc, vref, "V")):
        g = got.index_select(0, tid).float().cpu().numpy()
        assert np.array_equal(np.isnan(g), np.isnan(ref)), f"{n}: NaN slots moved"
        assert np.array_equal(g[~np.isnan(g)], ref[~np.isnan(ref)]), f"{n}: appended values differ"
    o_ref, lse_ref = O.prefill_paged(x["q"], kref, vref, x["block_table"], x["ctx_lens"], x["new_lens"],
                                     case.scale, True)
    bound = BD.prefill_paged(x["q"], kref, vref, x["block_table"], x["ctx_lens"], x["new_lens"], case.scale, True,
                             "bf16")
    _compare(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "bf16", what="chunked prefill past 4 GiB",
             bound=bound)
    # the E4M3 form of the append into blocks past byte 2^32 of a 4.5 GB cache
    del kc, vc
    _free()
    ids8 = _high_ids(x["k_cache"].shape[0], NB8, 2 * 16 * 128, seed=97)
    rng = np.random.default_rng(98)
    k8 = W.e4m3_codes(rng, x["k_cache"].shape)
    v8 = W.e4m3_codes(rng, x["v_cache"].shape)
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    kc8 = _big(u8(k8), ids8, NB8, torch.uint8)
    vc8 = _big(u8(v8), ids8, NB8, torch.uint8)
    table8 = _i32(_renumber(x["block_table"], ids8))
    ta.attn_cache_append_fp8(_dev(x["k_new"], "bf16"), _dev(x["v_new"], "bf16"), kc8, vc8, 0.05, 0.04, table8,
                             start, lens)
    o8, lse8 = ta.attn_fwd_paged_fp8(_dev(x["q"], "bf16"), kc8, vc8, 0.05, 0.04, table8, ctx, lens,
                                     scale=case.scale)
    torch.cuda.synchronize()
    k8_ref, v8_ref = F8.cache_append_fp8(x["k_new"], x["v_new"], k8, v8, x["block_table"], x["start_pos"], 0.05,
                                         0.04, x["new_lens"])
    t8 = torch.from_numpy(ids8).cuda()
    assert np.array_equal(kc8.index_select(0, t8).cpu().numpy(), k8_ref)
    assert np.array_equal(vc8.index_select(0, t8).cpu().numpy(), v8_ref)
    o_ref, lse_ref = F8.prefill_paged_fp8(x["q"], k8_ref, v8_ref, 0.05, 0.04, x["block_table"], x["ctx_lens"],
                                          x["new_lens"], case.scale, True)
    bound = BD.prefill_paged(x["q"], F8.dequantize(k8_ref, 0.05), F8.dequantize(v8_ref, 0.04), x["block_table"],
                             x["ctx_lens"], x["new_lens"], case.scale, True, "bf16")
    _compare(o8.float().cpu().numpy(), lse8.cpu().numpy(), o_ref, lse_ref, "bf16",
             what="chunked prefill over E4M3 caches past 4 GiB", bound=bound)
    del kc8, vc8
    _free()


def test_prefill_kv_past_2_gib(ta):
    """Contiguous K and V of 1.15e9 elements each (2.3 GB in bf16), so key rows sit past byte 2^31 of the
    tensor: 32 queries per head against 4.5M keys, non-causal. K/V repeat a random block of 1,000,003 rows
    (a prime period, so an offset that wrapped would read other rows) and the last 1000 keys of each head
    are drawn apart with three times the spread, so they dominate the softmax. Sampled rows against the
    oracle."""
    import torch
    Hq, Hkv, D, Tk, Tq, P = 4, 2, 128, 4_500_000, 32, 1_000_003
    assert Hkv * Tk * D < 2 ** 31 and Hkv * Tk * D * 2 > 2 ** 31
    rng = np.random.default_rng(99)
    q = W.round_to(rng.standard_normal((1, Hq, Tq, D), dtype=np.float32), "bf16")
    kv = []
    for _ in range(2):
        base = W.round_to(rng.standard_normal((Hkv, P, D), dtype=np.float32), "bf16")
        t = np.tile(base, (1, -(-Tk // P), 1))[:, :Tk]
        t[:, -1000:] = W.round_to(3.0 * rng.standard_normal((Hkv, 1000, D), dtype=np.float32), "bf16")
        kv.append(np.ascontiguousarray(t[None]))
        del base, t
    k, v = kv
    _note(f"[case] prefill with K/V of {k.size} elements each (Tk={Tk})")
    scale = 1.0 / np.sqrt(D)
    o, lse = ta.attn_fwd(_dev(q, "bf16"), _dev(k, "bf16"), _dev(v, "bf16"), scale=scale, causal=False)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    _free()
    picks = np.array([(0, h, i) for h in (0, 3) for i in (0, 17, 31)])
    o_ref, lse_ref = O.prefill_rows(q, k, v, scale, False, None, picks)
    og = o[picks[:, 0], picks[:, 1], picks[:, 2]]
    lg = lse[picks[:, 0], picks[:, 1], picks[:, 2]]
    _compare(og, lg, o_ref, lse_ref, "bf16", what="prefill with K/V past 2 GiB")
