"""GPU parity of the paged-cache append and the chunked prefill through the block table.

Both entry points are called through the C ABI (the ctypes binding) and
compared with the float64 CPU oracle on the same seeded inputs:
  - attn_cache_append must reproduce oracle.cache_append bit for bit (it is a
    copy), including the slots it must leave alone (NaN-filled);
  - attn_fwd_paged, run on the caches the GPU append wrote, must match
    oracle.prefill_paged to the accuracy target of the library (bf16 1e-2,
    fp16 2e-3 on O; 1e-4 relative on lse; padding rows exactly 0 / -inf).
Sizes span several 128-row query tiles and 64-key tiles with ragged tails,
prefixes that end mid-block, empty prefixes and empty chunks.
"""
import numpy as np
import pytest

import workloads as W
from oracle import bounds as BD
from oracle import oracle as O
from test_parity_gpu import TOL, LSE_REL, _compare, _dev, _note

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


def _append_gpu(ta, x, dtype, use_lens=True):
    """Run the GPU append on device copies of the inputs; returns the device caches."""
    import torch
    kc = _dev(x["k_cache"], dtype)
    vc = _dev(x["v_cache"], dtype)
    ta.attn_cache_append(_dev(x["k_new"], dtype), _dev(x["v_new"], dtype), kc, vc, _i32(x["block_table"]),
                         _i32(x["start_pos"]), _i32(x["new_lens"]) if use_lens else None)
    torch.cuda.synchronize()
    return kc, vc


def _same(gpu_t, ref):
    """Bitwise equality of a device tensor with dtype-rounded float32 values (NaN slots must stay NaN)."""
    g = gpu_t.float().cpu().numpy()
    return np.array_equal(np.isnan(g), np.isnan(ref)) and np.array_equal(g[~np.isnan(g)], ref[~np.isnan(ref)])


def _chunk_check(ta, case, causal=True, starts=None, lens=None, what=None, use_lens=True):
    import torch
    what = what or case.name
    x = W.chunk_inputs(case, nan_fill=True, starts=starts, lens=lens)
    _note(f"[case] {what} causal={causal} start={x['start_pos'].tolist()[:8]} n={x['new_lens'].tolist()[:8]} "
          f"Tq={x['q'].shape[2]} maxb={x['block_table'].shape[1]}")
    kc, vc = _append_gpu(ta, x, case.dtype, use_lens)
    kref, vref = O.cache_append(x["k_new"], x["v_new"], x["k_cache"], x["v_cache"], x["block_table"],
                                x["start_pos"], x["new_lens"] if use_lens else None)
    assert _same(kc, kref) and _same(vc, vref), f"{what}: append differs from the oracle"
    q_lens = x["new_lens"] if use_lens else None
    o, lse = ta.attn_fwd_paged(_dev(x["q"], case.dtype), kc, vc, _i32(x["block_table"]), _i32(x["ctx_lens"]),
                               _i32(q_lens) if q_lens is not None else None, scale=case.scale, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = O.prefill_paged(x["q"], kref, vref, x["block_table"], x["ctx_lens"], q_lens, case.scale,
                                     causal)
    bound = BD.prefill_paged(x["q"], kref, vref, x["block_table"], x["ctx_lens"], q_lens, case.scale, causal,
                             case.dtype)
    _compare(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, case.dtype, what=what, bound=bound)
    return x, kc, vc, o, lse


# ---------------------------------------------------------------- append + chunked prefill vs the oracle
@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "fp16"), (128, "fp16"), (64, "bf16")])
@pytest.mark.parametrize("causal", [True, False])
def test_chunk_append_then_prefill(ta, D, dtype, causal):
    """Prefixes 0..700 tokens (mid-block ends), chunks 1..300 rows (3 query tiles, ragged), GQA group 4."""
    case = W.ChunkCase("chunk", B=3, Hq=8, Hkv=2, D=D, dtype=dtype, ctx_lo=0, ctx_hi=700, chunk_lo=1,
                       chunk_hi=300, seed=61)
    _chunk_check(ta, case, causal=causal, what=f"chunk D={D} {dtype} causal={causal}")


@pytest.mark.parametrize("starts,lens", [([0, 0, 0], [1, 16, 17]),              # first chunk of a prompt
                                          ([15, 16, 17], [1, 1, 1]),             # one token across block edges
                                          ([31, 100, 250], [0, 130, 200]),        # an empty chunk
                                          ([1000, 64, 3], [64, 63, 65])])        # tile-sized chunks
def test_chunk_edges(ta, starts, lens):
    case = W.ChunkCase("edges", B=3, Hq=6, Hkv=3, D=128, dtype="bf16", ctx_lo=0, ctx_hi=1000, chunk_lo=1,
                       chunk_hi=max(lens) or 1, seed=62)
    _chunk_check(ta, case, starts=starts, lens=lens, what=f"chunk edges start={starts} n={lens}")


def test_chunk_widely_varied_prefixes(ta):
    """Prefixes from 0 to 3000 tokens and chunks from 0 to 400 rows in one batch: the workgroups take the
    (sequence, query tile) groups in decreasing work, so the order differs from launch order; every row
    still matches the oracle."""
    case = W.ChunkCase("varied", B=8, Hq=4, Hkv=2, D=128, dtype="bf16", ctx_lo=0, ctx_hi=3000, chunk_lo=0,
                       chunk_hi=400, seed=66)
    _chunk_check(ta, case, starts=[0, 3000, 17, 1500, 2999, 640, 0, 2222], lens=[400, 1, 0, 129, 256, 77, 5, 400],
                 what="chunk varied prefixes")


def test_chunk_batch_beyond_the_ordered_grid(ta):
    """70 sequences (more than the 64 whose groups are ordered by work): the launch-order path."""
    case = W.ChunkCase("many", B=70, Hq=4, Hkv=1, D=64, dtype="fp16", ctx_lo=0, ctx_hi=300, chunk_lo=1,
                       chunk_hi=40, seed=67)
    _chunk_check(ta, case, what="chunk B=70")


def test_chunk_all_rows_are_queries(ta):
    """q_lens NULL: every one of the Tq rows is a query (all chunks of equal length)."""
    case = W.ChunkCase("full", B=2, Hq=4, Hkv=1, D=64, dtype="fp16", ctx_lo=10, ctx_hi=400, chunk_lo=200,
                       chunk_hi=200, seed=63)
    _chunk_check(ta, case, use_lens=False, what="chunk q_lens=NULL")


def test_chunk_long_prefix_sampled(ta):
    """A 30,000-token prefix (a table of 1,919 blocks, near the limit of 2,048) plus a 700-row chunk;
    oracle on sampled rows of every head."""
    import torch
    case = W.ChunkCase("long", B=1, Hq=8, Hkv=2, D=128, dtype="bf16", ctx_lo=30000, ctx_hi=30000, chunk_lo=700,
                       chunk_hi=700, seed=64)
    x = W.chunk_inputs(case, nan_fill=True)
    _note(f"[case] long prefix start={x['start_pos'].tolist()} n={x['new_lens'].tolist()} "
          f"maxb={x['block_table'].shape[1]}")
    kc, vc = _append_gpu(ta, x, case.dtype)
    o, lse = ta.attn_fwd_paged(_dev(x["q"], case.dtype), kc, vc, _i32(x["block_table"]), _i32(x["ctx_lens"]),
                               _i32(x["new_lens"]), scale=case.scale, causal=True)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    kref, vref = O.cache_append(x["k_new"], x["v_new"], x["k_cache"], x["v_cache"], x["block_table"],
                                x["start_pos"], x["new_lens"])
    L = int(x["ctx_lens"][0])
    K = np.stack([O.gather_paged(kref, vref, x["block_table"], L, 0, h)[0] for h in range(case.Hkv)])[None]
    V = np.stack([O.gather_paged(kref, vref, x["block_table"], L, 0, h)[1] for h in range(case.Hkv)])[None]
    rows = np.array([0, 1, 63, 64, 127, 128, 255, 256, 511, 512, 640, 698, 699])
    picks = np.array([(0, h, i) for h in range(case.Hq) for i in rows])
    o_ref, lse_ref = O.prefill_rows(x["q"], K, V, case.scale, True, None, picks)
    _compare(o[0][picks[:, 1], picks[:, 2]], lse[0][picks[:, 1], picks[:, 2]], o_ref, lse_ref, "bf16",
             what="long prefix sampled")


# ---------------------------------------------------------------- cross-checks between entry points
def test_chunk_equals_contiguous_prefill(ta):
    """Reading K/V through the table changes nothing: the paged prefill of a chunk equals, bit for bit,
    the contiguous prefill (attn_fwd) of the same rows over the gathered keys/values."""
    import torch
    case = W.ChunkCase("vs-contig", B=3, Hq=8, Hkv=2, D=128, dtype="bf16", ctx_lo=50, ctx_hi=900, chunk_lo=1,
                       chunk_hi=260, seed=65)
    x, kc, vc, o, lse = _chunk_check(ta, case, what="chunk vs contiguous")
    kref = kc.float().cpu().numpy()
    vref = vc.float().cpu().numpy()
    for b in range(case.B):
        L, n = int(x["ctx_lens"][b]), int(x["new_lens"][b])
        K = np.stack([O.gather_paged(kref, vref, x["block_table"], L, b, h)[0] for h in range(case.Hkv)])[None]
        V = np.stack([O.gather_paged(kref, vref, x["block_table"], L, b, h)[1] for h in range(case.Hkv)])[None]
        qb = _dev(x["q"][b:b + 1, :, :n], case.dtype)
        oc, lc = ta.attn_fwd(qb, _dev(K, case.dtype), _dev(V, case.dtype), scale=case.scale, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(oc[0], o[b, :, :n]) and torch.equal(lc[0], lse[b, :, :n]), f"sequence {b}"


def test_single_row_chunk_matches_decode(ta):
    """A chunk of one token is a decode step: attn_fwd_paged and attn_decode_paged agree."""
    import torch
    case = W.ChunkCase("one", B=6, Hq=12, Hkv=2, D=128, dtype="bf16", ctx_lo=0, ctx_hi=3000, chunk_lo=1,
                       chunk_hi=1, seed=66)
    x, kc, vc, o, lse = _chunk_check(ta, case, what="single-row chunk")
    od, ld = ta.attn_decode_paged(_dev(x["q"][:, :, 0], case.dtype), kc, vc, _i32(x["block_table"]),
                                  _i32(x["ctx_lens"]), scale=case.scale)
    torch.cuda.synchronize()
    assert (od.float() - o[:, :, 0].float()).abs().max().item() <= 2 * TOL["bf16"]
    assert ((ld - lse[:, :, 0]).abs() / lse[:, :, 0].abs().clamp(min=1.0)).max().item() <= 2 * LSE_REL


def test_chunked_prompt_equals_one_shot_prefill(ta):
    """A prompt processed as three chunks (append, then prefill through the table) gives, row for row,
    the causal prefill of the whole prompt (oracle)."""
    import torch
    T, Hq, Hkv, D = 700, 4, 2, 128
    full = W.PrefillCase("prompt", B=1, Hq=Hq, Hkv=Hkv, T=T, D=D, dtype="bf16", causal=True, ragged=False,
                         seed=67)
    x = W.prefill_inputs(full)
    o_ref, lse_ref = O.prefill(x["q"], x["k"], x["v"], full.scale, True, None)
    nb = (T + 15) // 16
    table = np.random.default_rng(67).permutation(nb + 5)[:nb].astype(np.int32)[None]
    kc = torch.zeros((nb + 5, Hkv, 16, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    bt = _i32(table)
    for s, e in ((0, 200), (200, 201), (201, T)):
        n = e - s
        ta.attn_cache_append(_dev(x["k"][:, :, s:e], "bf16"), _dev(x["v"][:, :, s:e], "bf16"), kc, vc, bt,
                             _i32([s]), None)
        o, lse = ta.attn_fwd_paged(_dev(x["q"][:, :, s:e], "bf16"), kc, vc, bt, _i32([e]), None,
                                   scale=full.scale, causal=True)
        torch.cuda.synchronize()
        _note(f"[case] prompt chunk [{s},{e})")
        _compare(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref[:, :, s:e], lse_ref[:, :, s:e], "bf16",
                 what=f"prompt chunk [{s},{e}) of {n}")


def test_append_unmapped_and_out_of_table_tokens_are_skipped(ta):
    """Tokens whose block-table entry is -1, or whose position lies past the table, are not written."""
    import torch
    D, Hkv = 64, 2
    table = np.array([[3, -1], [1, 0]], dtype=np.int32)
    kc = torch.full((4, Hkv, 16, D), 7.0, dtype=torch.float16, device="cuda")
    vc = kc.clone()
    rng = np.random.default_rng(68)
    kn = W.round_to(rng.standard_normal((2, Hkv, 24, D), dtype=np.float32), "fp16")
    vn = W.round_to(rng.standard_normal((2, Hkv, 24, D), dtype=np.float32), "fp16")
    # sequence 0: positions 8..31 (block 1 unmapped); sequence 1: positions 20..43 (past the 2-block table)
    ta.attn_cache_append(_dev(kn, "fp16"), _dev(vn, "fp16"), kc, vc, _i32(table), _i32([8, 20]), None)
    torch.cuda.synchronize()
    k = kc.float().cpu().numpy()
    exp = np.full((4, Hkv, 16, D), 7.0, dtype=np.float32)
    exp[3, :, 8:16] = kn[0, :, 0:8]
    exp[0, :, 4:16] = kn[1, :, 0:12]
    assert np.array_equal(k, exp)
    del vn


# ---------------------------------------------------------------- host-side argument checks
def test_paged_prefill_rejects_bad_arguments(ta):
    import torch
    q = torch.zeros((1, 4, 8, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((4, 2, 16, 128), dtype=torch.bfloat16, device="cuda")
    ctx = _i32([8])
    with pytest.raises(ta.AttnError, match="max_blocks_per_seq"):
        ta.attn_fwd_paged(q, kc, kc, _i32(np.zeros((1, 2049))), ctx)
    with pytest.raises(ta.AttnError, match="head size"):
        q2 = torch.zeros((1, 4, 8, 96), dtype=torch.bfloat16, device="cuda")
        k2 = torch.zeros((4, 2, 16, 96), dtype=torch.bfloat16, device="cuda")
        ta.attn_fwd_paged(q2, k2, k2, _i32(np.zeros((1, 2))), ctx)
    with pytest.raises(ta.AttnError, match="multiple"):
        q3 = torch.zeros((1, 3, 8, 128), dtype=torch.bfloat16, device="cuda")
        ta.attn_fwd_paged(q3, kc, kc, _i32(np.zeros((1, 2))), ctx)
    with pytest.raises(ta.AttnError, match="block_size"):
        k4 = torch.zeros((4, 2, 8, 128), dtype=torch.bfloat16, device="cuda")
        ta.attn_fwd_paged(q, k4, k4, _i32(np.zeros((1, 2))), ctx)
