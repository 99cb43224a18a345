"""Every compute entry point captured into one HIP graph (through the C ABI).

One captured sequence: append a chunk into 16-bit caches, into rotary caches (K rotated) and into E4M3
caches; chunked prefill over each of them; paged decode over the 16-bit, E4M3 and rotary caches;
contiguous prefill in 16-bit and E4M3; the split-K linear product. The graph is replayed several times
with new inputs copied into its input buffers, with the same calls made eagerly on the default stream
in between; every replay must equal the eager results bit for bit (the kernels are deterministic and
the appends idempotent for equal inputs), and the last replay must match the float64 oracle to the
tolerances of the parity tests. The library allocates nothing and never synchronises, so the calls
are capturable as they stand; the decode workspace comes from the caller (allocated before capture).
"""
import numpy as np
import pytest

import workloads as W
from oracle import bounds as BD
from oracle import fp8 as F8
from oracle import gemm as G
from oracle import oracle as O
from oracle import rope as R
from test_parity_gpu import _compare, _dev, _note

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


KS, VS = 0.05, 0.04  # E4M3 cache scales


def _draw(rng, shape, dtype):
    return W.round_to(rng.standard_normal(shape, dtype=np.float32), dtype)


def test_graph_replays_every_entry_point(ta):
    import torch
    dt = "bf16"
    case = W.ChunkCase("graph chunk", B=3, Hq=8, Hkv=2, D=128, dtype=dt, ctx_lo=100, ctx_hi=900, chunk_lo=1,
                       chunk_hi=150, seed=81)
    x = W.chunk_inputs(case)
    B, Hq, Hkv, D = case.B, case.Hq, case.Hkv, case.D
    bt, start, lens, ctx = (_i32(x[n]) for n in ("block_table", "start_pos", "new_lens", "ctx_lens"))
    tab_np = W.rope_table(int(x["ctx_lens"].max()) + 1, D)
    tab = torch.from_numpy(tab_np).cuda()
    rng = np.random.default_rng(82)
    k8_np = W.e4m3_codes(rng, x["k_cache"].shape)
    v8_np = W.e4m3_codes(rng, x["v_cache"].shape)
    caches = dict(kc=_dev(x["k_cache"], dt), vc=_dev(x["v_cache"], dt), kr=_dev(x["k_cache"], dt),
                  vr=_dev(x["v_cache"], dt), k8=_u8(k8_np), v8=_u8(v8_np))
    pcase = W.PrefillCase("graph prefill", B=2, Hq=8, Hkv=2, T=200, D=128, dtype=dt, causal=True, ragged=True,
                          seed=83)
    p = W.prefill_inputs(pcase)
    p8 = W.prefill_inputs_fp8(W.PrefillCase("graph fp8", B=1, Hq=4, Hkv=1, T=300, D=128, dtype=dt, causal=True,
                                            ragged=False, seed=84))
    M, N, K = 2, 320, 1032
    g_in = W.gemm_inputs(M, N, K, dt, seed=85)
    # input buffers the graph reads (refilled before each replay)
    inp = dict(q=_dev(x["q"], dt), kn=_dev(x["k_new"], dt), vn=_dev(x["v_new"], dt), qd=_dev(x["q"][:, :, 0], dt),
               pq=_dev(p["q"], dt), pk=_dev(p["k"], dt), pv=_dev(p["v"], dt), sl=_i32(p["seq_lens"]),
               q8=_u8(p8["q"]), k8p=_u8(p8["k"]), v8p=_u8(p8["v"]), gx=_dev(g_in["x"], dt), gw=_dev(g_in["w"], dt))
    ws = ta.decode_workspace(inp["q"].device, ta.attn_decode_workspace_bytes(B, Hq, Hkv, D, x["block_table"].shape[1]))

    def step():
        c = caches
        out = {}
        ta.attn_cache_append(inp["kn"], inp["vn"], c["kc"], c["vc"], bt, start, lens)
        ta.attn_cache_append(inp["kn"], inp["vn"], c["kr"], c["vr"], bt, start, lens, rope=tab)
        ta.attn_cache_append_fp8(inp["kn"], inp["vn"], c["k8"], c["v8"], KS, VS, bt, start, lens)
        out["chunk"] = ta.attn_fwd_paged(inp["q"], c["kc"], c["vc"], bt, ctx, lens)
        out["chunk_rope"] = ta.attn_fwd_paged(inp["q"], c["kr"], c["vr"], bt, ctx, lens, rope=tab)
        out["chunk_fp8"] = ta.attn_fwd_paged_fp8(inp["q"], c["k8"], c["v8"], KS, VS, bt, ctx, lens)
        out["decode"] = ta.attn_decode_paged(inp["qd"], c["kc"], c["vc"], bt, ctx, workspace=ws)
        out["decode_fp8"] = ta.attn_decode_paged_fp8(inp["qd"], c["k8"], c["v8"], KS, VS, bt, ctx, workspace=ws)
        out["decode_rope"] = ta.attn_decode_paged(inp["qd"], c["kr"], c["vr"], bt, ctx, workspace=ws, rope=tab)
        out["prefill"] = ta.attn_fwd(inp["pq"], inp["pk"], inp["pv"], causal=True, seq_lens=inp["sl"])
        out["prefill_fp8"] = ta.attn_fwd_fp8(inp["q8"], inp["k8p"], inp["v8p"], 0.5, 0.25, 0.5, causal=True)
        out["gemm"] = (ta.attn_gemm_splitk(inp["gx"], inp["gw"]),)
        return out

    step()  # warm-up outside the capture (library load, kernel attributes)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        captured = step()
    torch.cuda.synchronize()

    for rep in range(3):
        new = dict(q=_draw(rng, x["q"].shape, dt), kn=_draw(rng, x["k_new"].shape, dt),
                   vn=_draw(rng, x["v_new"].shape, dt), qd=_draw(rng, (B, Hq, D), dt),
                   pq=_draw(rng, p["q"].shape, dt), gx=_draw(rng, (M, K), dt))
        new["q8"] = W.e4m3_codes(rng, p8["q"].shape)
        for n in ("q", "kn", "vn", "qd", "pq", "gx"):
            inp[n].copy_(_dev(new[n], dt))
        inp["q8"].copy_(_u8(new["q8"]))
        torch.cuda.synchronize()
        _note(f"[case] graph replay {rep} of every entry point")
        g.replay()
        torch.cuda.synchronize()
        got = {k: tuple(t.clone() for t in v if t is not None) for k, v in captured.items()}
        eager = step()
        torch.cuda.synchronize()
        for k, v in eager.items():
            ref = tuple(t for t in v if t is not None)
            assert len(ref) == len(got[k]) and all(torch.equal(a, b) for a, b in zip(got[k], ref)), \
                f"replay {rep}: {k} differs from the eager call"

    # the last replay against the oracle
    kref, vref = O.cache_append(new["kn"], new["vn"], x["k_cache"], x["v_cache"], x["block_table"], x["start_pos"],
                                x["new_lens"])
    o, lse = got["chunk"]
    o_ref, lse_ref = O.prefill_paged(new["q"], kref, vref, x["block_table"], x["ctx_lens"], x["new_lens"],
                                     1.0 / np.sqrt(D), True)
    bound = BD.prefill_paged(new["q"], kref, vref, x["block_table"], x["ctx_lens"], x["new_lens"], 1.0 / np.sqrt(D),
                             True, dt)
    _compare(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, dt, what="graph: chunked prefill",
             bound=bound)
    o, lse = got["decode"]
    o_ref, lse_ref = O.decode_paged(new["qd"], kref, vref, x["block_table"], x["ctx_lens"], 1.0 / np.sqrt(D))
    bound = BD.decode_paged(new["qd"], kref, vref, x["block_table"], x["ctx_lens"], 1.0 / np.sqrt(D), dt)
    _compare(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, dt, what="graph: decode", bound=bound)
    o, lse = got["prefill"]
    o_ref, lse_ref = O.prefill(new["pq"], p["k"], p["v"], 1.0 / np.sqrt(D), True, p["seq_lens"])
    bound = BD.prefill(new["pq"], p["k"], p["v"], 1.0 / np.sqrt(D), True, p["seq_lens"], dt)
    _compare(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, dt, what="graph: prefill", bound=bound)
    y = got["gemm"][0].float().cpu().numpy()
    assert (np.abs(y - G.linear(new["gx"], g_in["w"])) <= G.error_bound(new["gx"], g_in["w"], dt)).all()
    # E4M3 caches: the appended codes are the oracle's
    k8_ref, v8_ref = F8.cache_append_fp8(new["kn"], new["vn"], k8_np, v8_np, x["block_table"], x["start_pos"], KS,
                                         VS, x["new_lens"])
    assert np.array_equal(caches["k8"].cpu().numpy(), k8_ref) and np.array_equal(caches["v8"].cpu().numpy(), v8_ref)
    # rotary caches: K rows rotated at their positions, at most one unit of bf16 from the oracle's rounding
    kr_ref = R.cache_append_rope(new["kn"], new["vn"], x["k_cache"], x["v_cache"], x["block_table"], x["start_pos"],
                                 tab_np, dt, x["new_lens"])[0]
    kr = caches["kr"].float().cpu().numpy().astype(np.float64)
    _, e = np.frexp(np.where(kr_ref == 0, 1.0, kr_ref))
    assert (np.abs(kr - kr_ref) <= np.exp2(e.astype(np.float64) - 8)).all()
