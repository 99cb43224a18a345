"""GPU parity of the FP8 prefill (attn_fwd_fp8: E4M3 q, k, v; both products on the fp8 matrix cores).

Reference: the float64 prefill definition on the dequantized inputs (oracle/fp8.py). The kernel rounds
the probabilities to E4M3 for the P.V product, so the tolerance is the bound that rounding allows (derived
in oracle/fp8.prefill_fp8_bound): per output element |dO| <= (2^-4 + L * 2^-17) * max |v| of the kv
head, plus one unit in the last place of the output type; lse (computed from the unrounded
probabilities and the fp32 scores) within 1e-4 * max(1, |lse|); padded rows exactly 0 / -inf. The mean
error, far below the bound, is printed for each case.
"""
import numpy as np
import pytest

import workloads as W
from oracle import fp8 as F8
from oracle import oracle as O
from test_parity_gpu import LSE_REL, _note, _ulp

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


def _run(ta, x, scales, scale, causal, out_dtype):
    import torch
    od = torch.bfloat16 if out_dtype == "bf16" else torch.float16
    sl = None if x["seq_lens"] is None else torch.from_numpy(x["seq_lens"]).cuda()
    o, lse = ta.attn_fwd_fp8(_u8(x["q"]), _u8(x["k"]), _u8(x["v"]), *scales, scale=scale, causal=causal,
                             seq_lens=sl, out_dtype=od)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def _check(o, lse, o_ref, lse_ref, bound_bh, G, out_dtype, what, rows=None):
    """bound_bh [B, Hkv]; o/o_ref [B, Hq, T, D] (or picked rows with `rows` = (b, hq) arrays)."""
    if rows is None:
        B, Hq = o_ref.shape[:2]
        bnd = np.repeat(bound_bh, G, axis=1)[:, :, None, None]
        valid = np.isfinite(lse_ref)
        ov = np.broadcast_to(valid[..., None], o_ref.shape)
        bnd = np.broadcast_to(bnd, o_ref.shape)
    else:
        b, hq = rows
        bnd = bound_bh[b, hq // G][:, None] * np.ones_like(o_ref)
        valid = np.isfinite(lse_ref)
        ov = np.broadcast_to(valid[:, None], o_ref.shape)
    err = np.abs(o - o_ref)
    allow = bnd + _ulp(o_ref, out_dtype)
    ratio = float((err[ov] / allow[ov]).max()) if ov.any() else 0.0
    lerr = float((np.abs(lse[valid] - lse_ref[valid]) / np.maximum(1.0, np.abs(lse_ref[valid]))).max())
    _note(f"[parity] {what}: max|dO|={err[ov].max():.3e} mean|dO|={err[ov].mean():.3e} "
          f"(bound {bnd[ov].max():.3e}) max err/bound={ratio:.3f} max rel dlse={lerr:.3e}")
    assert np.isfinite(o[ov]).all()
    assert ratio <= 1.0
    assert lerr <= LSE_REL
    inv = ~valid
    if inv.any():
        oi = np.broadcast_to(inv[..., None], o_ref.shape)
        assert np.all(o[oi] == 0.0) and np.all(np.isneginf(lse[inv]))


def _case_check(ta, case, scales=(0.25, 0.25, 0.5), scale=None, Tq=None, Tk=None, causal=None, out="bf16",
                what=None):
    x = W.prefill_inputs_fp8(case, Tq=Tq, Tk=Tk)
    scale = case.scale if scale is None else scale
    causal = case.causal if causal is None else causal
    what = what or case.name
    _note(f"[case] fp8 prefill {what} causal={causal} scales={scales} q{x['q'].shape} k{x['k'].shape}")
    o, lse = _run(ta, x, scales, scale, causal, out)
    o_ref, lse_ref = F8.prefill_fp8(x["q"], x["k"], x["v"], *scales, scale, causal, x["seq_lens"])
    bound = F8.prefill_fp8_bound(x["v"], scales[2], x["k"].shape[2])
    _check(o, lse, o_ref, lse_ref, bound, case.Hq // case.Hkv, out, what)


def test_fp8_prefill_llama_causal_gqa(ta):
    case = W.PrefillCase("fp8 llama", B=2, Hq=8, Hkv=2, T=700, D=128, dtype="bf16", causal=True, ragged=False,
                         seed=101)
    _case_check(ta, case)


def test_fp8_prefill_bert_ragged_fp16_out(ta):
    case = W.PrefillCase("fp8 bert", B=4, Hq=6, Hkv=6, T=333, D=64, dtype="fp16", causal=False, ragged=True,
                         seed=102)
    _case_check(ta, case, scales=(0.5, 0.125, 0.25), out="fp16")


@pytest.mark.parametrize("Tq,Tk", [(77, 301), (300, 45), (1, 200), (129, 129)])
def test_fp8_prefill_tq_ne_tk(ta, Tq, Tk):
    case = W.PrefillCase("fp8 tq!=tk", B=2, Hq=4, Hkv=1, T=0, D=128, dtype="bf16", causal=True, ragged=False,
                         seed=103)
    _case_check(ta, case, Tq=Tq, Tk=Tk, what=f"Tq={Tq} Tk={Tk} causal")
    _case_check(ta, case, Tq=Tq, Tk=Tk, causal=False, what=f"Tq={Tq} Tk={Tk} non-causal")


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.5])
def test_fp8_prefill_scale_values(ta, scale):
    case = W.PrefillCase("fp8 scale", B=1, Hq=2, Hkv=2, T=200, D=64, dtype="bf16", causal=True, ragged=False,
                         seed=104)
    _case_check(ta, case, scale=scale, what=f"scale={scale}")


def test_fp8_prefill_peaked_scores(ta):
    """Large q/k scales: scores spread over tens of log2 units, the running max moves often."""
    case = W.PrefillCase("fp8 peaked", B=1, Hq=4, Hkv=1, T=600, D=128, dtype="bf16", causal=True, ragged=False,
                         seed=105)
    _case_check(ta, case, scales=(2.0, 2.0, 1.0), what="peaked")


def test_fp8_prefill_long_causal_sampled(ta):
    """The 16,384-token causal configuration (the benchmark's launch shape) on sampled rows."""
    case = W.PrefillCase("fp8 long", B=1, Hq=32, Hkv=8, T=16384, D=128, dtype="bf16", causal=True, ragged=False,
                         seed=106)
    x = W.prefill_inputs_fp8(case)
    scales = (0.25, 0.25, 0.5)
    o, lse = _run(ta, x, scales, case.scale, True, "bf16")
    rng = np.random.default_rng(107)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 8191, 16383], rng.integers(0, case.T, 10)]))
    picks = np.array([(0, h, i) for h in range(case.Hq) for i in rows])
    qd, kd, vd = (F8.dequantize(x[n], s) for n, s in (("q", scales[0]), ("k", scales[1]), ("v", scales[2])))
    o_ref, lse_ref = O.prefill_rows(qd, kd, vd, case.scale, True, None, picks)
    bound = F8.prefill_fp8_bound(x["v"], scales[2], case.T)
    _check(o[0][picks[:, 1], picks[:, 2]], lse[0][picks[:, 1], picks[:, 2]], o_ref, lse_ref, bound, 4, "bf16",
           "fp8 long sampled", rows=(picks[:, 0], picks[:, 1]))
