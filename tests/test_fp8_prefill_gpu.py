"""GPU parity of the FP8 prefill (attn_fwd_fp8: E4M3 q, k, v; both products on the fp8 matrix cores).

Two references, both on the dequantized inputs:
  * the float64 prefill definition (oracle/fp8.py): the kernel rounds the probabilities to E4M3 for the
    P.V product, so the allowance is the budget that rounding admits per output element
    (oracle/bounds.prefill_fp8: 2^-4 sum_j P_ij |v_jd| + 2^-17 max_j P_ij sum_j |v_jd| over the row's own
    visible keys, plus fp32 and output-rounding terms), pinned by CPU simulations in
    tests/test_oracle_bounds.py;
  * the same FP8 arithmetic carried out in float64 (oracle/bounds.prefill_fp8_model_rows: 64-key tiles,
    the running max moved when a tile exceeds it by more than 1, p 2^7 rounded to E4M3), within the much
    tighter budget of what fp32 evaluation can change (keys at a rounding boundary, fp32 sums, the
    output rounding, and the fp8 instruction's dot-product accuracy, 2^-13 of the sum of magnitudes,
    re-measured by the last test here). Through O it exposes a dropped or doubled key tile on rows of up
    to a few thousand keys; lse exposes it at every length. Rows whose tile schedule itself is ambiguous
    under that accuracy fall back to the first check only.
lse (from the unrounded probabilities and the fp32 scores) within 1e-4 * max(1, |lse|); padded rows
exactly 0 / -inf.
"""
import numpy as np
import pytest

import workloads as W
from oracle import bounds as BD
from oracle import fp8 as F8
from oracle import oracle as O
from test_parity_gpu import LSE_REL, _note

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


def _check(o, lse, o_ref, lse_ref, bound, what, model=None):
    """o, o_ref, bound: [..., D] (full tensors or picked rows); model: (o_model, budget, ambiguous) for
    the same rows, or None."""
    valid = np.isfinite(lse_ref)
    ov = np.broadcast_to(valid[..., None], o_ref.shape)
    err = np.abs(o - o_ref)
    ratio = float((err[ov] / bound[ov]).max()) if ov.any() else 0.0
    lerr = float((np.abs(lse[valid] - lse_ref[valid]) / np.maximum(1.0, np.abs(lse_ref[valid]))).max())
    msg = (f"[parity] {what}: max|dO|={err[ov].max():.3e} mean|dO|={err[ov].mean():.3e} "
           f"max err/budget={ratio:.3f} max rel dlse={lerr:.3e}")
    mratio = 0.0
    if model is not None:
        mo, mb, amb = model
        use = ov & ~np.broadcast_to(amb[..., None], o_ref.shape)
        mratio = float((np.abs(o - mo)[use] / mb[use]).max()) if use.any() else 0.0
        msg += f" | vs the float64 FP8 model: max err/tight budget={mratio:.3f} ({int(amb.sum())} ambiguous rows)"
    _note(msg)
    assert np.isfinite(o[ov]).all()
    assert ratio <= 1.0
    assert mratio <= 1.0
    assert lerr <= LSE_REL
    inv = ~valid
    if inv.any():
        oi = np.broadcast_to(inv[..., None], o_ref.shape)
        assert np.all(o[oi] == 0.0) and np.all(np.isneginf(lse[inv]))


def _deq(x, scales):
    return tuple(F8.dequantize(x[n], s) for n, s in (("q", scales[0]), ("k", scales[1]), ("v", scales[2])))


def _case_check(ta, case, scales=(0.25, 0.25, 0.5), scale=None, Tq=None, Tk=None, causal=None, out="bf16",
                what=None):
    x = W.prefill_inputs_fp8(case, Tq=Tq, Tk=Tk)
    scale = case.scale if scale is None else scale
    causal = case.causal if causal is None else causal
    what = what or case.name
    _note(f"[case] fp8 prefill {what} causal={causal} scales={scales} q{x['q'].shape} k{x['k'].shape}")
    o, lse = _run(ta, x, scales, scale, causal, out)
    o_ref, lse_ref = F8.prefill_fp8(x["q"], x["k"], x["v"], *scales, scale, causal, x["seq_lens"])
    qd, kd, vd = _deq(x, scales)
    bound = BD.prefill_fp8(qd, kd, vd, scale, causal, x["seq_lens"], out)
    B, Hq, Tq_, _ = qd.shape
    picks = np.array([(b, h, i) for b in range(B) for h in range(Hq) for i in range(Tq_)])
    mo, mb, amb = BD.prefill_fp8_model_rows(qd, kd, vd, scale, causal, x["seq_lens"], picks, out)
    shape = o_ref.shape
    _check(o, lse, o_ref, lse_ref, bound, what,
           model=(mo.reshape(shape), mb.reshape(shape), amb.reshape(shape[:-1])))


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


@pytest.mark.parametrize("T", [64, 128, 192, 256, 320, 513])
@pytest.mark.parametrize("D", [64, 128])
def test_fp8_prefill_ring_lengths(ta, T, D):
    """Key lengths of 1 to 9 tiles of 64: the four-deep K/V rings' prologue (up to 4 K and 2 V tiles issued
    before the first step, the empty ones past the end), their first reuse (tile 5) and the last step's
    product after the loop, causal and not."""
    case = W.PrefillCase("fp8 ring", B=1, Hq=4, Hkv=2, T=T, D=D, dtype="bf16", causal=True, ragged=False,
                         seed=108 + T + D)
    _case_check(ta, case, what=f"T={T} D={D} causal")
    _case_check(ta, case, causal=False, what=f"T={T} D={D} non-causal")


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
    qd, kd, vd = _deq(x, scales)
    o_ref, lse_ref = O.prefill_rows(qd, kd, vd, case.scale, True, None, picks)
    bound = BD.prefill_fp8_rows(qd, kd, vd, case.scale, True, None, picks, "bf16")
    model = BD.prefill_fp8_model_rows(qd, kd, vd, case.scale, True, None, picks, "bf16")
    _check(o[0][picks[:, 1], picks[:, 2]], lse[0][picks[:, 1], picks[:, 2]], o_ref, lse_ref, bound,
           "fp8 long sampled", model=model)


@pytest.mark.parametrize("D", [64, 128])
def test_matrix_instruction_dot_accuracy(ta, D):
    """The accuracy the budgets assume for the scores' dot products, measured through the library: with one
    key, lse = m ln 2 and m = (q . k) c, so lse gives the kernel's dot product. The fp8 instruction must stay
    within F8_DOT (2^-13) of sum |q_e k_e| (oracle/bounds.py), the bf16 one within fp32's gamma_D."""
    import torch
    rng = np.random.default_rng(5 + D)
    Tq = 4096
    scale = 1.0 / np.sqrt(D)
    c = float(np.float32(np.float32(scale) * np.float32(np.log2(np.e))))
    q8 = W.e4m3_codes(rng, (1, 1, Tq, D))
    k8 = W.e4m3_codes(rng, (1, 1, 1, D))
    v8 = W.e4m3_codes(rng, (1, 1, 1, D))
    _, lse = ta.attn_fwd_fp8(_u8(q8), _u8(k8), _u8(v8), 1.0, 1.0, 1.0, scale=scale, causal=False)
    q16 = W.round_to(rng.standard_normal((1, 1, Tq, D), dtype=np.float32) * 2, "bf16")
    k16 = W.round_to(rng.standard_normal((1, 1, 1, D), dtype=np.float32) * 2, "bf16")
    dv = lambda a: torch.from_numpy(a).to(torch.bfloat16).cuda()  # noqa: E731
    _, lse16 = ta.attn_fwd(dv(q16), dv(k16), dv(k16), scale=scale, causal=False)
    torch.cuda.synchronize()
    for name, lg, qv, kv, allow in (
            ("fp8", lse, F8.e4m3_to_float(q8)[0, 0], F8.e4m3_to_float(k8)[0, 0, 0], BD.F8_DOT),
            ("bf16", lse16, q16[0, 0].astype(np.float64), k16[0, 0, 0].astype(np.float64), D * 2.0 ** -24)):
        s_gpu = lg.cpu().numpy()[0, 0].astype(np.float64) / (np.log(2.0) * c)
        rel = np.abs(s_gpu - qv @ kv) / (np.abs(qv) @ np.abs(kv))
        _note(f"[accuracy] {name} D={D}: max |dot error| / sum |products| = {rel.max():.3e} "
              f"(2^{np.log2(rel.max()):.1f}; allowed {allow:.2e} plus the fp32 roundings of the scale and lse)")
        assert rel.max() <= allow + 8 * 2.0 ** -24
