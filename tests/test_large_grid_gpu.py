"""GPU parity of the contiguous 16-bit prefill on grids of several workgroups per CU.

Shapes with ceil(Tq / 128) * Hq * B well above the 256 CUs (workgroups that
wait for a slot and run in later rounds), each covering a case of its own:
the last, partial query tile (Tq not a multiple of 128), both head sizes and
16-bit types, causal and not, ragged batches (workgroups with no rows, rows
past a sequence's end), Tq != Tk (bottom-right causal alignment) and a
negative scale (the sign flip of Q). The oracle runs on sampled rows of every
(batch, head): rows 0, 31, 32, 127, 128, 255, 256, the ends of each 256-row
span, and random ones; the allowance is max(stated bound, derived budget) as
in test_parity_gpu.py. Padded rows must be exactly 0 / -inf.
"""
import sys

import numpy as np
import pytest

import workloads as W
from oracle import bounds as BD
from oracle import oracle as O

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "fp16": 2e-3}
LSE_REL = 1e-4
SPAN = 256


@pytest.fixture(scope="module")
def ta(gpu):
    import torch  # noqa: F401
    import tiled_attention_02_amd as ta
    ta.lib()
    return ta


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _rows(Tq, rng):
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 129, 191, 192, 255]
    for b0 in range(0, Tq, SPAN):
        fixed += [b0, b0 + 1, b0 + SPAN - 1]
    fixed += list(rng.integers(0, Tq, 12)) + [Tq - 1]
    return np.unique(np.array([r for r in fixed if 0 <= r < Tq], dtype=np.int64))


# name, B, Hq, Hkv, Tq, Tk, D, dtype, causal, ragged, scale (None: 1/sqrt(D))
CASES = [
    ("llama-like 2x1100 causal", 2, 32, 8, 1100, 1100, 128, "bf16", True, False, None),
    ("D64 fp16 non-causal", 1, 64, 8, 1030, 1030, 64, "fp16", False, False, None),
    ("ragged batch causal", 8, 16, 4, 600, 600, 128, "bf16", True, True, None),
    ("ragged D64 non-causal", 6, 24, 24, 700, 700, 64, "bf16", False, True, None),
    ("Tq<Tk bottom-right", 1, 64, 16, 1000, 1300, 128, "bf16", True, False, None),
    ("fp16 D128 causal", 2, 40, 8, 777, 777, 128, "fp16", True, False, None),
    ("negative scale", 1, 32, 4, 2048, 2048, 128, "bf16", True, False, -0.0883883),
]


@pytest.mark.parametrize("name,B,Hq,Hkv,Tq,Tk,D,dtype,causal,ragged,scale", CASES, ids=[c[0] for c in CASES])
def test_large_grid_prefill(ta, name, B, Hq, Hkv, Tq, Tk, D, dtype, causal, ragged, scale):
    import torch
    assert -(-Tq // 128) * Hq * B >= 512, "more workgroups than the chip holds at once"
    case = W.PrefillCase(name, B=B, Hq=Hq, Hkv=Hkv, T=Tq, D=D, dtype=dtype, causal=causal, ragged=ragged,
                         seed=700 + Hq + Tq, scale=0.0 if scale is None else scale)
    x = W.prefill_inputs(case, nan_padding=ragged, Tq=Tq, Tk=Tk)
    sc = case.scale
    _note(f"[case] large grid {name}: B={B} Hq={Hq} Hkv={Hkv} Tq={Tq} Tk={Tk} D={D} {dtype} causal={causal} "
          f"scale={sc:.6g}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x[n])).to(tdt).cuda() for n in ("q", "k", "v"))
    sl = None if x["seq_lens"] is None else torch.from_numpy(x["seq_lens"]).cuda()
    o, lse = ta.attn_fwd(q, k, v, scale=sc, causal=causal, seq_lens=sl)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()

    rng = np.random.default_rng(7)
    rows = _rows(Tq, rng)
    picks = np.array([(b, h, i) for b in range(B) for h in range(Hq) for i in rows])
    o_ref, lse_ref = O.prefill_rows(x["q"], x["k"], x["v"], sc, causal, x["seq_lens"], picks)
    bound = BD.prefill_rows(x["q"], x["k"], x["v"], sc, causal, x["seq_lens"], picks, dtype)
    og = o[picks[:, 0], picks[:, 1], picks[:, 2]].astype(np.float64)
    lg = lse[picks[:, 0], picks[:, 1], picks[:, 2]].astype(np.float64)
    valid = np.isfinite(lse_ref)
    err = np.abs(og - o_ref)[valid]
    allow = np.maximum(TOL[dtype], bound[valid])
    ratio = float((err / allow).max()) if err.size else 0.0
    lerr = float((np.abs(lg[valid] - lse_ref[valid]) / np.maximum(1.0, np.abs(lse_ref[valid]))).max()) \
        if valid.any() else 0.0
    _note(f"[parity] large grid {name}: {picks.shape[0]} rows, max|dO|={err.max() if err.size else 0:.3e} "
          f"max err/allowed={ratio:.3f} max rel dlse={lerr:.3e}")
    assert np.isfinite(og[valid]).all()
    assert ratio <= 1.0
    assert lerr <= LSE_REL
    if (~valid).any():
        assert np.all(og[~valid] == 0.0) and np.all(np.isneginf(lg[~valid]))
    if ragged:
        # every padded row of the whole output, not only the sampled ones
        for b in range(B):
            L = int(x["seq_lens"][b])
            assert np.all(o[b, :, L:] == 0.0) and np.all(np.isneginf(lse[b, :, L:]))
