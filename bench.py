#!/usr/bin/env python3
"""Benchmark of libattn on one MI355X.

One step = one pass of the whole hot path on seeded synthetic inputs:
  * causal bf16 prefill, B=1, Hq=32, Hkv=8, T=16384, D=128 (attn_fwd),
  * paged bf16 decode, B=64, Hq=12, Hkv=2, D=128, ctx ~ U[512, 4096],
    16-token blocks (attn_decode_paged), and
  * the same decode over an FP8 (E4M3) cache, one byte per element, codes
    drawn field by field (attn_decode_paged_fp8), and
  * a chunked prefill through the paged cache: 1024-token chunks of 4
    sequences with cached prefixes ~ U[2048, 8192], Llama3-8B heads
    (attn_cache_append of the chunk's K/V into each of 8 layers' caches,
    then attn_fwd_paged on one of them), once plain and once with the rotary
    embedding fused in (rotating append, rotated queries), and once over E4M3
    caches (quantizing append), and
  * the long causal prefill's shape on E4M3 q, k, v (attn_fwd_fp8), and
  * the four Llama3-8B linear layers at 2 activation rows (attn_gemm_splitk).
After the timed steps, two launch-sized prefill workloads get legs of their own
("bert_prefill": the BERT-base-shaped ragged fp16 batch, B=8, H=12, D=64,
lengths ~ U[64, 512]; "llama_prefill": the Llama3-8B-shaped causal bf16
prefill, B=2, Hq=32, Hkv=8, T=512, D=128), each timed per call after the
eviction pass and back to back over rotating copies of its inputs.
Each call is timed with HIP events on the stream it runs on (mean, median and
minimum over the timed steps). Before each call (outside its events) a read
pass over a 1 GiB buffer evicts the inputs from the 256 MB Infinity Cache and
the L2s, so the timed call reads its inputs from HBM; a read pass leaves clean
lines behind, whereas a write pass would leave a gigabyte of dirty lines whose
write-back would land inside the timed region. "context" holds figures
reported beside the headline ones: the rate of a plain streaming read, the MFMA peak derived from the device's CU count and clock, the decode
timed over 4 rotating cache copies instead of the eviction pass, and the host
processor. After timing, the outputs of the timed calls are compared with the
float64 oracle ("parity_on_timed_buffers").

Prints ONE JSON line. value = prefill TFLOP/s (algorithmic flops: 4*D per
unmasked query/key pair); the decode figure (algorithmic HBM bytes: K and V of
valid tokens once per kv head, plus q, o, lse, ctx_lens and the block-table
entries read) sits in "decode". roofline = the prefill kernel against the
dense bf16 MFMA peak (2.5 PFLOP/s); decode.roofline against 8 TB/s HBM.
cpu_baseline = the float64 CPU oracle timed on a bounded sample of the same
prefill workload on this host.
"""
import argparse
import hashlib
import json
import re
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s (bf16 causal prefill) + decode HBM GB/s, % of MI355X peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = {
    "prefill": ["tiled_attention_02_amd/csrc/prefill_fwd.hip", "tiled_attention_02_amd/csrc/attn_device.h"],
    "decode": ["tiled_attention_02_amd/csrc/decode_paged.hip", "tiled_attention_02_amd/csrc/attn_device.h"],
    "chunked_prefill": ["tiled_attention_02_amd/csrc/prefill_fwd.hip", "tiled_attention_02_amd/csrc/attn_device.h"],
    "append": ["tiled_attention_02_amd/csrc/paged_cache.hip"],
    "decode_fp8": ["tiled_attention_02_amd/csrc/decode_paged.hip", "tiled_attention_02_amd/csrc/attn_device.h"],
    "append_rope": ["tiled_attention_02_amd/csrc/paged_cache.hip", "tiled_attention_02_amd/csrc/attn_device.h"],
    "prefill_fp8": ["tiled_attention_02_amd/csrc/prefill_fwd.hip", "tiled_attention_02_amd/csrc/attn_device.h"],
    "append_fp8": ["tiled_attention_02_amd/csrc/paged_cache.hip", "tiled_attention_02_amd/csrc/attn_device.h"],
    "chunked_prefill_fp8": ["tiled_attention_02_amd/csrc/prefill_fwd.hip",
                            "tiled_attention_02_amd/csrc/attn_device.h"],
    "gemm": ["tiled_attention_02_amd/csrc/gemm_splitk.hip", "tiled_attention_02_amd/csrc/attn_device.h"],
}
APPEND_LAYERS = 8
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


_COMMENTS = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def code_sha(texts):
    """Hash of C++/HIP source texts with comments, trailing blanks and empty lines removed."""
    h = hashlib.sha256()
    for text in texts:
        code = "\n".join(ln.rstrip() for ln in _COMMENTS.sub("", text).splitlines() if ln.strip())
        h.update(code.encode())
    return h.hexdigest()[:16]


def source_sha(kind):
    """The code (not the comments) of the kernel sources the committed traffic counters are tied to: a change
    of code voids the counters, a change of comments does not."""
    texts = []
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel)) as f:
            texts.append(f.read())
    return code_sha(texts)


def measured_traffic(kind):
    """HBM bytes per launch from committed rocprofv3 counters, if they match the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kind)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_sha(kind):
        return None
    return rec.get("hbm_bytes_per_launch")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-flush", action="store_true", help="skip the cache flush between calls")
    p.add_argument("--only", choices=["prefill", "prefill_fp8", "decode", "decode_fp8", "chunked", "gemm"],
                   default=None,
                   help="profile helper: run only one of the two calls (not a benchmark line)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="run a plain device copy of this many MiB (counter calibration) and exit")
    return p.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _oracle_threads():
    """Threads the oracle's numpy calls use (BLAS pool size), else the usable cores."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return len(os.sched_getaffinity(0))


def host_cpu():
    """The host processor the oracle runs on: model name and usable cores."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "usable_cores": len(os.sched_getaffinity(0)), "oracle_threads": _oracle_threads()}


def cpu_baseline_prefill(x, case, budget_heads=32, row_stride=8):
    """Time the float64 oracle on a bounded sample of the prefill workload."""
    import numpy as np
    from oracle import oracle as O
    threads = _oracle_threads()
    heads = list(range(0, case.Hq, max(1, case.Hq // budget_heads)))[:budget_heads]
    rows = np.arange(0, case.T, row_stride)
    picks = np.array([(0, h, i) for h in heads for i in rows])
    t0 = time.perf_counter()
    O.prefill_rows(x["q"], x["k"], x["v"], case.scale, True, None, picks)
    dt = time.perf_counter() - t0
    flops = 4.0 * case.D * float((rows + 1).sum()) * len(heads)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 oracle on {len(heads)} of {case.Hq} heads x {len(rows)} query rows "
                      f"(every {row_stride}th) of the 16384-token causal prefill; {dt:.1f} s wall; "
                      f"algorithmic flops of the sampled rows / wall time"}


def cpu_baseline_prefill_fp8(x, case, qs, ks, vs, budget_heads=8, row_stride=16):
    """Time the float64 oracle (dequantize, then the definition) on a bounded sample of the FP8 prefill."""
    import numpy as np
    from oracle import fp8 as F8
    from oracle import oracle as O
    threads = _oracle_threads()
    heads = list(range(0, case.Hq, max(1, case.Hq // budget_heads)))[:budget_heads]
    rows = np.arange(0, case.T, row_stride)
    picks = np.array([(0, h, i) for h in heads for i in rows])
    t0 = time.perf_counter()
    qd, kd, vd = F8.dequantize(x["q"], qs), F8.dequantize(x["k"], ks), F8.dequantize(x["v"], vs)
    O.prefill_rows(qd, kd, vd, case.scale, True, None, picks)
    dt = time.perf_counter() - t0
    flops = 4.0 * case.D * float((rows + 1).sum()) * len(heads)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 oracle (dequantize, then the definition) on {len(heads)} of {case.Hq} heads x "
                      f"{len(rows)} query rows (every {row_stride}th) of the 16384-token causal prefill; "
                      f"{dt:.1f} s wall"}


def cpu_baseline_gemm(gx, min_seconds=5.0):
    """The float64 oracle over the four linear layers at M = 2, repeated for a stable figure."""
    import workloads as W
    from oracle import gemm as G
    reps = 0
    t0 = time.perf_counter()
    while True:
        for d in gx.values():
            G.linear(d["x"], d["w"])
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    nbytes = sum(W.gemm_bytes(d["x"].shape[0], d["w"].shape[0], d["w"].shape[1]) for d in gx.values()) * reps
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": f"float64 oracle (numpy matmul) over the four linear layers at M = 2, the whole workload, "
                      f"repeated {reps} times; {dt:.1f} s wall"}


def cpu_baseline_decode(x, case, nseq=64, min_seconds=5.0):
    import numpy as np
    import workloads as W
    from oracle import oracle as O
    sl = slice(0, nseq)
    reps = 0
    t0 = time.perf_counter()
    while True:  # the whole batch takes well under a second: repeat it for a stable figure
        O.decode_paged(x["q"][sl], x["k_cache"], x["v_cache"], x["block_table"][sl], x["ctx_lens"][sl], case.scale)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    nbytes = W.decode_bytes(x["ctx_lens"][sl], case.Hq, case.Hkv, case.D) * reps
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": f"float64 oracle on the whole batch ({nseq} sequences), repeated {reps} times; "
                      f"{dt:.1f} s wall"}


def cpu_baseline_decode_fp8(x, case, ks, vs, nseq=64, min_seconds=5.0):
    import workloads as W
    from oracle import fp8 as F8
    sl = slice(0, nseq)
    reps = 0
    t0 = time.perf_counter()
    while True:
        F8.decode_paged_fp8(x["q"][sl], x["k_cache"], x["v_cache"], ks, vs, x["block_table"][sl], x["ctx_lens"][sl],
                            case.scale)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    nbytes = W.decode_bytes(x["ctx_lens"][sl], case.Hq, case.Hkv, case.D, kv_elem=1) * reps
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": f"float64 oracle (dequantize, then the decode definition) on the whole batch ({nseq} "
                      f"sequences), repeated {reps} times; {dt:.1f} s wall"}


def cpu_baseline_chunked(x, case, nseq=1, rope=None):
    """Time the float64 oracle on the first sequence(s) of the chunked-prefill batch (all heads, all rows)."""
    import workloads as W
    from oracle import oracle as O
    from oracle import rope as R
    sl = slice(0, nseq)
    t0 = time.perf_counter()
    if rope is None:
        O.prefill_paged(x["q"][sl], x["k_cache"], x["v_cache"], x["block_table"][sl], x["ctx_lens"][sl],
                        x["new_lens"][sl], case.scale, True)
    else:
        R.prefill_paged_rope(x["q"][sl], x["k_cache"], x["v_cache"], x["block_table"][sl], x["ctx_lens"][sl],
                             x["new_lens"][sl], rope, case.scale, case.dtype, True)
    dt = time.perf_counter() - t0
    flops = W.chunk_flops(x["ctx_lens"][sl], x["new_lens"][sl], case.Hq, case.D, True)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": f"float64 oracle (prefill through the block table) on {nseq} of {case.B} sequences, "
                      f"all {case.Hq} heads and rows; {dt:.1f} s wall"}


def cpu_baseline_chunked_fp8(x, case, k8, v8, ks, vs, nseq=1):
    """Time the float64 oracle (dequantize, then the chunked prefill) on the first sequence of the batch."""
    import workloads as W
    from oracle import fp8 as F8
    sl = slice(0, nseq)
    t0 = time.perf_counter()
    F8.prefill_paged_fp8(x["q"][sl], k8, v8, ks, vs, x["block_table"][sl], x["ctx_lens"][sl], x["new_lens"][sl],
                         case.scale, True)
    dt = time.perf_counter() - t0
    flops = W.chunk_flops(x["ctx_lens"][sl], x["new_lens"][sl], case.Hq, case.D, True)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": f"float64 oracle (dequantize the E4M3 cache, then the chunked prefill) on {nseq} of "
                      f"{case.B} sequences, all {case.Hq} heads and rows; {dt:.1f} s wall"}


def _parity(o_gpu, o_ref, lse_gpu=None, lse_ref=None, tol=1e-2, bound=None, strict=False, what=""):
    """Element-wise check of GPU outputs against the oracle's (the rules of the parity tests):
    strict: |dO| <= tol (the five measured workloads); bound given: |dO| <= max(tol, bound), the budget
    of the stated arithmetic (oracle/bounds.py; tol = 0 for the FP8 prefill, whose budget is the whole
    allowance); otherwise max(tol, half a bf16 ulp at |O| + tol). |dlse| <= 1e-4 * max(1, |lse|)."""
    import numpy as np
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    err = np.abs(o_gpu - o_ref)
    if strict:
        allow = np.full(err.shape, tol)
    elif bound is not None:
        allow = np.maximum(tol, bound)
    else:
        allow = np.maximum(tol, 0.5 * 2.0 ** (np.floor(np.log2(np.maximum(np.abs(o_ref) + tol, 2.0 ** -14))) - 7))
    res = {"what": what, "elements": int(err.size), "max_abs_err": float(err.max()),
           "max_err_over_allowed": float((err / allow).max()),
           "rule": "stated bound" if strict else ("derived budget" if bound is not None else "half ulp")}
    ok = bool(np.isfinite(o_gpu).all()) and res["max_err_over_allowed"] <= 1.0
    if lse_gpu is not None:
        lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
        lse_ref = np.asarray(lse_ref, dtype=np.float64)
        rel = np.abs(lse_gpu - lse_ref) / np.maximum(1.0, np.abs(lse_ref))
        res["max_rel_lse_err"] = float(rel.max())
        ok = ok and res["max_rel_lse_err"] <= 1e-4
    res["ok"] = ok
    return res


def parity_on_timed_buffers(ta, torch, np, W, pc, xp, o, lse, xp8, scales8, o8, lse8, dc, xd, do, dlse, xd8, ks8,
                            vs8, do8, dlse8, cc, xc, rope_tab, calls, co, clse, ck8, cv8, gx, gdev):
    """The outputs of the timed calls (the same buffers, after the timed steps) against the float64 oracle on a
    sample: prefill and FP8 prefill on 4 heads x 8 rows of the 16k config, both decodes on the whole batch,
    each chunked leg (re-run once on its own caches: the legs share the output buffer) on its first sequence,
    every linear layer whole. Part of the CPU-baseline leg (it runs the oracle)."""
    from oracle import bounds as BD
    from oracle import fp8 as F8
    from oracle import gemm as G
    from oracle import oracle as O
    from oracle import rope as R
    res = {}
    torch.cuda.synchronize()
    heads, rows = [0, 7, 13, 31], [0, 1, 127, 128, 4095, 8191, 12000, 16383]
    picks = np.array([(0, h, i) for h in heads for i in rows])
    og, lg = o.float().cpu().numpy(), lse.cpu().numpy()
    orf, lrf = O.prefill_rows(xp["q"], xp["k"], xp["v"], pc.scale, True, None, picks)
    res["prefill"] = _parity(og[0, picks[:, 1], picks[:, 2]], orf, lg[0, picks[:, 1], picks[:, 2]], lrf,
                             strict=True, what="4 heads x 8 rows")
    qs, kps, vps = scales8
    og8, lg8 = o8.float().cpu().numpy(), lse8.cpu().numpy()
    qd, kd, vd = F8.dequantize(xp8["q"], qs), F8.dequantize(xp8["k"], kps), F8.dequantize(xp8["v"], vps)
    orf8, lrf8 = O.prefill_rows(qd, kd, vd, pc.scale, True, None, picks)
    bnd8 = BD.prefill_fp8_rows(qd, kd, vd, pc.scale, True, None, picks, "bf16")
    og8p = og8[0, picks[:, 1], picks[:, 2]]
    res["prefill_fp8"] = _parity(og8p, orf8, lg8[0, picks[:, 1], picks[:, 2]], lrf8, tol=0.0, bound=bnd8,
                                 what="4 heads x 8 rows; budget of the E4M3 rounding of P")
    mo8, mb8, amb8 = BD.prefill_fp8_model_rows(qd, kd, vd, pc.scale, True, None, picks, "bf16")
    res["prefill_fp8_model"] = _parity(og8p[~amb8], mo8[~amb8], tol=0.0, bound=mb8[~amb8],
                                       what="the same rows against the FP8 arithmetic in float64 (tight budget)")
    dref, dlref = O.decode_paged(xd["q"], xd["k_cache"], xd["v_cache"], xd["block_table"], xd["ctx_lens"], dc.scale)
    res["decode"] = _parity(do.float().cpu().numpy(), dref, dlse.cpu().numpy(), dlref, strict=True,
                            what="whole batch")
    d8ref, dl8ref = F8.decode_paged_fp8(xd8["q"], xd8["k_cache"], xd8["v_cache"], ks8, vs8, xd8["block_table"],
                                        xd8["ctx_lens"], dc.scale)
    d8b = BD.decode_paged(xd8["q"], F8.dequantize(xd8["k_cache"], ks8), F8.dequantize(xd8["v_cache"], vs8),
                          xd8["block_table"], xd8["ctx_lens"], dc.scale, "bf16")
    res["decode_fp8"] = _parity(do8.float().cpu().numpy(), d8ref, dlse8.cpu().numpy(), dl8ref, bound=d8b,
                                what="whole batch")
    sl = slice(0, 1)
    kref, vref = O.cache_append(xc["k_new"], xc["v_new"], xc["k_cache"], xc["v_cache"], xc["block_table"],
                                xc["start_pos"], xc["new_lens"])
    for name, call in calls:
        call()
        torch.cuda.synchronize()
        og_c, lg_c = co[0:1].float().cpu().numpy(), clse[0:1].cpu().numpy()
        if name == "chunked":
            r, lr_ = O.prefill_paged(xc["q"][sl], kref, vref, xc["block_table"][sl], xc["ctx_lens"][sl],
                                     xc["new_lens"][sl], cc.scale, True)
        elif name == "chunked_rope":
            tab = rope_tab.cpu().numpy()
            kr, vr = R.cache_append_rope(xc["k_new"], xc["v_new"], xc["k_cache"], xc["v_cache"], xc["block_table"],
                                         xc["start_pos"], tab, cc.dtype, xc["new_lens"])
            r, lr_ = R.prefill_paged_rope(xc["q"][sl], kr, vr, xc["block_table"][sl], xc["ctx_lens"][sl],
                                          xc["new_lens"][sl], tab, cc.scale, cc.dtype, True)
        else:
            k8r, v8r = F8.cache_append_fp8(xc["k_new"], xc["v_new"], ck8, cv8, xc["block_table"], xc["start_pos"],
                                           ks8, vs8, xc["new_lens"])
            r, lr_ = F8.prefill_paged_fp8(xc["q"][sl], k8r, v8r, ks8, vs8, xc["block_table"][sl], xc["ctx_lens"][sl],
                                          xc["new_lens"][sl], cc.scale, True)
        n = int(xc["new_lens"][0])
        res[name] = _parity(og_c[:, :, :n], r[:, :, :n], lg_c[:, :, :n], lr_[:, :, :n],
                            what="first sequence, all heads and rows")
    worst = 0.0
    for name, d in gx.items():
        yg = gdev[name][2].float().cpu().numpy()
        ratio = float((np.abs(yg - G.linear(d["x"], d["w"])) / G.error_bound(d["x"], d["w"], "bf16")).max())
        worst = max(worst, ratio)
    res["gemm"] = {"what": "four layers, every element", "max_err_over_bound": worst, "ok": worst <= 1.0}
    res["all_ok"] = all(v.get("ok", False) for v in res.values() if isinstance(v, dict))
    return res


def clock_derived_peak(torch):
    """Dense bf16 MFMA peak from the chip's CU count and maximum shader clock read on the box:
    nCU x 4096 flop/clk (a 32x32x16 bf16 MFMA is 32768 flop in 32 clocks on each of 4 SIMDs) x sclk.
    The clock comes from the HIP runtime already loaded in this process (no second load)."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD)
    except OSError:
        return None
    khz = ctypes.c_int(0)
    dev = torch.cuda.current_device()
    HIP_DEVICE_ATTRIBUTE_CLOCK_RATE = 5  # hipDeviceAttributeClockRate (kHz) in hip_runtime_api.h
    if hip.hipDeviceGetAttribute(ctypes.byref(khz), HIP_DEVICE_ATTRIBUTE_CLOCK_RATE, dev) != 0 or khz.value <= 0:
        return None
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    return {"cus": int(ncu), "max_sclk_mhz": khz.value / 1e3,
            "bf16_dense_tflops": round(ncu * 4096 * khz.value * 1e3 / 1e12, 1)}


def decode_rotation_crosscheck(ta, torch, np, dq, kc, vc, bt, cl, scale, ws, copies=4, reps=24):
    """Decode timed without the eviction pass, rotating through `copies` independent copies of the caches
    (each 150 MB, together past the 256 MB Infinity Cache), so each call still finds its cache cold."""
    kcs = [kc] + [kc.clone() for _ in range(copies - 1)]
    vcs = [vc] + [vc.clone() for _ in range(copies - 1)]
    out = torch.empty_like(dq)
    lse = torch.empty(dq.shape[:2], dtype=torch.float32, device=dq.device)
    for i in range(copies):
        ta.attn_decode_paged(dq, kcs[i], vcs[i], bt, cl, scale=scale, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    ts = []
    for r in range(reps):
        i = r % copies
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ta.attn_decode_paged(dq, kcs[i], vcs[i], bt, cl, scale=scale, out=out, lse=lse, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    # the same calls back to back, as a model's layers would make them (one call per layer's cache, no
    # events between): one event pair around each pass over the copies
    bursts = []
    for r in range(max(1, reps // copies)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(copies):
            ta.attn_decode_paged(dq, kcs[i], vcs[i], bt, cl, scale=scale, out=out, lse=lse, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        bursts.append(e0.elapsed_time(e1) / copies)
    del kcs, vcs
    return float(np.median(ts)) * 1e3, float(np.min(ts)) * 1e3, float(np.median(bursts)) * 1e3


def small_prefill_leg(ta, torch, np, W, dev, case, evict, steps, copies):
    """A launch-sized prefill workload (the BERT-shaped ragged batch, the Llama3-8B-shaped 512-token causal
    prefill): timed per call after the eviction pass (events around each call), and back to back over
    `copies` independent copies of the inputs (more bytes in total than the 256 MB Infinity Cache holds, so
    each call reads its inputs from HBM, as a model's layers would). The back-to-back pass is one HIP graph of
    the `copies` calls, replayed with events around each replay: the launches run back to back on the GPU,
    without the Python binding's per-call host time (a few microseconds, as long as these kernels), which a
    loop of calls would measure instead. Returns (result dict, inputs, the first copy's o and lse; these last
    from a graph replay)."""
    x = W.prefill_inputs(case, nan_padding=case.ragged)
    tdt = torch.float16 if case.dtype == "fp16" else torch.bfloat16
    base = [torch.from_numpy(x[n]).to(tdt).to(dev) for n in ("q", "k", "v")]
    sets = []
    for c in range(copies):
        q, k, v = base if c == 0 else [t.clone() for t in base]
        sets.append((q, k, v, torch.empty_like(q), torch.empty(q.shape[:3], dtype=torch.float32, device=dev)))
    sl = None if x["seq_lens"] is None else torch.from_numpy(x["seq_lens"]).to(dev)

    def call(i):
        q, k, v, o, lse = sets[i]
        ta.attn_fwd(q, k, v, scale=case.scale, causal=case.causal, seq_lens=sl, out=o, lse=lse)

    for i in range(copies):
        call(i)
    torch.cuda.synchronize()
    per = []
    for _ in range(steps):
        evict()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call(0)
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for i in range(copies):
            call(i)
    torch.cuda.synchronize()
    b2b = []
    for _ in range(max(5, steps // 2)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        b2b.append(e0.elapsed_time(e1) / copies)
    flops = W.prefill_flops(case.B, case.Hq, case.T, case.T, case.D, case.causal, x["seq_lens"])
    nbytes = W.prefill_bytes(case.B, case.Hq, case.Hkv, case.T, case.T, case.D, x["seq_lens"])
    t_b2b, t_per = float(np.mean(b2b)) * 1e-3, float(np.mean(per)) * 1e-3
    tfs = flops / t_b2b / 1e12
    res = {
        "workload": case.name + (f", lengths {[int(v) for v in x['seq_lens']]}" if x["seq_lens"] is not None else ""),
        "value": round(tfs, 2), "unit": "TFLOP/s",
        "timing": f"back to back over {copies} input copies: one HIP graph of the {copies} calls, events "
                  "around each replay, per-call mean; us_per_call: one call after the eviction pass, events "
                  "around it",
        "us_per_call_back_to_back": round(t_b2b * 1e6, 2),
        "us_per_call_back_to_back_min": round(float(np.min(b2b)) * 1e3, 2),
        "us_per_call": round(t_per * 1e6, 2), "us_per_call_median": round(float(np.median(per)) * 1e3, 2),
        "tflops_per_call": round(flops / t_per / 1e12, 2),
        "gflop_per_call": round(flops / 1e9, 4), "mb_per_call": round(nbytes / 1e6, 3),
        "roofline": {"bound": "mfma", "achieved": round(tfs, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tfs / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "prefill_kernel", "algorithmic_flops_per_launch": flops,
                     "hbm_frac": round(nbytes / t_b2b / 1e9 / PEAK_HBM_GBS, 4),
                     "note": "arithmetic intensity below the ridge (about 312 flop/byte): the launch is short enough "
                             "that its fixed costs set the time; hbm_frac is the algorithmic bytes' rate against "
                             "8 TB/s"}}
    return res, x, sets[0][3], sets[0][4]


def cpu_baseline_small_prefill(x, case, min_seconds=5.0):
    """The float64 oracle on the whole workload, repeated for a stable figure."""
    import workloads as W
    from oracle import oracle as O
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.prefill(x["q"], x["k"], x["v"], case.scale, case.causal, x["seq_lens"])
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    flops = W.prefill_flops(case.B, case.Hq, case.T, case.T, case.D, case.causal, x["seq_lens"]) * reps
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _oracle_threads(), "kind": "oracle",
            "sample": f"float64 oracle on the whole workload (every head and row), repeated {reps} times; "
                      f"{dt:.1f} s wall"}


def context_measurements(ta, W, torch, np, dev, flush_rows, flush_dst, evict):
    """Figures reported beside the headline numbers (not part of `value`): the rate of a plain streaming
    read, i.e. the 1 GiB eviction pass itself (torch.sum over rows of 4096 float32), the HBM read rate a
    simple kernel attains here."""
    rd = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.sum(flush_rows, dim=1, out=flush_dst)
        e1.record()
        torch.cuda.synchronize()
        rd.append(e0.elapsed_time(e1))
    nbytes = flush_rows.numel() * 4
    return {
        "streaming_read_gbs": {"value": round(nbytes / (float(np.median(rd)) * 1e-3) / 1e9, 1),
                               "what": "torch.sum over a 1 GiB float32 buffer in rows of 4096 (the eviction pass), median of 5"},
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "libattn's benchmark runs on one GPU only: it has no multi-GPU path "
                                   "(every figure is a single-GPU figure)", "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch
    import tiled_attention_02_amd as ta
    import workloads as W

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ta.lib()

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}))
        return

    pc, dc = W.LONG, W.QWEN
    log(f"[bench] building inputs: {pc.name}; {dc.name}")
    xp = W.prefill_inputs(pc)
    xd = W.decode_inputs(dc)
    bf = torch.bfloat16
    q = torch.from_numpy(xp["q"]).to(bf).to(dev)
    k = torch.from_numpy(xp["k"]).to(bf).to(dev)
    v = torch.from_numpy(xp["v"]).to(bf).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    dq = torch.from_numpy(xd["q"]).to(bf).to(dev)
    kc = torch.from_numpy(xd["k_cache"]).to(bf).to(dev)
    vc = torch.from_numpy(xd["v_cache"]).to(bf).to(dev)
    bt = torch.from_numpy(xd["block_table"]).to(dev)
    cl = torch.from_numpy(xd["ctx_lens"]).to(dev)
    do = torch.empty_like(dq)
    dlse = torch.empty(dq.shape[:2], dtype=torch.float32, device=dev)
    ws = torch.empty(max(256, ta.attn_decode_workspace_bytes(dc.B, dc.Hq, dc.Hkv, dc.D, bt.shape[1])),
                     dtype=torch.uint8, device=dev)
    flush_src = torch.ones((1 << 18, 1024), dtype=torch.float32, device=dev)  # 1 GiB
    flush_rows = flush_src.view(-1, 4096)
    flush_dst = torch.empty(flush_rows.shape[0], dtype=torch.float32, device=dev)

    # the long prefill again on E4M3 inputs (both products on the fp8 matrix cores)
    xp8 = W.prefill_inputs_fp8(pc)
    QS8, KSP8, VSP8 = 0.25, 0.25, 0.5
    q8, k8p, v8p = (torch.from_numpy(xp8[n]).to(dev) for n in ("q", "k", "v"))
    o8 = torch.empty_like(o)
    lse8 = torch.empty_like(lse)

    # the decode batch again, over an E4M3 cache (same q, table and lengths)
    xd8 = W.decode_inputs_fp8(dc)
    KS8, VS8 = 0.25, 0.0625
    kc8 = torch.from_numpy(xd8["k_cache"]).to(dev)
    vc8 = torch.from_numpy(xd8["v_cache"]).to(dev)
    do8 = torch.empty_like(dq)
    dlse8 = torch.empty_like(dlse)

    cc = W.CHUNK
    log(f"[bench] building inputs: {cc.name}")
    xc = W.chunk_inputs(cc)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)  # noqa: E731
    cq = torch.from_numpy(xc["q"]).to(bf).to(dev)
    ckn = torch.from_numpy(xc["k_new"]).to(bf).to(dev)
    cvn = torch.from_numpy(xc["v_new"]).to(bf).to(dev)
    ckc = torch.from_numpy(xc["k_cache"]).to(bf).to(dev)
    cvc = torch.from_numpy(xc["v_cache"]).to(bf).to(dev)
    cbt, cst, cnl, ccl = (i32(xc[n]) for n in ("block_table", "start_pos", "new_lens", "ctx_lens"))
    co = torch.empty_like(cq)
    clse = torch.empty(cq.shape[:3], dtype=torch.float32, device=dev)
    # the append is timed as a burst over APPEND_LAYERS layers, each with its
    # own chunk and its own cache (as a model appends once per layer): one
    # ~10 us call between two events would mostly time the launch
    app_sets = [(ckn, cvn, ckc, cvc)] + [tuple(t.clone() for t in (ckn, cvn, ckc, cvc))
                                         for _ in range(APPEND_LAYERS - 1)]

    # the rotary leg: the same chunk with RoPE fused into the append and the
    # query load (its own caches, so each leg keeps its own cache contents)
    rope_tab = torch.from_numpy(W.rope_table(16384, cc.D)).to(dev)
    rope_sets = [tuple(t.clone() for t in (ckn, cvn, ckc, cvc)) for _ in range(APPEND_LAYERS)]
    # the FP8 leg: the chunk quantized into E4M3 caches, then the chunked prefill over them
    c8 = np.random.default_rng(cc.seed + 1000)
    ck8 = torch.from_numpy(W.e4m3_codes(c8, xc["k_cache"].shape)).to(dev)
    cv8 = torch.from_numpy(W.e4m3_codes(c8, xc["v_cache"].shape)).to(dev)
    fp8_sets = [(ckn, cvn, ck8, cv8)] + [tuple(t.clone() for t in (ckn, cvn, ck8, cv8))
                                         for _ in range(APPEND_LAYERS - 1)]

    # the linear layers of a Llama3-8B / Granite-8B block at decode batch 2 (split-K GEMM)
    log("[bench] building inputs: Llama3-8B linear layers, M = 2")
    gx = {name: W.gemm_inputs(W.LINEAR_M, N, K, "bf16", seed=80 + i)
          for i, (name, (N, K)) in enumerate(W.LINEAR_SHAPES.items())}
    gdev = {name: (torch.from_numpy(d["x"]).to(bf).to(dev), torch.from_numpy(d["w"]).to(bf).to(dev),
                   torch.empty((W.LINEAR_M, d["w"].shape[0]), dtype=bf, device=dev)) for name, d in gx.items()}
    gbytes = {name: W.gemm_bytes(W.LINEAR_M, *W.LINEAR_SHAPES[name]) for name in gx}

    pflops = W.prefill_flops(pc.B, pc.Hq, pc.T, pc.T, pc.D, True)
    dbytes = W.decode_bytes(xd["ctx_lens"], dc.Hq, dc.Hkv, dc.D)
    d8bytes = W.decode_bytes(xd8["ctx_lens"], dc.Hq, dc.Hkv, dc.D, kv_elem=1)
    cflops = W.chunk_flops(xc["ctx_lens"], xc["new_lens"], cc.Hq, cc.D, True)
    abytes = W.append_bytes(xc["new_lens"], cc.Hkv, cc.D)
    # The step's timed parts, in order: (name, call, calls per event pair).
    # Each part starts after the eviction pass and sits between two events on
    # the stream it runs on.
    parts = []
    if args.only in (None, "prefill"):
        parts.append(("prefill", lambda: ta.attn_fwd(q, k, v, scale=pc.scale, causal=True, out=o, lse=lse), 1))
    if args.only in (None, "prefill_fp8"):
        parts.append(("prefill_fp8", lambda: ta.attn_fwd_fp8(q8, k8p, v8p, QS8, KSP8, VSP8, scale=pc.scale,
                                                             causal=True, out=o8, lse=lse8), 1))
    if args.only in (None, "decode"):
        parts.append(("decode", lambda: ta.attn_decode_paged(dq, kc, vc, bt, cl, scale=dc.scale, out=do, lse=dlse,
                                                             workspace=ws), 1))
    if args.only in (None, "decode_fp8"):
        parts.append(("decode_fp8", lambda: ta.attn_decode_paged_fp8(dq, kc8, vc8, KS8, VS8, bt, cl, scale=dc.scale,
                                                                     out=do8, lse=dlse8, workspace=ws), 1))
    for rope, tag in ((None, ""), (rope_tab, "_rope")):
        if args.only not in (None, "chunked"):
            break
        sets = app_sets if rope is None else rope_sets

        def appends(sets=sets, rope=rope):
            # the chunk's K/V go into every layer's cache
            for kn_, vn_, kc_, vc_ in sets:
                ta.attn_cache_append(kn_, vn_, kc_, vc_, cbt, cst, cnl, rope=rope)

        def chunk_prefill(sets=sets, rope=rope):
            # then the chunk attends to prefix + itself (first layer's cache)
            ta.attn_fwd_paged(cq, sets[0][2], sets[0][3], cbt, ccl, cnl, scale=cc.scale, causal=True, out=co,
                              lse=clse, rope=rope)

        parts.append(("append" + tag, appends, APPEND_LAYERS))
        parts.append(("chunked_prefill" + tag, chunk_prefill, 1))
    if args.only in (None, "chunked"):
        def appends8():
            for kn_, vn_, kc_, vc_ in fp8_sets:
                ta.attn_cache_append_fp8(kn_, vn_, kc_, vc_, KS8, VS8, cbt, cst, cnl)

        def chunk_prefill8():
            ta.attn_fwd_paged_fp8(cq, ck8, cv8, KS8, VS8, cbt, ccl, cnl, scale=cc.scale, causal=True, out=co,
                                  lse=clse)

        parts.append(("append_fp8", appends8, APPEND_LAYERS))
        parts.append(("chunked_prefill_fp8", chunk_prefill8, 1))

    if args.only in (None, "gemm"):
        for name, (gxd, gwd, gyd) in gdev.items():
            parts.append(("gemm_" + name, (lambda x_=gxd, w_=gwd, y_=gyd: ta.attn_gemm_splitk(x_, w_, out=y_)), 1))

    def evict():
        # read-only pass over 1 GiB: pushes the inputs out of every cache level
        # without leaving dirty lines to write back during the timed call
        if not args.no_flush:
            torch.sum(flush_rows, dim=1, out=flush_dst)

    def step(evs):
        for i, (_, call, _) in enumerate(parts):
            evict()
            evs[2 * i].record()
            call()
            evs[2 * i + 1].record()

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(parts))]  # noqa: E731
    for i in range(args.warmup):
        step(mk())
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps")
    evs = [mk() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-call mean (ms) of every part; a burst counts as n calls
    ms = {name: float(np.mean([e[2 * i].elapsed_time(e[2 * i + 1]) / n for e in evs]))
          for i, (name, _, n) in enumerate(parts)}
    ms_min = {name: float(np.min([e[2 * i].elapsed_time(e[2 * i + 1]) / n for e in evs]))
              for i, (name, _, n) in enumerate(parts)}
    ms_med = {name: float(np.median([e[2 * i].elapsed_time(e[2 * i + 1]) / n for e in evs]))
              for i, (name, _, n) in enumerate(parts)}
    log("[bench] " + "; ".join(f"{k} {v * 1e3:.1f} us (min {ms_min[k] * 1e3:.1f})" for k, v in ms.items()) +
        f"; wall/step {wall / args.steps * 1e3:.2f} ms")
    if args.only:
        print(json.dumps({"only": args.only, "ms_per_call": ms}))
        return
    p_avg, d_avg, d8_avg = ms["prefill"], ms["decode"], ms["decode_fp8"]
    p8_avg = ms["prefill_fp8"]
    a_avg, c_avg = ms["append"], ms["chunked_prefill"]
    ar_avg, cr_avg = ms["append_rope"], ms["chunked_prefill_rope"]
    a8_avg, c8_avg = ms["append_fp8"], ms["chunked_prefill_fp8"]

    p_tfs = pflops / (p_avg * 1e-3) / 1e12
    p8_tfs = pflops / (p8_avg * 1e-3) / 1e12
    d_gbs = dbytes / (d_avg * 1e-3) / 1e9
    c_tfs = cflops / (c_avg * 1e-3) / 1e12
    a_gbs = abytes / (a_avg * 1e-3) / 1e9
    d8_gbs = d8bytes / (d8_avg * 1e-3) / 1e9
    cr_tfs = cflops / (cr_avg * 1e-3) / 1e12
    ar_gbs = abytes / (ar_avg * 1e-3) / 1e9
    c8_tfs = cflops / (c8_avg * 1e-3) / 1e12
    a8bytes = abytes * 3 // 4  # the chunk's K and V read as 16-bit values, written as 1-byte codes
    a8_gbs = a8bytes / (a8_avg * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(p_tfs, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sum(ms[name] * n for name, _, n in parts), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal bf16 prefill B=1 Hq=32 Hkv=8 T=16384 D=128 (value; again on E4M3 inputs: "
                               "prefill_fp8) + paged bf16 decode "
                               "B=64 Hq=12 Hkv=2 D=128 ctx~U[512,4096] block=16 (decode; again over an E4M3 cache: decode_fp8) + "
                               "chunked bf16 prefill "
                               "B=4 Hq=32 Hkv=8 D=128 prefix~U[2048,8192] chunk=1024 through the block table "
                               "(chunked; again with RoPE fused: chunked_rope; again over E4M3 caches: "
                               "chunked_fp8) + split-K GEMM of the four Llama3-8B linear layers at M=2 (gemm) + "
                               "ragged fp16 encoder prefill B=8 H=12 D=64 lengths~U[64,512] (bert_prefill) + causal "
                               "bf16 prefill B=2 Hq=32 Hkv=8 T=512 D=128 (llama_prefill)",
                   "prefill_gflop_per_call": round(pflops / 1e9, 3),
                   "decode_mb_per_call": round(dbytes / 1e6, 3),
                   "cache_eviction_before_each_call": "none" if args.no_flush else "1 GiB read pass",
                   "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 3)},
        "roofline": {"bound": "mfma", "achieved": round(p_tfs, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(p_tfs / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic("prefill"),
                     "kernel": "prefill_kernel", "ms_per_launch": round(p_avg, 4),
                     "ms_per_launch_median": round(ms_med["prefill"], 4), "ms_per_launch_min": round(ms_min["prefill"], 4),
                     "algorithmic_flops_per_launch": pflops},
        "prefill_fp8": {"value": round(p8_tfs, 2), "unit": "TFLOP/s", "ms_per_call": round(p8_avg, 4),
                        "workload": pc.name + ", E4M3 q/k/v (scales 0.25, 0.25, 0.5), bf16 output",
                        "roofline": {"bound": "mfma", "achieved": round(p8_tfs, 2), "peak": PEAK_FP8_TFLOPS,
                                     "unit": "TFLOP/s", "frac": round(p8_tfs / PEAK_FP8_TFLOPS, 4),
                                     "traffic": measured_traffic("prefill_fp8"),
                                     "kernel": "prefill_kernel (FP8 form: fp8 x fp8 products)",
                                     "algorithmic_flops_per_launch": pflops}},
        "decode": {"value": round(d_gbs, 1), "unit": "GB/s", "us_per_call": round(d_avg * 1e3, 2),
                   "us_per_call_median": round(ms_med["decode"] * 1e3, 2), "us_per_call_min": round(ms_min["decode"] * 1e3, 2),
                   "roofline": {"bound": "hbm", "achieved": round(d_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(d_gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic("decode"),
                                "kernels": "decode_split_kernel + decode_combine_kernel",
                                "algorithmic_bytes_per_call": dbytes}},
        "decode_fp8": {"value": round(d8_gbs, 1), "unit": "GB/s", "us_per_call": round(d8_avg * 1e3, 2),
                       "k_scale": KS8, "v_scale": VS8,
                       "roofline": {"bound": "hbm", "achieved": round(d8_gbs, 1), "peak": PEAK_HBM_GBS,
                                    "unit": "GB/s", "frac": round(d8_gbs / PEAK_HBM_GBS, 4),
                                    "traffic": measured_traffic("decode_fp8"),
                                    "kernels": "decode_split_kernel<fp8> + decode_combine_kernel",
                                    "algorithmic_bytes_per_call": d8bytes}},
        "chunked": {
            "workload": cc.name, "ctx_lens": [int(c) for c in xc["ctx_lens"]],
            "prefill": {"value": round(c_tfs, 2), "unit": "TFLOP/s", "us_per_call": round(c_avg * 1e3, 2),
                        "roofline": {"bound": "mfma", "achieved": round(c_tfs, 2), "peak": PEAK_BF16_TFLOPS,
                                     "unit": "TFLOP/s", "frac": round(c_tfs / PEAK_BF16_TFLOPS, 4),
                                     "traffic": measured_traffic("chunked_prefill"),
                                     "kernel": "prefill_kernel (paged form)", "algorithmic_flops_per_launch": cflops}},
            "append": {"value": round(a_gbs, 1), "unit": "GB/s", "us_per_call": round(a_avg * 1e3, 2),
                       "timing": f"a burst of {APPEND_LAYERS} appends (one per layer, each with its own chunk "
                                 "and cache) between two events, after the eviction pass; per-call mean",
                       "roofline": {"bound": "hbm", "achieved": round(a_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                    "frac": round(a_gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic("append"),
                                    "kernel": "append_kernel", "algorithmic_bytes_per_launch": abytes}}},
        "chunked_rope": {
            "workload": cc.name + ", rotary embedding fused (K rotated in the append, Q in the prefill's Q load)",
            "prefill": {"value": round(cr_tfs, 2), "unit": "TFLOP/s", "us_per_call": round(cr_avg * 1e3, 2),
                        "roofline": {"bound": "mfma", "achieved": round(cr_tfs, 2), "peak": PEAK_BF16_TFLOPS,
                                     "unit": "TFLOP/s", "frac": round(cr_tfs / PEAK_BF16_TFLOPS, 4),
                                     "traffic": measured_traffic("chunked_prefill"),
                                     "kernel": "prefill_kernel (paged form, rotated queries)",
                                     "algorithmic_flops_per_launch": cflops}},
            "append": {"value": round(ar_gbs, 1), "unit": "GB/s", "us_per_call": round(ar_avg * 1e3, 2),
                       "timing": f"a burst of {APPEND_LAYERS} appends, as for chunked.append",
                       "roofline": {"bound": "hbm", "achieved": round(ar_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                    "frac": round(ar_gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic("append_rope"),
                                    "kernel": "append_rope_kernel", "algorithmic_bytes_per_launch": abytes,
                                    "note": "bytes: the chunk's K and V read and written once; the table rows "
                                            "read are not counted"}}},
        "chunked_fp8": {
            "workload": cc.name + ", over E4M3 caches (k_scale, v_scale as decode_fp8)",
            "prefill": {"value": round(c8_tfs, 2), "unit": "TFLOP/s", "us_per_call": round(c8_avg * 1e3, 2),
                        "roofline": {"bound": "mfma", "achieved": round(c8_tfs, 2), "peak": PEAK_BF16_TFLOPS,
                                     "unit": "TFLOP/s", "frac": round(c8_tfs / PEAK_BF16_TFLOPS, 4),
                                     "traffic": measured_traffic("chunked_prefill_fp8"),
                                     "kernel": "prefill_kernel (paged form, E4M3 tiles; bf16 products)",
                                     "algorithmic_flops_per_launch": cflops}},
            "append": {"value": round(a8_gbs, 1), "unit": "GB/s", "us_per_call": round(a8_avg * 1e3, 2),
                       "timing": f"a burst of {APPEND_LAYERS} quantizing appends, as for chunked.append",
                       "roofline": {"bound": "hbm", "achieved": round(a8_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                    "frac": round(a8_gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic("append_fp8"),
                                    "kernel": "append_kernel (E4M3 codes)", "algorithmic_bytes_per_launch": a8bytes}}},
    }
    g_us = {name: ms["gemm_" + name] * 1e3 for name in gx}
    g_gbs = sum(gbytes.values()) / (sum(g_us.values()) * 1e-6) / 1e9
    gu_gbs = gbytes["gate_up_proj"] / (g_us["gate_up_proj"] * 1e-6) / 1e9
    out["gemm"] = {
        "workload": "split-K GEMM y = x w^T, bf16, the four linear layers of a Llama3-8B / Granite-8B block "
                    "(q/k/v 6144x4096, o 4096x4096, gate/up 28672x4096, down 4096x14336) at M = 2 tokens, "
                    "each call after the eviction pass (weights cold, as in a decode step)",
        "value": round(g_gbs, 1), "unit": "GB/s", "us_per_layer": round(sum(g_us.values()), 2),
        "layers": {name: {"us_per_call": round(g_us[name], 2),
                          "GB_per_s": round(gbytes[name] / (g_us[name] * 1e-6) / 1e9, 1),
                          "config": "tuned table"} for name in gx},
        "roofline": {"bound": "hbm", "achieved": round(gu_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic("gemm"),
                     "kernel": "gemm_splitk_kernel (gate/up projection, the largest launch)",
                     "algorithmic_bytes_per_launch": gbytes["gate_up_proj"]}}
    small = {}
    for key, case, copies in (("bert_prefill", W.BERT, 24), ("llama_prefill", W.LLAMA, 16)):
        log(f"[bench] {case.name}: per call and back to back over {copies} input copies")
        small[key] = small_prefill_leg(ta, torch, np, W, dev, case, evict, max(args.steps, 20), copies)
        out[key] = small[key][0]
    out["context"] = context_measurements(ta, W, torch, np, dev, flush_rows, flush_dst, evict)
    out["context"]["clock_derived_peak"] = clock_derived_peak(torch)
    out["context"]["host_cpu"] = host_cpu()
    rot_med, rot_min, burst = decode_rotation_crosscheck(ta, torch, np, dq, kc, vc, bt, cl, dc.scale, ws)
    out["context"]["decode_rotating_4_cache_copies"] = {
        "us_per_call_median": round(rot_med, 2), "us_per_call_min": round(rot_min, 2),
        "GB_per_s_median": round(dbytes / (rot_med * 1e-6) / 1e9, 1),
        "us_per_call_back_to_back": round(burst, 2),
        "GB_per_s_back_to_back": round(dbytes / (burst * 1e-6) / 1e9, 1),
        "what": "attn_decode_paged without the eviction pass, rotating 4 independent copies of the caches: "
                "events around each call, and around passes of 4 back-to-back calls (one per copy, as a "
                "model's layers make them) divided by 4"}
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline: float64 oracle on a sample of the prefill workload")
        out["cpu_baseline"] = cpu_baseline_prefill(xp, pc)
        log("[bench] cpu baseline: float64 oracle on a sample of the FP8 prefill workload")
        out["prefill_fp8"]["cpu_baseline"] = cpu_baseline_prefill_fp8(xp8, pc, QS8, KSP8, VSP8)
        log("[bench] cpu baseline: float64 oracle on a sample of the decode workload")
        out["decode"]["cpu_baseline"] = cpu_baseline_decode(xd, dc)
        log("[bench] cpu baseline: float64 oracle on the FP8 decode workload")
        out["decode_fp8"]["cpu_baseline"] = cpu_baseline_decode_fp8(xd8, dc, KS8, VS8)
        log("[bench] cpu baseline: float64 oracle on a sample of the chunked-prefill workload")
        out["chunked"]["cpu_baseline"] = cpu_baseline_chunked(xc, cc)
        log("[bench] cpu baseline: float64 oracle on a sample of the FP8 chunked-prefill workload")
        out["chunked_fp8"]["cpu_baseline"] = cpu_baseline_chunked_fp8(xc, cc, ck8.cpu().numpy(), cv8.cpu().numpy(),
                                                                      KS8, VS8)
        log("[bench] cpu baseline: float64 oracle on a sample of the rotary chunked-prefill workload")
        out["chunked_rope"]["cpu_baseline"] = cpu_baseline_chunked(xc, cc, rope=W.rope_table(16384, cc.D))
        log("[bench] cpu baseline: float64 oracle on the linear layers")
        out["gemm"]["cpu_baseline"] = cpu_baseline_gemm(gx)
        for key, case in (("bert_prefill", W.BERT), ("llama_prefill", W.LLAMA)):
            log(f"[bench] cpu baseline: float64 oracle on the whole {key} workload")
            out[key]["cpu_baseline"] = cpu_baseline_small_prefill(small[key][1], case)
        log("[bench] parity of the timed calls' outputs against the oracle (sampled)")
        pcalls = {name: call for name, call, _ in parts}
        chunk_calls = [("chunked", pcalls["chunked_prefill"]), ("chunked_rope", pcalls["chunked_prefill_rope"]),
                       ("chunked_fp8", pcalls["chunked_prefill_fp8"])]
        out["parity_on_timed_buffers"] = parity_on_timed_buffers(
            ta, torch, np, W, pc, xp, o, lse, xp8, (QS8, KSP8, VSP8), o8, lse8, dc, xd, do, dlse, xd8, KS8, VS8,
            do8, dlse8, cc, xc, rope_tab, chunk_calls, co, clse, ck8.cpu().numpy(), cv8.cpu().numpy(), gx, gdev)
        from oracle import oracle as O
        pr = out["parity_on_timed_buffers"]
        for key, case in (("bert_prefill", W.BERT), ("llama_prefill", W.LLAMA)):
            _, xs, os_, ls_ = small[key]
            orf, lrf = O.prefill(xs["q"], xs["k"], xs["v"], case.scale, case.causal, xs["seq_lens"])
            valid = np.isfinite(lrf)
            tol = 2e-3 if case.dtype == "fp16" else 1e-2
            og, lg = os_.float().cpu().numpy(), ls_.cpu().numpy()
            pr[key] = _parity(og[valid], orf[valid], lg[valid], lrf[valid], tol=tol, strict=True,
                              what="every valid row of the timed call's output")
            pr[key]["padding_rows_exact"] = bool((og[~valid] == 0).all() and np.isneginf(lg[~valid]).all())
            pr[key]["ok"] = pr[key]["ok"] and pr[key]["padding_rows_exact"]
        pr["all_ok"] = all(v.get("ok", False) for v in pr.values() if isinstance(v, dict))
        log(f"[bench] parity on timed buffers: all ok = {out['parity_on_timed_buffers']['all_ok']}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
