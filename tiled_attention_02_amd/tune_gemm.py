"""Exhaustive configuration search for attn_gemm_splitk, one weight shape at a time.

The SplitK GEMM of the linear layers is tuned per weight shape by trying
every configuration (comemg.com, "天下苦英偉達久矣！PyTorch免CUDA加速推理，
Triton時代要來？", section "GEMM 內核調優"). This script times every
(rows, waves, unroll) configuration of attn_gemm_splitk_cfg on the current GPU
for each shape and prints the fastest, as entries for the library's table of
tuned configurations.

Each timed call starts with the weight evicted from the caches (a read pass
over 1 GiB), as in a decode step, where a layer's weight was last read a whole
model earlier.

Usage: python -m tiled_attention_02_amd.tune_gemm [--M 2] [--dtype bf16] [--reps 20] [N,K ...]
(no shapes: the Llama3-8B / Granite-8B linear layers).
"""
from __future__ import annotations

import argparse
import itertools
import json
import sys

DEFAULT_SHAPES = {
    "qkv_proj": (6144, 4096),
    "o_proj": (4096, 4096),
    "gate_up_proj": (28672, 4096),
    "down_proj": (4096, 14336),
}
ROWS = (16, 32)
WAVES = (1, 2, 4, 6, 8, 12, 16)
UNROLL = (1, 2, 4, 8)


def time_config(ta, torch, x, w, y, cfg, reps, flush_rows, flush_dst):
    times = []
    for _ in range(reps):
        torch.sum(flush_rows, dim=1, out=flush_dst)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        ta.attn_gemm_splitk(x, w, out=y, config=cfg)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    times.sort()
    return times[len(times) // 2]  # median, microseconds


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--M", type=int, default=2)
    ap.add_argument("--dtype", choices=("bf16", "fp16"), default="bf16")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("shapes", nargs="*", help="N,K pairs")
    args = ap.parse_args(argv)
    import torch
    import tiled_attention_02_amd as ta
    dt = torch.bfloat16 if args.dtype == "bf16" else torch.float16
    shapes = {f"{n}x{k}": (n, k) for n, k in (tuple(map(int, s.split(","))) for s in args.shapes)} \
        if args.shapes else DEFAULT_SHAPES
    flush_rows = torch.ones((1 << 28) // 4096, 4096, dtype=torch.float32, device="cuda")
    flush_dst = torch.empty(flush_rows.shape[0], dtype=torch.float32, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(0)
    results = {}
    for name, (N, K) in shapes.items():
        x = torch.randn((args.M, K), generator=gen, device="cuda").to(dt)
        w = (torch.randn((N, K), generator=gen, device="cuda") / K ** 0.5).to(dt)
        y = torch.empty((args.M, N), dtype=dt, device="cuda")
        rows = []
        for cfg in itertools.product(ROWS, WAVES, UNROLL):
            us = time_config(ta, torch, x, w, y, cfg, args.reps, flush_rows, flush_dst)
            rows.append((us, cfg))
            print(f"[tune] {name} N={N} K={K} cfg={cfg}: {us:.2f} us", flush=True)
        rows.sort()
        best_us, best = rows[0]
        default_us = time_config(ta, torch, x, w, y, None, args.reps, flush_rows, flush_dst)
        gbs = (N * K + args.M * K + args.M * N) * 2 / best_us * 1e-3
        results[name] = dict(N=N, K=K, best=best, best_us=best_us, best_GBs=gbs, table_us=default_us,
                             top5=[(u, c) for u, c in rows[:5]])
        print(f"[tune] {name}: best {best} {best_us:.2f} us ({gbs:.0f} GB/s); "
              f"current library choice {default_us:.2f} us", flush=True)
        del x, w, y
    print("// tuned entries {N, K, {rows, waves, unroll}}")
    for name, r in results.items():
        print(f"    {{{r['N']}, {r['K']}, {{{r['best'][0]}, {r['best'][1]}, {r['best'][2]}}}}},  // {name}")
    print(json.dumps(results))
    return 0


if __name__ == "__main__":
    sys.exit(main())
