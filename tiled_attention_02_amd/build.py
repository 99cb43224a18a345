"""Build libattn.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m tiled_attention_02_amd.build   (or build() from Python)
The library is written next to this file so it travels with the source tree.
A second library, libattn_single.so, is the same code with the prefill's
debug key loop (ATTN_SINGLE_BUFFER: one K and one V buffer, nothing
overlapped); the tests compare its output with the pipelined kernel's bit for
bit, which would expose a staging race.
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libattn.so")
LIB_SINGLE = os.path.join(HERE, "libattn_single.so")
SOURCES = ["libattn.cpp", "prefill_fwd.hip", "decode_paged.hip", "paged_cache.hip", "gemm_splitk.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libattn")


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc link failed")
    os.replace(tmp, out)


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source for gfx950 (in parallel), link libattn.so and libattn_single.so; returns the
    path of libattn.so."""
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    common = [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              f"-I{os.path.join(ROOT, 'include')}", *extra]
    jobs = []  # (source, object, extra flags)
    for src in SOURCES:
        jobs.append((src, os.path.join(bdir, os.path.splitext(src)[0] + ".o"), []))
    jobs.append(("prefill_fwd.hip", os.path.join(bdir, "prefill_fwd_single.o"), ["-DATTN_SINGLE_BUFFER"]))
    procs = []
    for src, obj, flags in jobs:
        cmd = [hipcc(), *common, *flags, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(out)
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed on {', '.join(failed)}")
    objs = [obj for _, obj, flags in jobs if not flags]
    _link(objs, LIB)
    single = [o if not o.endswith("prefill_fwd.o") else os.path.join(bdir, "prefill_fwd_single.o") for o in objs]
    _link(single, LIB_SINGLE)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
