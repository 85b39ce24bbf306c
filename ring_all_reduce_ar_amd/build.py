"""Build liballreduce.so in-tree with hipcc for gfx950.

    python ring_all_reduce_ar_amd/build.py

(Run it as a file, not with -m: importing the package loads the library,
which may be missing or stale before the build.)

Flags: -O3; no FMA contraction (-ffp-contract=off) so sums and products are
rounded exactly as written; packed-fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops); only the ar_* symbols
exported (-fvisibility=hidden).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liballreduce.so")
OBJDIR = os.path.join(PKG, "_build")
# Two translation units per dtype (ring kernels, tree kernels: the heavy
# template instantiations), the dtype switch / copy kernels and the C ABI;
# compiled in parallel, then linked.
SOURCES = [os.path.join(CSRC, f) for f in
           ("dtype_f32.hip", "dtype_f16.hip", "dtype_bf16.hip", "dtype_i32.hip", "tree_f32.hip", "tree_f16.hip",
            "tree_bf16.hip", "tree_i32.hip", "kernels.hip", "noalloc.hip", "api.cpp")]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-command-line-argument",
         f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc_compile(src: str, obj: str):
    return [HIPCC, *FLAGS, "-c", "-o", obj, src]


def hipcc_link(objs, out: str):
    return [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out, *objs]


def _stale(src: str, obj: str) -> bool:
    if not os.path.exists(obj):
        return True
    deps = [src] + [os.path.join(CSRC, h) for h in os.listdir(CSRC) if h.endswith(".h")] + \
           [os.path.join(INCLUDE, h) for h in os.listdir(INCLUDE)]
    return max(os.path.getmtime(d) for d in deps) > os.path.getmtime(obj)


def build(verbose: bool = False, jobs: int = 0, incremental: bool = False) -> str:
    """Compile every source into liballreduce.so (always recompiles unless
    `incremental`, which skips objects newer than their source and headers)."""
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 16)
    objs = [os.path.join(OBJDIR, os.path.basename(s) + ".o") for s in SOURCES]
    pending = [(s, o) for s, o in zip(SOURCES, objs) if not incremental or _stale(s, o)]
    running = []
    failed = []
    while pending or running:
        while pending and len(running) < jobs:
            src, obj = pending.pop(0)
            cmd = hipcc_compile(src, obj)
            if verbose:
                print(" ".join(cmd), flush=True)
            running.append((src, subprocess.Popen(cmd)))
        src, proc = running.pop(0)
        if proc.wait() != 0:
            failed.append(src)
    if failed:
        raise subprocess.CalledProcessError(1, f"hipcc failed for {failed}")
    tmp = f"{LIB}.tmp{os.getpid():x}"  # per-process name: concurrent builds rename atomically
    subprocess.run(hipcc_link(objs, tmp), check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, incremental="--incremental" in sys.argv))
