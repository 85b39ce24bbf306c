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
SOURCES = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "kernels.hip")]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def hipcc_command(out: str, extra=()):
    return [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
            "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}", *extra,
            "-o", out, *SOURCES]


def build(verbose: bool = False) -> str:
    """Compile every source into liballreduce.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
