"""Compile libkda.so (all HIP sources in csrc/) for gfx950 with hipcc, in-tree.

Usage: python -m linear_attention_chunkwise_amd.build   (or build.build()).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkda.so")
# debug build of the same sources in which every kernel first fills its LDS with NaN
# (-DKDA_POISON_LDS); loaded only by the test that looks for reads of unwritten LDS
POISON_LIB = os.path.join(HERE, "libkda_poison.so")
ARCH = os.environ.get("KDA_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-variable", "-Wno-uninitialized",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, poison: bool = False) -> str:
    """Always recompile (the build check must compile every time it is called).  poison: the
    LDS-poisoning debug build (POISON_LIB) instead of the library."""
    out = POISON_LIB if poison else LIB
    extra = ["-DKDA_POISON_LDS"] if poison else []
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["hipcc", *HIPCC_FLAGS, *extra, f"-I{INCLUDE}", f"-I{CSRC}", *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
    sys.exit(0)
