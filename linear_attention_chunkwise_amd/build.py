"""Compile libkda.so (all HIP sources in csrc/) for gfx950 with hipcc, in-tree.

Each source is compiled to an object on its own (in parallel, under _build/ at the repository
root), then the objects are linked into the shared library.

Usage: python -m linear_attention_chunkwise_amd.build   (or build.build()).
"""
from __future__ import annotations

import concurrent.futures
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
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-variable", "-Wno-uninitialized",
]
COMPILE_FLAGS = [f for f in HIPCC_FLAGS if f != "-shared"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _jobs(poison: bool):
    """(command, object path) for each source of one library variant."""
    extra = ["-DKDA_POISON_LDS"] if poison else []
    d = os.path.join(BUILD_DIR, "poison" if poison else "lib")
    os.makedirs(d, exist_ok=True)
    out = []
    for src in sources():
        obj = os.path.join(d, os.path.basename(src)[:-4] + ".o")
        out.append((["hipcc", *COMPILE_FLAGS, *extra, f"-I{INCLUDE}", f"-I{CSRC}", "-c", src, "-o", obj], obj))
    return out


def _link(objs, out: str, verbose: bool) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_variants(variants=(False, True), verbose: bool = False) -> list:
    """Always recompile (the build check must compile every time it is called): every source of
    every requested variant (False: the library, True: the LDS-poisoning debug build) at once."""
    jobs = {p: _jobs(p) for p in variants}
    flat = [j for p in variants for j in jobs[p]]
    workers = max(1, min(len(flat), os.cpu_count() or 1, 8))

    def run(job):
        cmd, _ = job
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)

    with concurrent.futures.ThreadPoolExecutor(workers) as pool:
        for f in [pool.submit(run, j) for j in flat]:
            f.result()
    return [_link([o for _, o in jobs[p]], POISON_LIB if p else LIB, verbose) for p in variants]


def build(verbose: bool = False, poison: bool = False) -> str:
    """One variant: the library (poison False) or the LDS-poisoning debug build."""
    return build_variants((poison,), verbose)[0]


if __name__ == "__main__":
    build_variants(verbose=True)
    print(LIB)
