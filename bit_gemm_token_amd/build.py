"""Build libbgt.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbgt.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no contraction: every float op is the one written (fma only where explicit)
    "-ffp-contract=off",
    # keep the compiler from forming packed fp32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
BUILD_DIR = os.path.join(ROOT, "_build")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd[-3:]))


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libbgt.so (always recompiles): one hipcc
    per translation unit in parallel (each launches only its own kernels), then
    one link."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, os.path.basename(src) + ".o") for src in sources()]
    cmds = [[HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
            for src, obj in zip(sources(), objs)]
    workers = max(1, min(len(cmds), os.cpu_count() or 1))
    try:
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as pool:
            for f in [pool.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = LIB + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(BUILD_DIR, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
