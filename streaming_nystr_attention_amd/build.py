"""Build the gfx950 HIP library ``lib/libo1.so`` in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libo1.so")
SOURCES = ["o1_api.hip", "o1_decode.hip", "o1_prefill.hip", "o1_exact.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr[-8000:]}")


def build(verbose: bool = False) -> str:
    """Compile every HIP source (in parallel, one object each) and link them
    into one shared library (always recompiles)."""
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(LIB_DIR, exist_ok=True)
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tag = f".tmp{os.getpid()}"
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    objs = [os.path.join(LIB_DIR, os.path.splitext(s)[0] + tag + ".o") for s in SOURCES]
    jobs = [[hipcc, *compile_flags, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    try:
        with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as pool:
            for f in [pool.submit(_run, j, verbose) for j in jobs]:
                f.result()
        tmp = LIB + tag
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
