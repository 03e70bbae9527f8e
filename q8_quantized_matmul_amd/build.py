"""Build libq8_0.so (the gfx950 HIP library behind include/q8_0.h) in-tree.

Run as ``python q8_quantized_matmul_amd/build.py``.  Always recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libq8_0.so")
SOURCES = ["api.hip", "quantize.hip", "matvec.hip", "moe.hip", "gemm.hip", "skinny.hip", "probe.hip",
           "debug.hip"]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU forms.
# No fast-math: the quantizer relies on IEEE division and roundf.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-shared", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose, what):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the gfx feature flag; drop that one warning.
    noise = [l for l in res.stderr.splitlines()
             if "packed-fp32-ops" not in l and "is not a recognized feature" not in l
             and l.strip() != "1 warning generated."]
    if res.returncode != 0:
        sys.stderr.write(res.stderr)
        raise RuntimeError(f"hipcc failed building {what}")
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link the library."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    jobs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        jobs.append((obj, [hipcc(), *compile_flags, *inc, "-c", "-o", obj,
                           os.path.join(CSRC, src)]))
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(workers) as pool:
        list(pool.map(lambda j: _run(j[1], verbose, j[0]), jobs))
    tmp = LIB + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
          *[obj for obj, _ in jobs]], verbose, "libq8_0.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
