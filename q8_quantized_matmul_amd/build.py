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
SOURCES = ["api.hip", "quantize.hip", "matvec.hip", "moe.hip", "gemm.hip", "skinny.hip", "probe.hip"]

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


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the gfx feature flag; drop that one warning.
    noise = [l for l in res.stderr.splitlines()
             if "packed-fp32-ops" not in l and "is not a recognized feature" not in l
             and l.strip() != "1 warning generated."]
    if res.returncode != 0:
        sys.stderr.write(res.stderr)
        raise RuntimeError("hipcc failed building libq8_0.so")
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
