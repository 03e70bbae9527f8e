"""Compiler resource report of every gfx950 kernel (CPU only: hipcc
cross-compiles): no kernel on a timed path may use scratch memory.

A register spill turns into per-lane scratch traffic through the caches and
HBM (a 4-VGPR spill in the multi-matrix decode kernel once added 2 MB of
writes per launch), so the device code of every source is compiled with the
library's flags and the compiler's per-kernel resource remarks are checked.
Only the debug instantiations that also store the block sums S_b may use
scratch: they are for checking, not timing.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from q8_quantized_matmul_amd import build

# Mangled names of the block-sum (debug) instantiations: the bool that
# selects the S_b output is true.
DEBUG = [
    re.compile(r"gemm_t4_kernelILb1E"),
    re.compile(r"gemm_lds_kernelILb1E"),
    re.compile(r"gemm_kernelILi\d+ELi\d+ELi\d+ELb1E"),
    # matvec_kernel<LPR, WPR, CPW, RG, GROUPED, STORE_S, STAGED>
    re.compile(r"matvec_kernelILi\d+ELi\d+ELi\d+ELi\d+ELb[01]ELb1E"),
    re.compile(r"generic_(grouped_)?kernelILb1E"),
    re.compile(r"skinny_kernel.*ELb1E"),
]


def _resources(src, out_dir):
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-shared", "-Wall")]
    cmd = [build.hipcc(), *flags, "-I", build.CSRC, "-I", os.path.join(build.ROOT, "include"),
           "--cuda-device-only", "-c", "-o", os.path.join(out_dir, os.path.basename(src) + ".o"),
           "-Rpass-analysis=kernel-resource-usage", src]
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def _parse(text):
    """{kernel name: scratch bytes per lane} from the resource remarks."""
    out, name = {}, None
    for line in text.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name:
            out[name] = int(m.group(1))
    return out


@pytest.mark.skipif(shutil.which(build.hipcc()) is None and not os.path.exists(build.hipcc()),
                    reason="hipcc not available")
def test_no_scratch_outside_debug_kernels():
    with tempfile.TemporaryDirectory() as tmp:
        procs = [(s, _resources(os.path.join(build.CSRC, s), tmp)) for s in build.SOURCES]
        found = {}
        for s, p in procs:
            _, err = p.communicate()
            assert p.returncode == 0, f"{s}: hipcc failed\n{err[-2000:]}"
            found.update(_parse(err))
    assert len(found) > 50, "no resource remarks parsed"
    spilling = {n: b for n, b in found.items()
                if b > 0 and not any(d.search(n) for d in DEBUG)}
    assert not spilling, f"kernels using scratch: {spilling}"
