"""Shared helpers for the GPU parity tests: oracle calls on torch tensors and
the element-wise acceptance check.

Acceptance (stated for the Q8_0 path): quantized activations bit-exact;
block sums S_b bit-exact; fp32 outputs |gpu - oracle| <= 1e-5 * mag + 1e-6
with mag = sum_b |d_w d_x S_b| (computed by the oracle in float64).  NaN
outputs must sit at the same places on both sides.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

REL_TOL = 1e-5
ABS_TOL = 1e-6


def say(*msg):
    print(*msg, flush=True)
    sys.stdout.flush()


def cpu_u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").contiguous().numpy()


def oracle_quantize(x: torch.Tensor) -> np.ndarray:
    return oracle.quantize(x.detach().to("cpu", torch.float32).contiguous().numpy())


def assert_close(gpu, ref, mag, where=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    mag = np.asarray(mag, dtype=np.float64)
    assert gpu.shape == ref.shape, (where, gpu.shape, ref.shape)
    nan_g, nan_r = np.isnan(gpu), np.isnan(ref)
    assert np.array_equal(nan_g, nan_r), f"{where}: NaN pattern differs ({nan_g.sum()} vs {nan_r.sum()})"
    fin = ~nan_r
    err = np.abs(gpu[fin] - ref[fin])
    bound = REL_TOL * mag[fin] + ABS_TOL
    bad = err > bound
    if bad.any():
        i = np.argmax(err / bound)
        raise AssertionError(f"{where}: {int(bad.sum())} of {err.size} outside tolerance; worst "
                             f"err {err[i]:.3e} bound {bound[i]:.3e} gpu {gpu[fin][i]!r} ref {ref[fin][i]!r}")
    return float((err / np.maximum(mag[fin], 1e-30)).max()) if err.size else 0.0
