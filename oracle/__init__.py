"""CPU oracle for the Q8_0 quantized matmul (TEST INFRASTRUCTURE ONLY).

Thin ctypes wrapper over ``q8o.c``: a plain, slow C restatement of the
method (single-threaded unless ``set_threads`` asks for OpenMP threads over
independent outputs, which gives bit-identical results) (see the header of ``q8o.c`` for the passages it
follows and the readings it takes).  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP library, and the HIP library never calls it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q8o.c")
_LIB = os.path.join(_HERE, "libq8o.so")

BLOCK_ELEMS = 32
BLOCK_BYTES = 34

_lib = None


def build() -> str:
    """Compile q8o.c into oracle/libq8o.so with gcc (always recompiles)."""
    cmd = [
        "gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
        "-fPIC", "-shared", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.q8o_set_threads.argtypes = [ctypes.c_int]
    lib.q8o_set_threads.restype = None
    lib.q8o_get_threads.argtypes = []
    lib.q8o_get_threads.restype = ctypes.c_int
    lib.q8o_f16_from_f32.argtypes = [ctypes.c_float]
    lib.q8o_f16_from_f32.restype = ctypes.c_uint16
    lib.q8o_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.q8o_f16_to_f64.restype = ctypes.c_double
    lib.q8o_quantize.argtypes = [vp, i64, i64, vp]
    lib.q8o_quantize.restype = ctypes.c_int
    lib.q8o_matmul.argtypes = [vp, i64, i64, vp, i64, vp, vp, vp]
    lib.q8o_matmul.restype = ctypes.c_int
    lib.q8o_moe_grouped.argtypes = [vp, i32, i64, i64, vp, i32, vp, i32, i64, vp, vp]
    lib.q8o_moe_grouped.restype = ctypes.c_int
    lib.q8o_swiglu.argtypes = [vp, vp, i64, ctypes.c_float, vp]
    lib.q8o_swiglu.restype = None
    lib.q8o_moe_combine.argtypes = [vp, vp, i64, i32, i64, vp, vp]
    lib.q8o_moe_combine.restype = None
    _lib = lib
    return lib


def host_threads() -> int:
    """Threads for the oracle on this host: OMP_NUM_THREADS if set (the
    share of the host a job may use), else every core, at most 16."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    n = int(env) if env.isdigit() and int(env) > 0 else (os.cpu_count() or 1)
    return max(1, min(n, 16))


def set_threads(n: int) -> None:
    """OpenMP threads for the loops over independent outputs (1 = serial)."""
    _load().q8o_set_threads(int(n))


def get_threads() -> int:
    return int(_load().q8o_get_threads())


class threads:
    """Context manager: run the oracle on n threads inside the block."""

    def __init__(self, n: int | None = None):
        self.n = host_threads() if n is None else n

    def __enter__(self):
        self.prev = get_threads()
        set_threads(self.n)
        return self

    def __exit__(self, *exc):
        set_threads(self.prev)
        return False


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def f16_from_f32(v: float) -> int:
    """binary16 bits of fp32 v, round to nearest even (written from IEEE 754)."""
    return int(_load().q8o_f16_from_f32(float(np.float32(v))))


def f16_to_f64(bits: int) -> float:
    return float(_load().q8o_f16_to_f64(int(bits)))


def quantize(x: np.ndarray) -> np.ndarray:
    """x: fp32 [rows][k] -> uint8 [rows][k/32*34] Q8_0 blocks."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    rows, k = x.shape
    if k % BLOCK_ELEMS:
        raise ValueError("k must be a multiple of 32")
    out = np.empty((rows, k // BLOCK_ELEMS * BLOCK_BYTES), dtype=np.uint8)
    rc = _load().q8o_quantize(_ptr(x), rows, k, _ptr(out))
    if rc != 0:
        raise ValueError(f"q8o_quantize failed ({rc})")
    return out


def matmul(w: np.ndarray, xq: np.ndarray, in_dim: int, *, want_mag: bool = True,
           want_blocksums: bool = False):
    """w: uint8 [out_dim][row_bytes], xq: uint8 [n_tok][row_bytes].

    Returns (out fp32 [n_tok][out_dim], mag fp64 or None, blocksums int32
    [n_tok][out_dim][nb] or None)."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    nb = in_dim // BLOCK_ELEMS
    row_bytes = nb * BLOCK_BYTES
    out_dim = w.size // row_bytes if row_bytes else 0
    n_tok = xq.size // row_bytes if row_bytes else 0
    out = np.empty((n_tok, out_dim), dtype=np.float32)
    mag = np.empty((n_tok, out_dim), dtype=np.float64) if want_mag else None
    bs = np.empty((n_tok, out_dim, nb), dtype=np.int32) if want_blocksums else None
    rc = _load().q8o_matmul(
        _ptr(w), in_dim, out_dim, _ptr(xq), n_tok, _ptr(out),
        _ptr(mag) if mag is not None else None,
        _ptr(bs) if bs is not None else None)
    if rc != 0:
        raise ValueError(f"q8o_matmul failed ({rc})")
    return out, mag, bs


def moe_grouped(expert_w, selected: np.ndarray, xq: np.ndarray, in_dim: int,
                out_dim: int, x_rows: int, want_mag: bool = True):
    """expert_w: list of uint8 [out_dim][row_bytes] arrays (index = expert id).

    Returns (out fp32 [n_tok][n_used][out_dim], mag or None, invalid_count)."""
    selected = np.ascontiguousarray(selected, dtype=np.int32)
    n_tok, n_used = selected.shape
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    mats = [np.ascontiguousarray(m, dtype=np.uint8) for m in expert_w]
    table = (ctypes.c_void_p * len(mats))(*[m.ctypes.data for m in mats])
    out = np.empty((n_tok, n_used, out_dim), dtype=np.float32)
    mag = np.empty((n_tok, n_used, out_dim), dtype=np.float64) if want_mag else None
    rc = _load().q8o_moe_grouped(
        ctypes.cast(table, ctypes.c_void_p), len(mats), in_dim, out_dim,
        _ptr(selected), n_used, _ptr(xq), x_rows, n_tok, _ptr(out),
        _ptr(mag) if mag is not None else None)
    if rc < 0:
        raise ValueError(f"q8o_moe_grouped failed ({rc})")
    return out, mag, rc


def swiglu(gate: np.ndarray, up: np.ndarray, clamp: float = 0.0) -> np.ndarray:
    """mid = silu(gate) * up elementwise (optional clamp), fp32 of the double."""
    gate = np.ascontiguousarray(gate, dtype=np.float32)
    up = np.ascontiguousarray(up, dtype=np.float32)
    assert gate.shape == up.shape
    mid = np.empty_like(gate)
    _load().q8o_swiglu(_ptr(gate), _ptr(up), gate.size, float(clamp), _ptr(mid))
    return mid


def moe_combine(y: np.ndarray, weights: np.ndarray, want_mag: bool = True):
    """y fp32 [n_tok][n_used][dim], weights fp32 [n_tok][n_used] ->
    (out fp32 [n_tok][dim], mag float64 or None)."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    weights = np.ascontiguousarray(weights, dtype=np.float32)
    n_tok, n_used, dim = y.shape
    assert weights.shape == (n_tok, n_used)
    out = np.empty((n_tok, dim), dtype=np.float32)
    mag = np.empty((n_tok, dim), dtype=np.float64) if want_mag else None
    _load().q8o_moe_combine(_ptr(y), _ptr(weights), n_tok, n_used, dim, _ptr(out),
                            _ptr(mag) if mag is not None else None)
    return out, mag
