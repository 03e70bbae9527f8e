"""Independent numpy restatements used to pin the oracle (test-only).

These do not call the oracle and share no code with it: binary16 comes from
numpy's own float16 conversion, rounding-half-away is computed in float64 as
trunc(r + copysign(0.5, r)), dot products are numpy float64 / int64 matmuls.
"""
from __future__ import annotations

import numpy as np

QK = 32
BB = 34


def split_blocks(blocks: np.ndarray, k: int):
    """uint8 [rows][k/32*34] -> (scale bits uint16 [rows][nb], q int8 [rows][nb][32])."""
    rows = blocks.shape[0]
    nb = k // QK
    b = blocks.reshape(rows, nb, BB)
    bits = b[:, :, 0].astype(np.uint16) | (b[:, :, 1].astype(np.uint16) << 8)
    q = b[:, :, 2:].view(np.int8)
    return bits, q


def join_blocks(bits: np.ndarray, q: np.ndarray) -> np.ndarray:
    rows, nb = bits.shape
    out = np.empty((rows, nb, BB), dtype=np.uint8)
    out[:, :, 0] = (bits & 0xFF).astype(np.uint8)
    out[:, :, 1] = (bits >> 8).astype(np.uint8)
    out[:, :, 2:] = q.view(np.uint8)
    return out.reshape(rows, nb * BB)


def scales_f64(bits: np.ndarray) -> np.ndarray:
    return bits.astype(np.uint16).view(np.float16).astype(np.float64)


def dequant_f64(blocks: np.ndarray, k: int) -> np.ndarray:
    bits, q = split_blocks(blocks, k)
    return (scales_f64(bits)[:, :, None] * q.astype(np.float64)).reshape(blocks.shape[0], k)


def quantize_ref(x: np.ndarray) -> np.ndarray:
    """The block rule with numpy primitives (finite inputs, normal scales)."""
    x = np.asarray(x, dtype=np.float32)
    rows, k = x.shape
    nb = k // QK
    xb = x.reshape(rows, nb, QK)
    amax = np.max(np.abs(xb), axis=2)
    d = (amax / np.float32(127.0)).astype(np.float32)        # fp32 IEEE division
    safe = np.where(d > 0, d, np.float32(1.0))
    r = (xb / safe[:, :, None]).astype(np.float32)           # fp32 IEEE division
    r64 = r.astype(np.float64)
    qf = np.trunc(r64 + np.copysign(0.5, r64))               # half away from zero
    qf = np.clip(qf, -127, 127)
    q = np.where(d[:, :, None] > 0, qf, 0).astype(np.int8)
    bits = d.astype(np.float16).view(np.uint16)              # numpy RNE binary16
    bits = np.where(d > 0, bits, 0).astype(np.uint16)
    return join_blocks(bits, q)


def matmul_f64(w_blocks: np.ndarray, x_blocks: np.ndarray, k: int) -> np.ndarray:
    """Brute force: dequantize both sides to float64, then a float64 matmul."""
    return dequant_f64(x_blocks, k) @ dequant_f64(w_blocks, k).T


def blocksums_i64(w_blocks: np.ndarray, x_blocks: np.ndarray, k: int) -> np.ndarray:
    _, qw = split_blocks(w_blocks, k)
    _, qx = split_blocks(x_blocks, k)
    return np.einsum("tbi,obi->tob", qx.astype(np.int64), qw.astype(np.int64))


def mag_f64(w_blocks: np.ndarray, x_blocks: np.ndarray, k: int) -> np.ndarray:
    bw, _ = split_blocks(w_blocks, k)
    bx, _ = split_blocks(x_blocks, k)
    s = blocksums_i64(w_blocks, x_blocks, k).astype(np.float64)
    sc = scales_f64(bx)[:, None, :] * scales_f64(bw)[None, :, :]
    return np.sum(np.abs(sc * s), axis=2)


def f32_ulp(v: np.ndarray) -> np.ndarray:
    v = np.abs(np.asarray(v, dtype=np.float32))
    return np.spacing(v).astype(np.float64)
