"""Pins for the oracle's binary16 conversion and block quantizer (CPU only).

The rule comes from ds4-learning "Part 3: 模型架构", section 2 (the Q8_K row
quantizer listing: amax, scale = amax/127, q = roundf(x/scale)), applied per
32-value block with a binary16 scale (Q8_0 block size from "Part 6: 代码走读",
trace 3).  Each check below is fixed by something other than the oracle:
hand-derived values, numpy's own binary16 conversion, or an invariant of the
rule.
"""
import math
import os

import numpy as np
import pytest

import oracle
from tests import refmath

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantize_closed_form.txt")


def _parse_float(tok: str) -> float:
    if tok.startswith(("0x", "-0x")):
        return float.fromhex(tok)
    return float(tok)


def _golden_cases():
    cases = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, bits, xs, qs = [p.strip() for p in line.split(";")]
            x = np.zeros(32, dtype=np.float32)
            vals = [_parse_float(t) for t in xs.split()]
            x[: len(vals)] = np.array(vals, dtype=np.float32)
            q = np.zeros(32, dtype=np.int8)
            qv = [int(t) for t in qs.split()]
            q[: len(qv)] = qv
            cases.append((name, int(bits, 16), x, q))
    return cases


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c[0])
def test_golden_closed_form(case):
    _, bits, x, q = case
    blk = oracle.quantize(x[None, :])[0]
    assert int(blk[0]) | (int(blk[1]) << 8) == bits
    np.testing.assert_array_equal(blk[2:].view(np.int8), q)


# ---- binary16 ----------------------------------------------------------------

def test_f16_to_f64_exhaustive_against_numpy():
    for bits in range(1 << 16):
        ref = float(np.array([bits], dtype=np.uint16).view(np.float16)[0])
        got = oracle.f16_to_f64(bits)
        if math.isnan(ref):
            assert math.isnan(got)
        else:
            assert got == ref and math.copysign(1, got) == math.copysign(1, ref), hex(bits)


def _f16_bits_numpy(v: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return v.astype(np.float32).astype(np.float16).view(np.uint16)


def test_f16_from_f32_edges_against_numpy():
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.996, 65520.0, 65536.0, 1e30,
            2.0 ** -14, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26,
            2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11,
            1.0 + 2.0 ** -11 + 2.0 ** -20, 2047.5, 2048.5, 2049.0, 4095.0,
            float("inf"), float("-inf"), 1e-45, 5.96e-8, 6.1e-5, 0.1, 1 / 3.0]
    for v in vals:
        v32 = np.float32(v)
        ref = int(_f16_bits_numpy(np.array([v32]))[0])
        assert oracle.f16_from_f32(v32) == ref, (v, hex(ref))


def test_f16_from_f32_random_bit_patterns_against_numpy():
    rng = np.random.default_rng(1234)
    # Random fp32 bit patterns concentrated on the binary16 range and beyond.
    exps = rng.integers(90, 160, size=60000, dtype=np.uint32)
    mant = rng.integers(0, 1 << 23, size=60000, dtype=np.uint32)
    sign = rng.integers(0, 2, size=60000, dtype=np.uint32)
    u = (sign << 31) | (exps << 23) | mant
    v = u.view(np.float32)
    ref = _f16_bits_numpy(v)
    got = np.array([oracle.f16_from_f32(x) for x in v], dtype=np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_f16_from_f32_halfway_points_round_to_even():
    # Exact midpoints between neighbouring binary16 values, normal and subnormal.
    for bits in list(range(0x0001, 0x0400, 37)) + list(range(0x0400, 0x7BFF, 331)):
        lo = float(np.array([bits], dtype=np.uint16).view(np.float16)[0])
        hi = float(np.array([bits + 1], dtype=np.uint16).view(np.float16)[0])
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2  # representable in fp32
        expect = bits if bits % 2 == 0 else bits + 1
        assert oracle.f16_from_f32(mid) == expect
        assert oracle.f16_from_f32(-mid) == expect | 0x8000


# ---- quantizer ---------------------------------------------------------------

def _rand_blocks(seed, rows, k, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((rows, k)) * scale).astype(np.float32)


@pytest.mark.parametrize("scale", [1.0, 0.02, 1e-3, 300.0])
def test_quantize_matches_numpy_rule(scale):
    x = _rand_blocks(7, 64, 512, scale)
    x[3, 40] *= 50.0
    x[5, :32] = 0.0
    np.testing.assert_array_equal(oracle.quantize(x), refmath.quantize_ref(x))


def test_quantize_ties_round_away_from_zero():
    # x = (k + 1/2) * d with d a power of two: the quotient is an exact tie.
    d = np.float32(2.0 ** -5)
    ks = np.arange(-63, 63)
    for start in range(0, len(ks), 31):
        x = np.zeros(32, dtype=np.float32)
        x[0] = 127 * d
        chunk = ks[start:start + 31]
        x[1:1 + len(chunk)] = (chunk + 0.5) * d
        q = oracle.quantize(x[None, :])[0, 2:].view(np.int8)
        expect = np.where(chunk >= 0, chunk + 1, chunk)  # away from zero
        np.testing.assert_array_equal(q[1:1 + len(chunk)], expect)


def test_quantize_invariants():
    x = _rand_blocks(11, 128, 256)
    blk = oracle.quantize(x)
    bits, q = refmath.split_blocks(blk, 256)
    # Every nonzero block reaches |q| = 127 exactly once per amax element.
    assert np.all(np.max(np.abs(q.astype(np.int32)), axis=2) == 127)
    # Sign symmetry, bit for bit.
    bn, qn = refmath.split_blocks(oracle.quantize(-x), 256)
    np.testing.assert_array_equal(bn, bits)
    np.testing.assert_array_equal(qn, -q)
    # Power-of-two equivariance while the scale stays a normal binary16.
    for p in (-3, 2, 5):
        b2, q2 = refmath.split_blocks(oracle.quantize(x * np.float32(2.0 ** p)), 256)
        np.testing.assert_array_equal(q2, q)
        np.testing.assert_array_equal(refmath.scales_f64(b2), refmath.scales_f64(bits) * 2.0 ** p)


def test_quantize_reconstruction_error_bound():
    # |x - d16*q| <= d32/2 (rounding of q) + |d32 - d16|*127 (scale rounding).
    x = _rand_blocks(3, 32, 1024)
    blk = oracle.quantize(x)
    deq = refmath.dequant_f64(blk, 1024).reshape(32, 32, 32)
    xb = x.astype(np.float64).reshape(32, 32, 32)
    d32 = (np.max(np.abs(x.reshape(32, 32, 32)), axis=2) / np.float32(127)).astype(np.float64)
    bits, _ = refmath.split_blocks(blk, 1024)
    d16 = refmath.scales_f64(bits)
    bound = d32 / 2 * (1 + 1e-6) + np.abs(d32 - d16) * 127
    assert np.all(np.abs(xb - deq) <= bound[:, :, None])


def test_quantize_bad_k_rejected():
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((1, 33), dtype=np.float32))


def test_quantize_layout_is_row_major_blocks():
    # Distinct amax per block shows which 34-byte slot each block lands in.
    rows, k = 3, 96
    x = np.zeros((rows, k), dtype=np.float32)
    for r in range(rows):
        for b in range(3):
            x[r, 32 * b] = 127.0 * 2 ** (r * 3 + b - 4)   # scale = 2^(r*3+b-4)
    blk = oracle.quantize(x)
    bits, q = refmath.split_blocks(blk, k)
    for r in range(rows):
        for b in range(3):
            assert refmath.scales_f64(bits)[r, b] == 2.0 ** (r * 3 + b - 4)
            assert q[r, b, 0] == 127 and not np.any(q[r, b, 1:])
