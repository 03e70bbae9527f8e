"""CPU pins of the oracle's expert-FFN steps: SwiGLU with the optional clamp
("Part 3: 模型架构", section 4, SwiGLU activation) and the weighted combine of
the experts' outputs ("Part 6: 代码走读", trace 5, step 4).

The pins do not restate the oracle's formula: SiLU values are checked against
an independent 50-digit decimal evaluation, closed forms (sigmoid(ln a) =
a/(1+a)), and the identity silu(x) - silu(-x) = x; the combine against exact
dyadic examples and invariants."""
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "swiglu_closed_form.txt")
getcontext().prec = 50


def _silu_decimal(g: float) -> Decimal:
    d = Decimal(float(g))
    return d / (1 + (-d).exp())


def _f32(x) -> np.float32:
    return np.float32(float(x))


def test_golden_closed_forms():
    rows = []
    for line in open(GOLDEN, encoding="utf-8"):
        line = line.split("#")[0].strip()
        if line:
            rows.append([float(v) for v in line.split()])
    assert len(rows) >= 8
    for g, u, clamp, expected in rows:
        got = oracle.swiglu(np.array([g], np.float32), np.array([u], np.float32), clamp)[0]
        assert np.isclose(got, expected, rtol=1e-9, atol=1e-12) or got == np.float32(expected), \
            (g, u, clamp, got, expected)


def test_silu_against_decimal():
    rng = np.random.default_rng(1)
    g = np.concatenate([rng.normal(0, 3, 2000), rng.uniform(-60, 60, 500), [0.5, -0.5, 1e-30, -1e-30]]).astype(np.float32)
    u = rng.normal(0, 2, g.size).astype(np.float32)
    got = oracle.swiglu(g, u)
    for i in range(g.size):
        exp = _f32(_silu_decimal(g[i]) * Decimal(float(u[i])))
        assert got[i] == exp, (g[i], u[i], got[i], exp)


def test_silu_odd_part_identity():
    # silu(x) - silu(-x) = x * (sigmoid(x) + sigmoid(-x)) = x.
    x = np.linspace(-30, 30, 601, dtype=np.float32)
    one = np.ones_like(x)
    a = oracle.swiglu(x, one).astype(np.float64)
    b = oracle.swiglu(-x, one).astype(np.float64)
    ulp = np.spacing(np.maximum(np.abs(a), np.abs(b)).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs((a - b) - x) <= 2 * ulp + 1e-30)


def test_silu_limits_and_sign():
    g = np.array([0.0, 50.0, -50.0, 1.0, -1.0], np.float32)
    mid = oracle.swiglu(g, np.ones_like(g))
    assert mid[0] == 0.0
    assert mid[1] == np.float32(50.0)            # sigmoid(50) = 1 - 2e-22
    assert -1e-19 < mid[2] < 0.0                 # -50 * e^-50
    assert mid[3] > 0 > mid[4] and abs(mid[3]) > abs(mid[4])  # silu is not odd


def test_clamp_semantics():
    nan = np.float32(np.nan)
    g = np.array([20, 20, -20, 1, 1, nan, 1], np.float32)
    u = np.array([1, 1, 1, 15, -15, 1, nan], np.float32)
    c = oracle.swiglu(g, u, 10.0)
    n = oracle.swiglu(g, u, 0.0)
    assert c[0] == oracle.swiglu(np.array([10], np.float32), np.array([1], np.float32))[0]
    assert n[0] == oracle.swiglu(np.array([20], np.float32), np.array([1], np.float32))[0]
    assert c[2] == n[2]                          # gate is only clamped from above
    assert c[3] == _f32(_silu_decimal(1.0) * 10) and c[4] == -c[3]
    assert n[3] == _f32(_silu_decimal(1.0) * 15)
    assert np.isnan(c[5]) and np.isnan(c[6])     # NaN passes the clamp


def test_combine_exact_examples():
    y = np.array([[[1, 2, -3], [3, 4, 5]], [[-8, 0, 1], [2, 2, 2]]], np.float32)
    w = np.array([[0.5, 0.25], [1.0, 0.125]], np.float32)
    out, mag = oracle.moe_combine(y, w)
    np.testing.assert_array_equal(out, np.array([[1.25, 2.0, -0.25], [-7.75, 0.25, 1.25]], np.float32))
    np.testing.assert_array_equal(mag, np.array([[1.25, 2.0, 2.75], [8.25, 0.25, 1.25]]))


def test_combine_invariants():
    rng = np.random.default_rng(2)
    y = rng.normal(0, 1, (5, 8, 33)).astype(np.float32)
    w = rng.uniform(0, 1, (5, 8)).astype(np.float32)
    out, mag = oracle.moe_combine(y, w)
    # one slot with weight 1 is the identity
    o1, _ = oracle.moe_combine(y[:, :1], np.ones((5, 1), np.float32))
    np.testing.assert_array_equal(o1, y[:, 0])
    # slot order does not matter beyond rounding of the double sum
    perm = rng.permutation(8)
    op, _ = oracle.moe_combine(y[:, perm], w[:, perm])
    assert np.all(np.abs(op.astype(np.float64) - out) <= np.spacing(np.abs(out)) + 1e-30)
    # against a float64 restatement
    ref = np.einsum("tj,tjo->to", w.astype(np.float64), y.astype(np.float64))
    assert np.all(np.abs(out - ref) <= 1e-6 * mag + 1e-12)
    # a NaN in one expert's output poisons that token's element only
    y2 = y.copy()
    y2[2, 3, 7] = np.nan
    o2, _ = oracle.moe_combine(y2, w)
    assert np.isnan(o2[2, 7]) and np.isnan(o2).sum() == 1
