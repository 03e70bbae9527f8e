"""The oracle on several OpenMP threads gives the same bits as on one.

Each output of the oracle (a quantized block, an out/mag/S_b entry, a grouped
pair's row) is computed by the same code in the same order whatever the
thread count; only which thread runs it changes.  These CPU tests compare the
two runs byte for byte on seeded inputs with ragged shapes, NaN-marked blocks
and invalid expert ids.
"""
import numpy as np

import oracle


def _both(fn, n=4):
    with oracle.threads(1):
        a = fn()
    with oracle.threads(n):
        assert oracle.get_threads() == n
        b = fn()
    assert oracle.get_threads() == 1
    return a, b


def test_quantize_threads_bit_identical():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((37, 320)).astype(np.float32)
    x[3, 40] = np.inf
    x[5, 64:96] = 0.0
    a, b = _both(lambda: oracle.quantize(x))
    assert np.array_equal(a, b)


def test_matmul_threads_bit_identical():
    rng = np.random.default_rng(12)
    k, n, t = 256, 53, 19
    wq = oracle.quantize((0.02 * rng.standard_normal((n, k))).astype(np.float32))
    xq = oracle.quantize(rng.standard_normal((t, k)).astype(np.float32))
    (o1, m1, s1), (o2, m2, s2) = _both(lambda: oracle.matmul(wq, xq, k, want_blocksums=True), 3)
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(m1.view(np.uint64), m2.view(np.uint64))
    assert np.array_equal(s1, s2)


def test_moe_grouped_threads_bit_identical():
    rng = np.random.default_rng(13)
    k, n, t, used, ne = 128, 40, 9, 3, 5
    mats = [oracle.quantize((0.02 * rng.standard_normal((n, k))).astype(np.float32))
            for _ in range(ne)]
    xq = oracle.quantize(rng.standard_normal((t, k)).astype(np.float32))
    sel = rng.integers(0, ne, size=(t, used)).astype(np.int32)
    sel[2, 1] = ne + 3  # invalid id: NaN row, counted
    (o1, m1, c1), (o2, m2, c2) = _both(lambda: oracle.moe_grouped(mats, sel, xq, k, n, 0), 4)
    assert c1 == c2 == 1
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(np.isnan(m1), np.isnan(m2))
    assert np.array_equal(np.nan_to_num(m1), np.nan_to_num(m2))


def test_host_threads_respects_environment(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    assert oracle.host_threads() == 3
    monkeypatch.setenv("OMP_NUM_THREADS", "64")
    assert oracle.host_threads() == 16
