"""Pins for the oracle's Q8_0 matmul and grouped-expert matmul (CPU only).

Definition (ds4-learning "Part 6: 代码走读", trace 3; "Part 3: 模型架构",
section 2, item 4): out[t][o] = sum over 32-value blocks of d_w * d_x * S_b,
S_b = sum of int8 products in the block.  Checked against brute-force float64
dequantize-then-dot, exact integer special cases and invariants.
"""
import numpy as np
import pytest

import oracle
from tests import refmath


def _mk(seed, out_dim, n_tok, k, w_std=0.02, x_std=1.0):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((out_dim, k)) * w_std).astype(np.float32)
    x = (rng.standard_normal((n_tok, k)) * x_std).astype(np.float32)
    return oracle.quantize(w), oracle.quantize(x)


def test_single_block_hand_values():
    # w q = [3, -2, 0...], d_w = 0.5 ; x q = [4, 5, 0...], d_x = 2
    # S = 12 - 10 = 2 ; out = 0.5 * 2 * 2 = 2
    w = refmath.join_blocks(np.array([[0x3800]], np.uint16),
                            np.array([[[3, -2] + [0] * 30]], np.int8))
    x = refmath.join_blocks(np.array([[0x4000]], np.uint16),
                            np.array([[[4, 5] + [0] * 30]], np.int8))
    out, mag, bs = oracle.matmul(w, x, 32, want_blocksums=True)
    assert out[0, 0] == 2.0 and mag[0, 0] == 2.0 and bs[0, 0, 0] == 2
    # Two blocks with opposite-sign terms: mag adds magnitudes, out cancels.
    w2 = refmath.join_blocks(np.array([[0x3C00, 0x3C00]], np.uint16),
                             np.array([[[1] + [0] * 31, [1] + [0] * 31]], np.int8))
    x2 = refmath.join_blocks(np.array([[0x3C00, 0x3C00]], np.uint16),
                             np.array([[[7] + [0] * 31, [-7] + [0] * 31]], np.int8))
    out, mag, _ = oracle.matmul(w2, x2, 64)
    assert out[0, 0] == 0.0 and mag[0, 0] == 14.0


@pytest.mark.parametrize("k,out_dim,n_tok", [(32, 5, 3), (256, 128, 4), (1024, 33, 7)])
def test_matches_bruteforce_f64(k, out_dim, n_tok):
    wq, xq = _mk(k + out_dim, out_dim, n_tok, k)
    out, mag, _ = oracle.matmul(wq, xq, k)
    ref = refmath.matmul_f64(wq, xq, k)
    refmag = refmath.mag_f64(wq, xq, k)
    np.testing.assert_allclose(mag, refmag, rtol=1e-13, atol=0)
    err = np.abs(out.astype(np.float64) - ref)
    assert np.all(err <= 0.5 * refmath.f32_ulp(ref) + 1e-12 * refmag + 1e-30)


def test_blocksums_match_int64_einsum():
    wq, xq = _mk(5, 17, 3, 256)
    _, _, bs = oracle.matmul(wq, xq, 256, want_blocksums=True)
    np.testing.assert_array_equal(bs.astype(np.int64), refmath.blocksums_i64(wq, xq, 256))


def test_unit_scales_reduce_to_integer_matmul():
    rng = np.random.default_rng(9)
    k, o, t = 512, 40, 6
    qw = rng.integers(-127, 128, size=(o, k // 32, 32)).astype(np.int8)
    qx = rng.integers(-127, 128, size=(t, k // 32, 32)).astype(np.int8)
    ones_w = np.full((o, k // 32), 0x3C00, np.uint16)
    ones_x = np.full((t, k // 32), 0x3C00, np.uint16)
    out, _, _ = oracle.matmul(refmath.join_blocks(ones_w, qw), refmath.join_blocks(ones_x, qx), k)
    ref = qx.reshape(t, k).astype(np.int64) @ qw.reshape(o, k).astype(np.int64).T
    np.testing.assert_array_equal(out, ref.astype(np.float32))


def test_zero_scale_contributes_nothing():
    k = 256
    wq, xq = _mk(21, 9, 3, k)
    bits, q = refmath.split_blocks(wq, k)
    bits = bits.copy()
    bits[:, 3] = 0                      # scale 0, quants untouched
    zeroed = refmath.join_blocks(bits, q)
    q2 = q.copy()
    q2[:, 3, :] = 0                      # same block with quants zeroed instead
    out_a, _, _ = oracle.matmul(zeroed, xq, k)
    out_b, _, _ = oracle.matmul(refmath.join_blocks(bits, q2), xq, k)
    np.testing.assert_array_equal(out_a, out_b)


def test_sign_and_scale_invariants():
    k = 512
    wq, xq = _mk(33, 31, 5, k)
    out, _, _ = oracle.matmul(wq, xq, k)
    bx, qx = refmath.split_blocks(xq, k)
    neg, _, _ = oracle.matmul(wq, refmath.join_blocks(bx, -qx), k)
    np.testing.assert_array_equal(neg, -out)
    bw, qw = refmath.split_blocks(wq, k)
    neg_w, _, _ = oracle.matmul(refmath.join_blocks(bw, -qw), xq, k)
    np.testing.assert_array_equal(neg_w, -out)
    # Doubling every weight scale (exponent field + 1, scales stay normal) doubles out.
    assert np.all((bw & 0x7C00) != 0) and np.all((bw & 0x7C00) < 0x7800)
    dbl, _, _ = oracle.matmul(refmath.join_blocks((bw + 0x0400).astype(np.uint16), qw), xq, k)
    np.testing.assert_array_equal(dbl, 2 * out)


def test_roles_of_w_and_x_are_symmetric():
    k = 256
    wq, xq = _mk(41, 12, 7, k)
    a, _, _ = oracle.matmul(wq, xq, k)
    b, _, _ = oracle.matmul(xq, wq, k)
    np.testing.assert_array_equal(a, b.T)


def test_linearity_in_scales_within_tolerance():
    # out is linear in the per-block scale products; fp32 rounding aside.
    k = 512
    wq, xq = _mk(51, 16, 4, k)
    bw, qw = refmath.split_blocks(wq, k)
    half = bw.copy()
    half[:, ::2] = 0
    other = bw.copy()
    other[:, 1::2] = 0
    full, mag, _ = oracle.matmul(wq, xq, k)
    a, _, _ = oracle.matmul(refmath.join_blocks(half, qw), xq, k)
    b, _, _ = oracle.matmul(refmath.join_blocks(other, qw), xq, k)
    err = np.abs(full.astype(np.float64) - (a.astype(np.float64) + b.astype(np.float64)))
    assert np.all(err <= 3e-7 * mag + 1e-30)


def test_nan_scale_poisons_only_its_outputs():
    k = 64
    wq, xq = _mk(61, 4, 3, k)
    bx, qx = refmath.split_blocks(xq, k)
    bx = bx.copy()
    bx[1, 0] = 0x7E00
    out, _, _ = oracle.matmul(wq, refmath.join_blocks(bx, qx), k)
    assert np.all(np.isnan(out[1])) and np.all(np.isfinite(out[[0, 2]]))


def test_moe_grouped_equals_dense_per_pair():
    k, od, n_exp, n_tok, n_used = 128, 24, 6, 5, 3
    rng = np.random.default_rng(71)
    experts = [_mk(100 + e, od, 1, k)[0] for e in range(n_exp)]
    sel = np.stack([rng.choice(n_exp, n_used, replace=False) for _ in range(n_tok)]).astype(np.int32)
    x = (rng.standard_normal((n_tok * n_used, k))).astype(np.float32)
    xq_all = oracle.quantize(x)
    for x_rows in (0, 1):
        xq = xq_all[:n_tok] if x_rows == 0 else xq_all
        out, mag, bad = oracle.moe_grouped(experts, sel, xq, k, od, x_rows)
        assert bad == 0
        for t in range(n_tok):
            for j in range(n_used):
                row = t if x_rows == 0 else t * n_used + j
                ref, rmag, _ = oracle.matmul(experts[sel[t, j]], xq[row:row + 1], k)
                np.testing.assert_array_equal(out[t, j], ref[0])
                np.testing.assert_array_equal(mag[t, j], rmag[0])


def test_moe_grouped_token_permutation_and_invalid_ids():
    k, od, n_exp = 64, 8, 4
    experts = [_mk(200 + e, od, 1, k)[0] for e in range(n_exp)]
    sel = np.array([[0, 2], [3, 1], [2, 0]], dtype=np.int32)
    xq = _mk(300, 1, 3, k)[1]
    out, _, _ = oracle.moe_grouped(experts, sel, xq, k, od, 0)
    perm = np.array([2, 0, 1])
    out_p, _, _ = oracle.moe_grouped(experts, sel[perm], xq[perm], k, od, 0)
    np.testing.assert_array_equal(out_p, out[perm])
    bad_sel = sel.copy()
    bad_sel[1, 0] = 7
    bad_sel[2, 1] = -1
    out_b, _, n_bad = oracle.moe_grouped(experts, bad_sel, xq, k, od, 0)
    assert n_bad == 2
    assert np.all(np.isnan(out_b[1, 0])) and np.all(np.isnan(out_b[2, 1]))
    np.testing.assert_array_equal(out_b[0], out[0])
