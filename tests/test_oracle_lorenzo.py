"""Pins of the oracle's Lorenzo-quantizer front end (CPU only).

The oracle writes the quantizer out cell by cell.  These tests check it
against what the definition fixes without re-evaluating it: closed forms for
constant and linear fields, the inverse (prefix sums of the residuals give
back the quantized field) together with the error bound, the tie rule of
round-half-even, and clamping.
"""
import numpy as np
import pytest

import oracle

R = 32768


@pytest.mark.parametrize("shape", [(1,), (9,), (4, 7), (3, 5, 6)])
def test_constant_field(shape):
    # q is the same number Q everywhere: every residual but the origin's
    # cancels, the origin keeps Q
    eb = 0.25
    f = np.full(shape, 3.0, np.float32)  # Q = rint(3 / 0.5) = 6
    codes, clamped = oracle.lorenzo_quant(f, eb)
    want = np.full(shape, R, np.uint32)
    want[(0,) * len(shape)] = R + 6
    assert clamped == 0
    assert np.array_equal(codes, want)


def test_ramp_2d():
    # f = c + a x + b y with 2 eb = 1: q = f exactly.  Residuals: origin c,
    # first row a, first column b, elsewhere 0 (mixed differences vanish)
    a, b, c = 3, -5, 7
    y, x = np.mgrid[0:6, 0:9]
    f = (c + a * x + b * y).astype(np.float32)
    codes, clamped = oracle.lorenzo_quant(f, 0.5)
    want = np.full(f.shape, R, np.int64)
    want[0, 0] += c
    want[0, 1:] += a
    want[1:, 0] += b
    assert clamped == 0
    assert np.array_equal(codes.astype(np.int64), want)


def test_ramp_3d():
    a, b, d, c = 2, 3, -4, 11
    z, y, x = np.mgrid[0:4, 0:5, 0:6]
    f = (c + a * x + b * y + d * z).astype(np.float32)
    codes, clamped = oracle.lorenzo_quant(f, 0.5)
    want = np.full(f.shape, R, np.int64)
    want[0, 0, 0] += c
    want[0, 0, 1:] += a
    want[0, 1:, 0] += b
    want[1:, 0, 0] += d
    assert clamped == 0
    assert np.array_equal(codes.astype(np.int64), want)


@pytest.mark.parametrize("shape", [(1000,), (37, 53), (9, 17, 23)])
@pytest.mark.parametrize("eb", [1e-3, 0.05])
def test_inverse_and_error_bound(shape, eb):
    # undo the predictor with prefix sums along every axis; the result q must
    # satisfy |f - 2 eb q| <= eb (round to nearest), up to double rounding
    rng = np.random.default_rng(len(shape) * 7 + int(eb * 1000))
    f = (rng.standard_normal(shape) * 3.0).astype(np.float32)
    codes, clamped = oracle.lorenzo_quant(f, eb)
    assert clamped == 0
    q = codes.astype(np.int64) - R
    for ax in range(q.ndim):
        q = np.cumsum(q, axis=ax)
    err = np.abs(f.astype(np.float64) - 2.0 * eb * q)
    assert err.max() <= eb * (1 + 1e-9)


def test_ties_round_half_even():
    # 2 eb = 1: q = f rounded to the nearest integer, ties to even
    f = np.array([0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5], np.float32)
    q = np.array([0, 2, 2, 4, 0, -2, -2], np.int64)
    codes, clamped = oracle.lorenzo_quant(f, 0.5)
    want = R + np.diff(np.concatenate([[0], q]))
    assert clamped == 0
    assert np.array_equal(codes.astype(np.int64), want)


def test_clamping():
    f = np.array([0.0, 40000.0, 0.0, -40000.0, 0.0, 100.0], np.float32)
    codes, clamped = oracle.lorenzo_quant(f, 0.5)
    # residuals 0, 40000, -40000, -40000, 40000, 100
    assert codes.tolist() == [R, 65535, 0, 0, 65535, R + 100]
    assert clamped == 4
