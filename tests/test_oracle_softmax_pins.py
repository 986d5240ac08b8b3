"""Pins of the oracle's row softmax to facts outside itself (no GPU needed).

Chosen so that a plausible slip (no shift by the row maximum, a shift by the
minimum, dividing by the maximum instead of the sum, exp of the negated
difference, a sum over the wrong axis, a reduction that skips the last column)
fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle

scipy_special = pytest.importorskip("scipy.special")


def _f16(values):
    return np.asarray(values, dtype=np.float64).astype(np.float16)


def test_two_column_rows_are_the_logistic_function():
    # softmax([a, b]) = [1 / (1 + e^(b - a)), 1 / (1 + e^(a - b))], written with math.exp per element.
    # The large pairs overflow e^x unless the row maximum is subtracted first.
    pairs = [(0.0, 0.0), (1.0, 2.0), (-3.5, 4.25), (7.0, -7.0), (60000.0, 59968.0), (-60000.0, -59999.0),
             (0.0, 11.0), (65504.0, 65504.0), (-65504.0, 0.0)]
    X = _f16(pairs)
    got = oracle.softmax_rows(X)
    for r, (a, b) in enumerate(X.astype(np.float64)):
        def logistic(d):
            return 1.0 / (1.0 + math.exp(d)) if d < 700 else 0.0
        expect = np.array([logistic(b - a), logistic(a - b)]).astype(np.float16)
        assert np.array_equal(got[r].view(np.uint16), expect.view(np.uint16)), (a, b, got[r], expect)


@pytest.mark.parametrize("n", [1, 2, 3, 7, 1000, 4096, 3001])
def test_constant_rows_are_uniform(n):
    X = np.stack([np.full(n, v, np.float16) for v in (0.0, -1.5, 3.0, 65504.0, -65504.0)])
    got = oracle.softmax_rows(X)
    expect = np.float16(1.0 / n)
    assert np.all(got == expect)


def test_matches_scipy_softmax():
    rng = np.random.default_rng(11)
    X = (rng.standard_normal((64, 517)) * 3.0).astype(np.float16)
    got, yd = oracle.softmax_rows(X, want_y=True)
    ref = scipy_special.softmax(X.astype(np.float64), axis=1)
    assert np.allclose(yd, ref, rtol=1e-13, atol=0)
    assert np.array_equal(got.view(np.uint16), ref.astype(np.float16).view(np.uint16))


def test_rows_sum_to_one_and_order_is_kept():
    rng = np.random.default_rng(12)
    X = (rng.standard_normal((16, 300)) * 4.0).astype(np.float16)
    _, yd = oracle.softmax_rows(X, want_y=True)
    assert np.allclose(yd.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    # monotone: a larger input never gets a smaller probability
    for r in range(X.shape[0]):
        o = np.argsort(X[r].astype(np.float64), kind="stable")
        assert np.all(np.diff(yd[r][o]) >= 0)


def test_shift_invariance_and_permutation_equivariance():
    rng = np.random.default_rng(13)
    Xi = rng.integers(-8, 9, (8, 64)).astype(np.float16)          # small integers: x + 16 is exact in fp16
    a = oracle.softmax_rows(Xi)
    b = oracle.softmax_rows((Xi.astype(np.float64) + 16.0).astype(np.float16))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    perm = rng.permutation(64)
    c = oracle.softmax_rows(Xi[:, perm])
    assert np.array_equal(c.view(np.uint16), a[:, perm].view(np.uint16))


def test_rows_are_independent():
    rng = np.random.default_rng(14)
    X = rng.standard_normal((5, 33)).astype(np.float16)
    whole = oracle.softmax_rows(X)
    for r in range(5):
        assert np.array_equal(whole[r].view(np.uint16), oracle.softmax_rows(X[r:r + 1])[0].view(np.uint16))


def test_special_values():
    inf, nan = np.inf, np.nan
    X = _f16([[-inf, 0.0, 0.0, -inf],
              [-inf, -inf, -inf, -inf],
              [1.0, inf, 2.0, 3.0],
              [1.0, nan, 2.0, 3.0],
              [-inf, 5.0, -inf, -inf]])
    got = oracle.softmax_rows(X).astype(np.float64)
    assert np.array_equal(got[0], [0.0, 0.5, 0.5, 0.0])
    assert np.all(np.isnan(got[1]))
    assert np.all(np.isnan(got[2]))
    assert np.all(np.isnan(got[3]))
    assert np.array_equal(got[4], [0.0, 1.0, 0.0, 0.0])


def test_single_column_and_empty_shapes():
    X = _f16([[3.0], [-65504.0], [0.0]])
    assert np.all(oracle.softmax_rows(X) == np.float16(1.0))
    assert oracle.softmax_rows(np.zeros((0, 5), np.float16)).shape == (0, 5)
    assert oracle.softmax_rows(np.zeros((4, 0), np.float16)).shape == (4, 0)


def test_tiny_inputs_brute_force_exact():
    # exhaustive over a small alphabet: rows of 3 values from {-2, -0.5, 0, 1, 3}, checked against the
    # definition evaluated with Python floats in a different order (max of the row subtracted last)
    vals = [-2.0, -0.5, 0.0, 1.0, 3.0]
    rows = np.array([[a, b, c] for a in vals for b in vals for c in vals], np.float16)
    got, yd = oracle.softmax_rows(rows, want_y=True)
    for r, row in enumerate(rows.astype(np.float64)):
        den = sum(math.exp(v) for v in row)
        ref = [math.exp(v) / den for v in row]
        assert np.allclose(yd[r], ref, rtol=1e-14, atol=0)
