"""Pins of the oracle's fp32 vector add (CPU only).

The pages' first kernel adds two float32 vectors element by element (TileLang
blog post "Designing High-Performance GPU Kernels with TileLang", section
"Step 3"), so every result is the IEEE binary32 sum, rounded to nearest-even.
The oracle forms it in fp64 and rounds once; these tests pin it to what IEEE
arithmetic fixes independently of that route: numpy's own binary32 addition
over every class of bit pattern, exact ties that separate round-to-nearest-even
from truncation or round-half-up, the overflow boundary, subnormals without
flushing, and the special values.
"""
import numpy as np
import pytest

import oracle
import workloads

f32 = np.float32


def add(a, b):
    return oracle.vector_add(np.asarray(a, dtype=np.float32), np.asarray(b, dtype=np.float32))


def same_bits(x, y):
    """Bit-for-bit equal, counting any two NaNs as equal (payloads may differ)."""
    x, y = np.asarray(x, np.float32), np.asarray(y, np.float32)
    both_nan = np.isnan(x) & np.isnan(y)
    return bool(np.all(both_nan | (x.view(np.uint32) == y.view(np.uint32))))


def test_matches_numpy_binary32_add_on_random_bit_patterns():
    a = workloads.random_f32_bits(1, 1_000_000)
    b = workloads.random_f32_bits(2, 1_000_000)
    with np.errstate(all="ignore"):
        ref = a + b  # numpy's float32 ufunc: one IEEE binary32 addition
    assert same_bits(add(a, b), ref)


def test_matches_numpy_on_close_magnitudes():
    # operands of similar size exercise cancellation and carries more than random bit patterns do
    rng = np.random.default_rng(3)
    a = rng.standard_normal(500_000).astype(np.float32)
    b = (-a * (1 + rng.uniform(-1e-6, 1e-6, a.shape))).astype(np.float32)
    assert same_bits(add(a, b), a + b)
    c = rng.standard_normal(500_000).astype(np.float32)
    assert same_bits(add(a, c), a + c)


def test_exact_small_sums():
    assert same_bits(add([1, 2.5, -7, 1024], [2, 0.25, 3, 1024]), [3, 2.75, -4, 2048])


def test_round_to_nearest_even_ties():
    u = 2.0 ** -23   # ulp of 1.0 in binary32
    # 1 + u/2 lies halfway between 1 and 1 + u: ties go to the even significand (1.0)
    assert same_bits(add([1.0], [u / 2]), [1.0])
    # (1 + u) + u/2 lies halfway between 1 + u (odd) and 1 + 2u (even): rounds up
    assert same_bits(add([1.0 + u], [u / 2]), [1.0 + 2 * u])
    # just above the tie rounds up, below it rounds down
    assert same_bits(add([1.0], [np.nextafter(f32(u / 2), f32(1))]), [1.0 + u])
    assert same_bits(add([1.0 + u], [np.nextafter(f32(u / 2), f32(0))]), [1.0 + u])
    # symmetric for negative values
    assert same_bits(add([-1.0], [-u / 2]), [-1.0])


def test_overflow_boundary():
    fmax = np.finfo(np.float32).max          # (2 - 2^-23) * 2^127, odd significand
    # half an ulp of fmax is 2^103: the tie rounds to the even neighbour 2^128, i.e. overflows to inf
    assert same_bits(add([fmax], [2.0 ** 103]), [np.inf])
    assert same_bits(add([fmax], [2.0 ** 102]), [fmax])
    assert same_bits(add([fmax, -fmax], [fmax, -fmax]), [np.inf, -np.inf])


def test_subnormals_are_not_flushed():
    tiny = 2.0 ** -149                        # smallest binary32 subnormal
    assert same_bits(add([tiny, tiny, 2.0 ** -126], [tiny, -tiny, -tiny]),
                     [2.0 ** -148, 0.0, 2.0 ** -126 - 2.0 ** -149])


def test_special_values():
    inf, nan = np.inf, np.nan
    got = add([inf, inf, -inf, nan, 1.0, 0.0, -0.0, -0.0, 5.0], [-inf, 1.0, -1.0, 1.0, nan, -0.0, -0.0, 0.0, -5.0])
    ref = np.array([nan, inf, -inf, nan, nan, 0.0, -0.0, 0.0, 0.0], np.float32)
    assert same_bits(got, ref)
    # x + (-x) is +0 under round-to-nearest, for every finite x
    x = workloads.random_f32_bits(4, 100_000)
    x = x[np.isfinite(x)]
    r = add(x, -x)
    assert np.all(r.view(np.uint32) == 0)


def test_commutative_and_zero_identity():
    a = workloads.random_f32_bits(5, 200_000)
    b = workloads.random_f32_bits(6, 200_000)
    assert same_bits(add(a, b), add(b, a))
    finite_nonzero = a[np.isfinite(a) & (a != 0)]
    assert same_bits(add(finite_nonzero, np.zeros_like(finite_nonzero)), finite_nonzero)


def test_empty_and_errors():
    assert oracle.vector_add(np.zeros(0, np.float32), np.zeros(0, np.float32)).shape == (0,)
    with pytest.raises(ValueError):
        oracle.vector_add(np.zeros(3, np.float32), np.zeros(4, np.float32))
