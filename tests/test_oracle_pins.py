"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Each test ties the oracle to mathematics, a textbook table, an independent
library routine, or exact brute force, chosen so that a plausible slip in the
oracle (a dropped term, a transposed operand, a wrong bias index, round-toward-
zero instead of nearest-even, the tanh GELU instead of the erf form, bias added
after GELU) fails at least one of them.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# binary16 codec: exhaustive
# --------------------------------------------------------------------------
ALL_BITS = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def test_decode_exhaustive_matches_numpy():
    d = oracle.f16_decode(ALL_BITS)
    ref = ALL_BITS.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(d), nan)
    assert np.array_equal(d[~nan], ref[~nan])
    # signed zeros keep their sign
    assert math.copysign(1.0, d[0x8000]) == -1.0


def test_encode_roundtrip_exhaustive():
    d = oracle.f16_decode(ALL_BITS)
    e = oracle.f16_encode(d)
    nan = np.isnan(d)
    assert np.array_equal(e[~nan], ALL_BITS[~nan])
    assert np.all((e[nan] & 0x7C00) == 0x7C00) and np.all((e[nan] & 0x3FF) != 0)


def test_encode_midpoints_round_to_even():
    # every midpoint between adjacent finite non-negative binary16 values
    pos = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)
    lo = pos[:-1].view(np.float16).astype(np.float64)
    hi = pos[1:].view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2  # exact in fp64
    e = oracle.f16_encode(mid)
    even = np.where(pos[:-1] % 2 == 0, pos[:-1], pos[1:])
    assert np.array_equal(e, even)
    assert np.array_equal(oracle.f16_encode(-mid), even | 0x8000)
    # independent library: numpy's double -> half cast
    assert np.array_equal(e, mid.astype(np.float16).view(np.uint16))


def test_encode_random_matches_numpy_cast():
    rng = np.random.default_rng(123)
    x = np.concatenate([
        rng.standard_normal(200000) * 10.0 ** rng.integers(-9, 6, 200000),
        rng.uniform(-65000, 65000, 50000),
        rng.uniform(-2 ** -14, 2 ** -14, 50000),   # subnormal range
    ])
    assert np.array_equal(oracle.f16_encode(x), x.astype(np.float16).view(np.uint16))


def test_encode_overflow_and_specials():
    assert oracle.f16_encode([65504.0])[0] == 0x7BFF
    assert oracle.f16_encode([65519.99])[0] == 0x7BFF
    assert oracle.f16_encode([65520.0])[0] == 0x7C00      # tie above max rounds to inf
    assert oracle.f16_encode([-1e9])[0] == 0xFC00
    assert oracle.f16_encode([2.0 ** -25])[0] == 0x0000    # tie with 0 -> even (0)
    assert oracle.f16_encode([3 * 2.0 ** -25])[0] == 0x0002  # tie 1.5 ulp -> 2
    assert oracle.f16_encode([-0.0])[0] == 0x8000


# --------------------------------------------------------------------------
# GEMM core: closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("K", [1, 256, 1000, 4096])
def test_all_ones_gives_K(K):
    A = np.ones((3, K), np.float16)
    B = np.ones((K, 5), np.float16)
    C = oracle.gemm(A, B)
    assert np.all(C.astype(np.float64) == np.float16(K).astype(np.float64))


def test_identity_left_and_right():
    B = workloads.random_f16(5, (64, 48))
    A = np.eye(64, dtype=np.float16)
    assert np.array_equal(oracle.gemm(A, B).view(np.uint16) & 0x7FFF | 0, B.view(np.uint16) & 0x7FFF)
    assert np.array_equal(oracle.gemm(A, B).astype(np.float64), B.astype(np.float64))
    A2 = workloads.random_f16(6, (40, 48))
    assert np.array_equal(oracle.gemm(A2, np.eye(48, dtype=np.float16)).astype(np.float64),
                          A2.astype(np.float64))


def test_permutation_rows():
    rng = np.random.default_rng(7)
    p = rng.permutation(33)
    P = np.zeros((33, 33), np.float16)
    P[np.arange(33), p] = 1
    B = workloads.random_f16(8, (33, 17))
    assert np.array_equal(oracle.gemm(P, B).astype(np.float64), B[p].astype(np.float64))


def _rank1(u, v, K=9, col=4):
    A = np.zeros((len(u), K), np.float16)
    A[:, col] = u
    B = workloads.random_f16(9, (K, len(v)))
    B[col, :] = v
    return A, B


def test_rank1_single_rounding_and_ties():
    # u_i * v_j is exact in fp64, so C must be the single RNE rounding of it.
    u = np.array([1 + 2 ** -10, 3.0, -0.75, 1 + 2 ** -10, 2 ** -12], np.float16)
    v = np.array([1.5, 1 + 2 ** -9, -3 - 2 ** -8, 0.1, 1.0 + 3 * 2 ** -10], np.float16)
    A, B = _rank1(u, v)
    C = oracle.gemm(A, B)
    exact = np.outer(u.astype(np.float64), v.astype(np.float64))
    assert np.array_equal(C.view(np.uint16), exact.astype(np.float16).view(np.uint16))
    # (1+2^-10)*1.5 = 1.5 + 1.5*2^-10 lies exactly halfway between two fp16 values:
    # nearest-even gives 1.5 + 2*2^-10, truncation would give 1.5 + 2^-10.
    assert float(C[0, 0]) == 1.5 + 2 * 2 ** -10


# --------------------------------------------------------------------------
# GEMM core: exact brute force with rationals
# --------------------------------------------------------------------------
def _f16_round_exact(q: Fraction):
    """Correctly round a rational to binary16 (RNE), written with exact arithmetic.
    Returns (bits, near_tie) where near_tie flags values within 2^-40 (relative)
    of a rounding boundary, where an fp64 accumulation may legitimately differ."""
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    if a == 0:
        return sign, False
    E = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** E > a:
        E -= 1
    E = max(E, -14)
    n = a / (Fraction(2) ** (E - 10))
    fl = n.numerator // n.denominator
    rem = n - fl
    near = abs(rem - Fraction(1, 2)) < Fraction(1, 2 ** 40) * n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    if fl < 1024:
        bits = fl
    else:
        bits = ((E + 15) << 10) + (fl - 1024)
    if bits >= 0x7C00:
        bits = 0x7C00
    return sign | bits, near


@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 3, 5), (3, 2, 7), (5, 7, 8), (8, 5, 3), (7, 8, 2)])
def test_bruteforce_fractions(shape):
    M, N, K = shape
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    # random bit patterns: all finite binary16 values incl. subnormals, both signs
    def rand_f16(sz):
        bits = rng.integers(0, 0x7C00, size=sz, dtype=np.uint32).astype(np.uint16)
        bits |= (rng.integers(0, 2, size=sz, dtype=np.uint16) << 15).astype(np.uint16)
        x = bits.view(np.float16)
        # keep products in range: scale exponents down by squashing huge values
        x = np.where(np.abs(x.astype(np.float64)) > 256, x / np.float16(512), x).astype(np.float16)
        return x
    A, B = rand_f16((M, K)), rand_f16((K, N))
    bias = rand_f16((N,))
    for epi in ("none", "bias"):
        C = oracle.gemm(A, B, bias if epi != "none" else None, epi)
        for i in range(M):
            for j in range(N):
                s = sum(Fraction(float(A[i, k])) * Fraction(float(B[k, j])) for k in range(K))
                if epi == "bias":
                    s += Fraction(float(bias[j]))
                bits, near = _f16_round_exact(s)
                if near:
                    continue
                got = int(C.view(np.uint16)[i, j])
                if s == 0:
                    assert got & 0x7FFF == 0
                else:
                    assert got == bits, (epi, i, j, hex(got), hex(bits))


# --------------------------------------------------------------------------
# GEMM core: independent library (numpy fp64 BLAS)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name,shape", [("gemm_256", None), ("ragged_4095x3001x1000", (129, 77, 1000))])
def test_fp64_sum_matches_numpy(name, shape):
    if shape is None:
        A, B, _ = workloads.make_inputs(name)
    else:
        A, B, _ = workloads.make_inputs(name, M=shape[0], N=shape[1], K=shape[2])
    C, Y = oracle.gemm(A, B, want_y=True)
    a, b = A.astype(np.float64), B.astype(np.float64)
    S = a @ b
    bound = 1e-12 * (np.abs(a) @ np.abs(b)) + 1e-300
    assert np.all(np.abs(Y - S) <= bound)
    # after rounding to fp16 the two agree except possibly at exact-tie neighbourhoods
    assert np.mean(C.view(np.uint16) == S.astype(np.float16).view(np.uint16)) > 0.9999


# --------------------------------------------------------------------------
# GELU: closed forms, textbook table, independent libraries
# --------------------------------------------------------------------------
def test_gelu_textbook_values():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "normal_cdf.txt")) if l.strip() and l[0] != "#"]
    for xs, phis in rows:
        x, phi = float(xs), float(phis)
        for s in (1.0, -1.0):
            xv = s * x
            # gelu(x) = x * Phi(x), Phi(-x) = 1 - Phi(x)
            expect = xv * (phi if s > 0 else 1.0 - phi)
            assert abs(oracle.gelu([xv])[0] - expect) <= 2e-15 * max(1.0, abs(x)), (xv, expect)


def test_gelu_identities():
    x = np.linspace(-8, 8, 100001)
    g = oracle.gelu(x)
    gm = oracle.gelu(-x)
    assert oracle.gelu([0.0])[0] == 0.0
    assert np.allclose(g - gm, x, rtol=0, atol=1e-14)
    big = x[x >= 6]
    assert np.all(np.abs(oracle.gelu(big) - big) < 1e-8 * big)
    # the tanh approximation differs from the exact form by ~1e-3 near |x| ~ 2:
    tanh_form = 0.5 * x * (1 + np.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))
    assert np.max(np.abs(g - tanh_form)) > 1e-4


def test_gelu_matches_scipy_and_torch():
    from scipy.special import erf
    import torch
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(300000) * 3, rng.uniform(-40, 40, 10000)])
    g = oracle.gelu(x)
    ref = 0.5 * x * (1 + erf(x / math.sqrt(2)))
    # 1 + erf(z) cancels for z << 0, so compare on the scale of the input
    scale = np.maximum(np.abs(x), 1e-300)
    assert np.all(np.abs(g - ref) <= 4e-16 * scale)
    tg = torch.nn.functional.gelu(torch.from_numpy(x), approximate="none").numpy()
    assert np.all(np.abs(g - tg) <= 4e-16 * scale)


# --------------------------------------------------------------------------
# epilogue wiring: bias index, broadcast, order of bias and GELU
# --------------------------------------------------------------------------
def test_bias_broadcast_over_rows():
    bias = workloads.random_f16(21, (37,), -4, 4)
    A = np.zeros((6, 10), np.float16)
    B = workloads.random_f16(22, (10, 37))
    C = oracle.gemm(A, B, bias, "bias")
    assert np.array_equal(C.astype(np.float64), np.broadcast_to(bias.astype(np.float64), (6, 37)))
    from scipy.special import erf
    Cg = oracle.gemm(A, B, bias, "bias_gelu")
    bb = bias.astype(np.float64)
    ref = (0.5 * bb * (1 + erf(bb / math.sqrt(2)))).astype(np.float16)
    assert np.array_equal(Cg.view(np.uint16), np.broadcast_to(ref.view(np.uint16), (6, 37)))


def test_gelu_applied_after_bias():
    # rank-1: S = u_i * v_j exact; C = fp16(gelu(S + bias_j))
    from scipy.special import erf
    u = np.array([1.0, -2.0, 0.5], np.float16)
    v = np.array([1.0, 2.0, -1.0, 3.0], np.float16)
    A, B = _rank1(u, v)
    bias = np.array([-3.0, 0.25, 1.5, -0.5], np.float16)
    C = oracle.gemm(A, B, bias, "bias_gelu")
    X = np.outer(u.astype(np.float64), v.astype(np.float64)) + bias.astype(np.float64)
    ref = (0.5 * X * (1 + erf(X / math.sqrt(2)))).astype(np.float16)
    assert np.array_equal(C.view(np.uint16), ref.view(np.uint16))
    wrong = (0.5 * (X - bias) * (1 + erf((X - bias) / math.sqrt(2))) + bias).astype(np.float16)
    assert not np.array_equal(C.view(np.uint16), wrong.view(np.uint16))


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def test_power_of_two_scaling_exact():
    A, B, _ = workloads.make_inputs("gemm_256", M=64, N=48, K=96)
    C, Y = oracle.gemm(A, B, want_y=True)
    C2, Y2 = oracle.gemm((A.astype(np.float32) * 4).astype(np.float16), B, want_y=True)
    assert np.array_equal(Y2, Y * 4)
    assert np.array_equal(C2.astype(np.float64), C.astype(np.float64) * 4)


def test_transpose_identity():
    A = workloads.random_f16(31, (23, 41))
    B = workloads.random_f16(32, (41, 19))
    C = oracle.gemm(A, B)
    Ct = oracle.gemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    assert np.array_equal(C.T.astype(np.float64), Ct.astype(np.float64))


def test_k_split_additivity():
    A = workloads.random_f16(41, (17, 300))
    B = workloads.random_f16(42, (300, 13))
    _, Y = oracle.gemm(A, B, want_y=True)
    _, Y1 = oracle.gemm(A[:, :111].copy(), B[:111].copy(), want_y=True)
    _, Y2 = oracle.gemm(A[:, 111:].copy(), B[111:].copy(), want_y=True)
    assert np.allclose(Y, Y1 + Y2, rtol=0, atol=1e-12)


def test_points_equal_full_product():
    A, B, bias = workloads.make_inputs("ragged_4095x3001x1000", M=70, N=90, K=1000)
    for epi in ("none", "bias", "bias_gelu"):
        C = oracle.gemm(A, B, bias, epi)
        rng = np.random.default_rng(3)
        r = rng.integers(0, 70, 500)
        c = rng.integers(0, 90, 500)
        P = oracle.gemm_points(A, B, bias, epi, r, c)
        assert np.array_equal(P.view(np.uint16), C.view(np.uint16)[r, c])


def test_thread_count_does_not_change_bits():
    A, B, bias = workloads.make_inputs("mlp_up_8192x16384x4096", M=40, N=64, K=512)
    C1 = oracle.gemm(A, B, bias, "bias_gelu", threads=1)
    C8 = oracle.gemm(A, B, bias, "bias_gelu", threads=8)
    assert np.array_equal(C1.view(np.uint16), C8.view(np.uint16))


# --------------------------------------------------------------------------
# degenerate sizes
# --------------------------------------------------------------------------
def test_degenerate_shapes():
    bias = workloads.random_f16(51, (5,))
    assert oracle.gemm(np.zeros((0, 4), np.float16), np.zeros((4, 5), np.float16)).shape == (0, 5)
    assert oracle.gemm(np.zeros((3, 4), np.float16), np.zeros((4, 0), np.float16)).shape == (3, 0)
    A0, B0 = np.zeros((3, 0), np.float16), np.zeros((0, 5), np.float16)
    assert np.all(oracle.gemm(A0, B0).astype(np.float64) == 0)
    assert np.array_equal(oracle.gemm(A0, B0, bias, "bias").astype(np.float64),
                          np.broadcast_to(bias.astype(np.float64), (3, 5)))


def test_workload_recipe_is_stable():
    # the generator's draws are part of the recipe: record the digest of a small instance
    A, B, bias = workloads.make_inputs("gemm_256")
    assert A.shape == (256, 256) and B.shape == (256, 256) and bias is None
    assert float(np.abs(A.astype(np.float32)).max()) <= 1.0
    A3, B3, b3 = workloads.make_inputs("mlp_up_8192x16384x4096", M=64, N=128, K=4096)
    assert abs(float(B3.astype(np.float64).std()) - 1 / 64) < 2e-4
    assert abs(float(b3.astype(np.float64).std()) - math.sqrt(0.1)) < 0.08
