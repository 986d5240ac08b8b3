"""Pins of the oracle's attention forward pass to facts outside itself (no GPU needed).

Chosen so that a plausible slip fails at least one of them: a missing or wrong
scale, the causal mask shifted by one or applied bottom-right, a softmax over the
wrong axis, Q and K swapped, V's index confused with K's, an unnormalised sum.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def _draw(seed, B, H, Nq, Nkv, D, sd=1.0):
    rng = np.random.default_rng(seed)
    Q = (rng.standard_normal((B, H, Nq, D)) * sd).astype(np.float16)
    K = (rng.standard_normal((B, H, Nkv, D)) * sd).astype(np.float16)
    V = rng.standard_normal((B, H, Nkv, D)).astype(np.float16)
    return Q, K, V


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 3, 17, 17, 16), (1, 2, 33, 33, 64), (1, 1, 9, 40, 8), (2, 1, 40, 9, 32)])
def test_matches_torch_sdpa_in_fp64(causal, shape):
    B, H, Nq, Nkv, D = shape
    Q, K, V = _draw(sum(shape), B, H, Nq, Nkv, D)
    got, od = oracle.attention(Q, K, V, causal=causal, want_y=True)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q.astype(np.float64)), torch.from_numpy(K.astype(np.float64)),
        torch.from_numpy(V.astype(np.float64)), is_causal=causal).numpy()
    assert np.allclose(od, ref, rtol=1e-12, atol=1e-14)
    assert np.array_equal(got.view(np.uint16), ref.astype(np.float16).view(np.uint16))


def test_explicit_scale_matches_torch():
    Q, K, V = _draw(5, 1, 2, 12, 12, 16)
    got, od = oracle.attention(Q, K, V, causal=False, scale=0.37, want_y=True)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q.astype(np.float64)), torch.from_numpy(K.astype(np.float64)),
        torch.from_numpy(V.astype(np.float64)), scale=0.37).numpy()
    assert np.allclose(od, ref, rtol=1e-12, atol=1e-14)


def test_identical_keys_give_the_mean_of_the_allowed_values():
    # all keys equal -> every allowed key has the same score -> O = mean of the allowed V rows, exactly
    B, H, N, D = 1, 1, 6, 4
    rng = np.random.default_rng(1)
    Q = rng.standard_normal((B, H, N, D)).astype(np.float16)
    K = np.tile(rng.standard_normal((1, 1, 1, D)).astype(np.float16), (B, H, N, 1))
    V = rng.integers(-20, 21, (B, H, N, D)).astype(np.float16)
    for causal in (False, True):
        _, od = oracle.attention(Q, K, V, causal=causal, want_y=True)
        for i in range(N):
            n = i + 1 if causal else N
            for d in range(D):
                exact = Fraction(int(V[0, 0, :n, d].astype(np.int64).sum()), n)
                assert abs(od[0, 0, i, d] - float(exact)) <= 1e-14 * max(1.0, abs(float(exact))), (causal, i, d)


def test_single_key_and_causal_first_row_return_that_value_row():
    Q, K, V = _draw(2, 2, 2, 5, 1, 16)
    got = oracle.attention(Q, K, V, causal=False)
    assert np.array_equal(got.view(np.uint16), np.broadcast_to(V, got.shape).view(np.uint16))
    Q, K, V = _draw(3, 1, 2, 7, 7, 16)
    got = oracle.attention(Q, K, V, causal=True)
    assert np.array_equal(got[:, :, 0].view(np.uint16), V[:, :, 0].view(np.uint16))


def test_one_dominant_key_selects_its_value_row():
    # key j* aligned with the query and far above the others: weights ~ one-hot on j*
    D, N = 8, 10
    Q = np.zeros((1, 1, 1, D), np.float16)
    Q[..., 0] = 30.0
    K = np.zeros((1, 1, N, D), np.float16)
    K[0, 0, 6, 0] = 30.0                     # score 900 / sqrt(8) for j = 6, 0 for the others
    V = np.arange(N * D, dtype=np.float64).reshape(1, 1, N, D).astype(np.float16)
    got = oracle.attention(Q, K, V)
    assert np.array_equal(got[0, 0, 0], V[0, 0, 6])


def test_key_value_permutation_invariance_non_causal():
    Q, K, V = _draw(4, 1, 2, 9, 13, 16)
    perm = np.random.default_rng(0).permutation(13)
    a = oracle.attention(Q, K, V)
    b = oracle.attention(Q, K[:, :, perm], V[:, :, perm])
    _, ad = oracle.attention(Q, K, V, want_y=True)
    _, bd = oracle.attention(Q, K[:, :, perm], V[:, :, perm], want_y=True)
    assert np.allclose(ad, bd, rtol=1e-13, atol=1e-15)
    assert np.mean(a == b) > 0.999


def test_scale_moves_between_q_and_the_scale_argument():
    # Q * 2 with scale / 2 scores identically (powers of two are exact)
    Q, K, V = _draw(6, 1, 1, 8, 8, 16, sd=0.5)
    a, ad = oracle.attention(Q, K, V, causal=True, scale=0.25, want_y=True)
    b, bd = oracle.attention((Q.astype(np.float64) * 2).astype(np.float16), K, V, causal=True, scale=0.125,
                             want_y=True)
    assert np.array_equal(ad, bd)


def test_brute_force_tiny():
    # the definition with Python floats, written independently: weights from math.exp of centred scores
    Q, K, V = _draw(7, 1, 1, 4, 5, 3)
    for causal in (False, True):
        _, od = oracle.attention(Q, K, V, causal=causal, want_y=True)
        q, k, v = (x[0, 0].astype(np.float64) for x in (Q, K, V))
        for i in range(4):
            js = [j for j in range(5) if not causal or j <= i]
            sc = [sum(q[i, d] * k[j, d] for d in range(3)) / math.sqrt(3) for j in js]
            c = sum(sc) / len(sc)
            w = [math.exp(x - c) for x in sc]
            for d in range(3):
                ref = sum(wj * v[j, d] for wj, j in zip(w, js)) / sum(w)
                assert abs(od[0, 0, i, d] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_rejects_zero_keys():
    Q, K, V = _draw(8, 1, 1, 3, 1, 4)
    with pytest.raises(RuntimeError):
        oracle.attention(Q, K[:, :, :0], V[:, :, :0])


@pytest.mark.parametrize("causal", [False, True])
def test_selected_rows_equal_the_full_computation(causal):
    Q, K, V = _draw(9, 2, 3, 21, 17, 8)
    full = oracle.attention(Q, K, V, causal=causal).reshape(-1, 8)
    rows = np.array([0, 5, 20, 21, 62, 63, 125, 64, 3])
    part = oracle.attention_rows(Q, K, V, rows, causal=causal)
    assert np.array_equal(part.view(np.uint16), full[rows].view(np.uint16))
    with pytest.raises(RuntimeError):
        oracle.attention_rows(Q, K, V, np.array([2 * 3 * 21]), causal=causal)
