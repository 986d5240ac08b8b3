"""GPU parity of the attention forward pass (through the C ABI) against the CPU oracle.

Covers both head dimensions, causal and non-causal masks, query and key lengths
that are not multiples of the 128-row query block or the 64-key block, more
queries than keys and the reverse, one key, explicit scales, constant values,
very peaked scores, and the four attention workloads at full size on sampled
query rows (first and last rows, block edges, random rows), which the oracle
computes row by row with the same absolute row index.  Bar: relative Frobenius
error <= 2e-3 and max |o - ref| / (1 + |ref|) <= 1e-2 (the GEMM's), no NaN.
"""

import numpy as np
import pytest

import oracle
import workloads
from parity import assert_parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def run(lib, Q, K, V, causal, scale=None, kernel=None):
    o = lib.flash_attn(dev(Q), dev(K), dev(V), causal=causal, scale=scale, kernel=kernel)
    torch.cuda.synchronize()
    return o.cpu().numpy()


KERNELS = {"block_serial": 1, "pipelined": 2}


SHAPES = [  # B, H, Nq, Nkv
    (1, 1, 1, 1), (1, 2, 100, 100), (2, 3, 129, 129), (1, 1, 200, 77), (1, 1, 77, 300),
    (1, 2, 513, 513), (2, 2, 256, 1000), (1, 1, 64, 64), (1, 3, 130, 65),
]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES)
def test_shapes(lib, shape, causal, D):
    B, H, Nq, Nkv = shape
    rng = np.random.default_rng(Nq * 7 + Nkv + D)
    Q = rng.standard_normal((B, H, Nq, D)).astype(np.float16)
    K = rng.standard_normal((B, H, Nkv, D)).astype(np.float16)
    V = rng.standard_normal((B, H, Nkv, D)).astype(np.float16)
    ref = oracle.attention(Q, K, V, causal=causal)
    got = run(lib, Q, K, V, causal)
    assert_parity(got, ref, (shape, causal, D))


@pytest.mark.parametrize("scale", [0.0, 0.05, 1.0])
def test_explicit_scales(lib, scale):
    Q, K, V = workloads.make_attention_inputs("attn_b2_h16_n1000_d64_causal", B=1, H=2, Nq=300, Nkv=300)
    for causal in (False, True):
        ref = oracle.attention(Q, K, V, causal=causal, scale=scale)
        got = run(lib, Q, K, V, causal, scale=scale)
        assert_parity(got, ref, (scale, causal))


def test_constant_values_and_peaked_scores(lib):
    rng = np.random.default_rng(3)
    D, N = 128, 300
    Q = (rng.standard_normal((1, 2, N, D)) * 4).astype(np.float16)   # scores with a spread of ~60: near one-hot
    K = (rng.standard_normal((1, 2, N, D)) * 4).astype(np.float16)
    V = np.full((1, 2, N, D), 0.75, np.float16)
    for causal in (False, True):
        got = run(lib, Q, K, V, causal)
        assert np.all(got == np.float16(0.75)), causal        # any convex combination of equal rows
        V2 = rng.standard_normal((1, 2, N, D)).astype(np.float16)
        ref = oracle.attention(Q, K, V2, causal=causal)
        assert_parity(run(lib, Q, K, V2, causal), ref, ("peaked", causal))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kernel", list(KERNELS))
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES)
def test_both_kernels(lib, shape, causal, kernel, D):
    # Both kernels (block-serial and software-pipelined) at both head dimensions, each checked on its own
    B, H, Nq, Nkv = shape
    rng = np.random.default_rng(Nq * 11 + Nkv + D)
    Q, K, V = (rng.standard_normal((B, H, n, D)).astype(np.float16) for n in (Nq, Nkv, Nkv))
    ref = oracle.attention(Q, K, V, causal=causal)
    assert_parity(run(lib, Q, K, V, causal, kernel=KERNELS[kernel]), ref, (shape, causal, kernel))


@pytest.mark.parametrize("kernel", list(KERNELS))
@pytest.mark.parametrize("scale", [0.0, -0.05, 0.05, 1.0])
@pytest.mark.parametrize("wname", ["attn_b1_h8_q777_kv1500_d128", "attn_b2_h16_n1000_d64_causal"])
def test_explicit_scales_by_kernel(lib, scale, kernel, wname):
    # zero and negative scales take the path that scales the scores before the row maximum (D = 128 and 64)
    Q, K, V = workloads.make_attention_inputs(wname, B=1, H=2, Nq=200, Nkv=333)
    for causal in (False, True):
        ref = oracle.attention(Q, K, V, causal=causal, scale=scale)
        assert_parity(run(lib, Q, K, V, causal, scale=scale, kernel=KERNELS[kernel]), ref, (scale, causal, kernel))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kernel", list(KERNELS))
def test_rising_scores_move_the_reference_maximum(lib, kernel, D):
    # Key rows grow in norm along the sequence, so a row's block maxima keep rising and the lazily raised
    # reference maximum moves many times mid-sequence (each time a block maximum passes it by more than 2^8);
    # in the pipelined kernel every such move recomputes the next block's first-half probabilities.
    rng = np.random.default_rng(21)
    N = 900
    Q = rng.standard_normal((1, 2, N, D))
    K = rng.standard_normal((1, 2, N, D)) * (1.0 + np.arange(N) / 20.0)[None, None, :, None] / 4.0
    V = rng.standard_normal((1, 2, N, D))
    Q, K, V = (x.astype(np.float16) for x in (Q, K, V))
    for causal in (False, True):
        ref = oracle.attention(Q, K, V, causal=causal)
        got = run(lib, Q, K, V, causal, kernel=KERNELS[kernel])
        assert not np.isnan(got).any()
        assert_parity(got, ref, ("rising", causal, kernel))


@pytest.mark.parametrize("kernel,D", [("block_serial", 64), ("block_serial", 128), ("pipelined", 64),
                                      ("pipelined", 128)])
@pytest.mark.parametrize("key", [650, 700])
def test_dominant_late_key_forces_rescale(lib, kernel, D, key):
    # One key far into the sequence (block 10; key 650 in the first half of its 64-key block, 700 in the
    # second) whose score passes the earlier keys' maximum by a log2 margin from about -1 to 58, depending on
    # the row, D and beta: its probability against the stale reference would overflow fp16 unless the lazy
    # rescale fires.
    # The kernels take that decision from each lane's sum of the block's probabilities, not the block maximum,
    # so a lane holding that one key must trigger it (rows past the threshold), and rows below the threshold
    # must keep the old reference.
    rng = np.random.default_rng(key + D)
    N = 900
    Q = rng.standard_normal((1, 2, N, D))
    Q[..., 0] += 3.0                                     # every row leans on dimension 0
    K = rng.standard_normal((1, 2, N, D)) * 0.25
    V = rng.standard_normal((1, 2, N, D))
    for beta in (20.0, 60.0):
        Kb = K.copy()
        Kb[:, :, key, :] = 0.0
        Kb[:, :, key, 0] = beta
        Q16, K16, V16 = (x.astype(np.float16) for x in (Q, Kb, V))
        for causal in (False, True):
            ref = oracle.attention(Q16, K16, V16, causal=causal)
            got = run(lib, Q16, K16, V16, causal, kernel=KERNELS[kernel])
            assert np.isfinite(got).all(), (kernel, D, key, beta, causal)
            assert_parity(got, ref, ("dominant key", kernel, D, key, beta, causal))


def _slab_rows(w, max_slabs=8):
    """Flat row indices of whole (batch, head) slabs: every slab when there are at most max_slabs of them,
    else the first, the last, the middle and seeded others, max_slabs in all."""
    nslab = w.B * w.H
    if nslab <= max_slabs:
        slabs = list(range(nslab))
    else:
        rng = np.random.default_rng(w.seed)
        pick = {0, nslab - 1, (w.B // 2) * w.H + w.H // 2}
        while len(pick) < max_slabs:
            pick.add(int(rng.integers(0, nslab)))
        slabs = sorted(pick)
    return slabs, np.concatenate([np.arange(sl * w.Nq, (sl + 1) * w.Nq, dtype=np.int64) for sl in slabs])


@pytest.mark.parametrize("name", list(workloads.ATTENTION_WORKLOADS))
def test_workloads_whole_slabs(lib, name):
    # Whole (batch, head) slabs of the full-size workloads: every query row of a slab against the oracle.
    # The two small workloads (32 and 8 slabs) are covered completely.
    w = workloads.ATTENTION_WORKLOADS[name]
    Q, K, V = workloads.make_attention_inputs(w)
    got = run(lib, Q, K, V, w.causal).reshape(-1, w.D)
    slabs, rows = _slab_rows(w, max_slabs=8 if w.Nq >= 4096 else 32)
    ref = oracle.attention_rows(Q, K, V, rows, causal=w.causal)
    assert_parity(got[rows], ref, (name, slabs))
    assert not np.isnan(got).any()
    if w.B * w.H <= 32:
        assert len(slabs) == w.B * w.H


def test_errors_and_empty(lib):
    import dense_tiled_gemm_04_amd as g
    z = lambda *s: torch.zeros(s, dtype=torch.float16, device="cuda")
    assert tuple(g.flash_attn(z(1, 1, 0, 64), z(1, 1, 5, 64), z(1, 1, 5, 64)).shape) == (1, 1, 0, 64)
    with pytest.raises(g.GemmError):
        g.flash_attn(z(1, 1, 4, 96), z(1, 1, 4, 96), z(1, 1, 4, 96))
    with pytest.raises(g.GemmError):
        g.flash_attn(z(1, 1, 4, 64), z(1, 1, 0, 64), z(1, 1, 0, 64))
    with pytest.raises(ValueError):
        g.flash_attn(z(1, 1, 4, 64), z(1, 1, 4, 64), z(1, 1, 5, 64))


def test_determinism(lib):
    import dense_tiled_gemm_04_amd as g
    Q, K, V = (dev(x) for x in workloads.make_attention_inputs("attn_b4_h32_n4096_d128_causal", B=1, H=2, Nq=1024,
                                                               Nkv=1024))
    a = g.flash_attn(Q, K, V, causal=True)
    b = g.flash_attn(Q, K, V, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("name", list(workloads.ATTENTION_WORKLOADS))
def test_block_serial_kernel_whole_slabs(lib, name):
    # The block-serial kernel, no longer the default at either head dimension, forced on the full-size
    # workloads: whole (batch, head) slabs against the oracle (2 slabs of each 4096-token workload, 8 otherwise).
    w = workloads.ATTENTION_WORKLOADS[name]
    Q, K, V = workloads.make_attention_inputs(w)
    got = run(lib, Q, K, V, w.causal, kernel=KERNELS["block_serial"]).reshape(-1, w.D)
    slabs, rows = _slab_rows(w, max_slabs=2 if w.Nq >= 4096 else 8)
    ref = oracle.attention_rows(Q, K, V, rows, causal=w.causal)
    assert_parity(got[rows], ref, (name, slabs))
    assert not np.isnan(got).any()
