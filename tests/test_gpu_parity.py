"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Every comparison uses the same seeded inputs on both sides.  Sizes here span
several tiles with ragged tails; every workload shape is checked completely,
element by element against the oracle's full result, in the launch
configuration the benchmark uses (the default dispatch), with B given as
B[K][N] and as Bt[N][K].
"""
import numpy as np
import pytest

import oracle
import workloads
from parity import assert_parity, metrics, ulp_distance

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def run(lib, A, B, bias, epi, config=None):
    out = lib.gemm_f16(dev(A), dev(B), dev(bias) if bias is not None else None, epi, config=config)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def configs_for(lib, M, N, K, epi):
    """All compiled configs able to run this (aligned, contiguous) call."""
    out = []
    for c in lib.configs():
        if c["b_transposed"]:
            continue
        if c["kind"] == "skinny" and M > c["bm"]:
            continue
        if c["loader"] == "dma" and K % c["bk"] != 0:
            continue
        if c["loader"] == "buf" and K % 8 != 0:
            continue
        if c["kind"] == "skinny" or c["loader"] == "dma":
            if K % 8 or N % 8:
                continue
        out.append(c["idx"])
    return out


# ---------------------------------------------------------------------------
# every config x every epilogue on small ragged shapes
# ---------------------------------------------------------------------------
SHAPES = [
    (300, 520, 256),     # several 128/256 tiles, ragged M and N, K multiple of 64
    (257, 136, 192),     # one row past a 256 tile
    (130, 264, 200),     # K tail (200 = 3*64 + 8)
    (16, 1032, 384),     # skinny
    (45, 200, 136),      # skinny, 3 m-blocks, ragged N panel, K tail
    (64, 64, 64),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("epi", ["none", "bias", "bias_gelu"])
def test_all_configs_small(lib, shape, epi):
    M, N, K = shape
    A, B, bias = workloads.make_inputs("mlp_up_8192x16384x4096", M=M, N=N, K=K)
    if epi == "none":
        bias = None
    ref = oracle.gemm(A, B, bias, epi)
    cfgs = configs_for(lib, M, N, K, epi)
    assert cfgs
    for idx in cfgs:
        got = run(lib, A, B, bias, epi, config=idx)
        m = assert_parity(got, ref, (shape, epi, lib.config_info(idx)["name"]))
        assert m["frac_exact"] > 0.97, m
    got = run(lib, A, B, bias, epi)  # default dispatch
    assert_parity(got, ref, (shape, epi, "default"))


@pytest.mark.parametrize("shape", [(333, 277, 100), (17, 33, 9), (1, 1, 1), (5, 3001, 7), (259, 129, 1000)])
@pytest.mark.parametrize("epi", ["none", "bias", "bias_gelu"])
def test_unaligned_shapes(lib, shape, epi):
    M, N, K = shape
    A, B, bias = workloads.make_inputs("ragged_4095x3001x1000", M=M, N=N, K=K)
    if epi == "none":
        bias = None
    ref = oracle.gemm(A, B, bias, epi)
    got = run(lib, A, B, bias, epi)
    assert_parity(got, ref, (shape, epi))


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------
def test_workload_gemm_256_full(lib):
    A, B, bias = workloads.make_inputs("gemm_256")
    ref = oracle.gemm(A, B)
    got = run(lib, A, B, None, "none")
    m = assert_parity(got, ref, "gemm_256")
    assert m["frac_exact"] > 0.99


def test_workload_ragged_full(lib):
    w = workloads.WORKLOADS["ragged_4095x3001x1000"]
    A, B, bias = workloads.make_inputs(w)
    ref = oracle.gemm(A, B, bias, w.epilogue)
    got = run(lib, A, B, bias, w.epilogue)
    m = assert_parity(got, ref, w.name)
    assert m["frac_exact"] > 0.99


def test_workload_skinny_full(lib):
    w = workloads.WORKLOADS["skinny_16x16384x8192"]
    A, B, bias = workloads.make_inputs(w)
    ref = oracle.gemm(A, B, bias, w.epilogue)
    got = run(lib, A, B, bias, w.epilogue)
    m = assert_parity(got, ref, w.name)
    assert m["frac_exact"] > 0.97


_FULL_REF = {}


def _full_reference(name):
    """Inputs and the oracle's complete fp16 result of a workload, computed once per session."""
    if name not in _FULL_REF:
        _FULL_REF.clear()  # one large workload in memory at a time
        w = workloads.WORKLOADS[name]
        A, B, bias = workloads.make_inputs(w)
        _FULL_REF[name] = (A, B, bias, oracle.gemm(A, B, bias, w.epilogue))
    return _FULL_REF[name]


@pytest.mark.parametrize("name", ["gemm_4096", "mlp_up_8192x16384x4096"])
@pytest.mark.parametrize("bt", [False, True])
def test_workload_large_full(lib, name, bt):
    import dense_tiled_gemm_04_amd as g
    w = workloads.WORKLOADS[name]
    A, B, bias, ref = _full_reference(name)
    Bdev = dev(np.ascontiguousarray(B.T)) if bt else dev(B)
    out = g.gemm_f16(dev(A), Bdev, dev(bias) if bias is not None else None, w.epilogue, b_transposed=bt)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    del out, Bdev
    m = assert_parity(got, ref, (name, "Bt" if bt else "B"))
    assert m["frac_exact"] > 0.97, m
    assert m["n"] == w.M * w.N


# ---------------------------------------------------------------------------
# bit-exact closed forms
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("K", [1, 64, 1000, 4096, 8192])
def test_all_ones_exact(lib, K):
    for M, N in ((256, 256), (16, 512), (100, 72)):
        A = np.ones((M, K), np.float16)
        B = np.ones((K, N), np.float16)
        got = run(lib, A, B, None, "none")
        assert np.all(got.astype(np.float64) == float(np.float16(K)))


def test_identity_passes_every_finite_fp16(lib):
    # A = I, B = every finite binary16 pattern (non-finite ones replaced by 0):
    # C must reproduce B bit for bit (up to the sign of zero) -> no subnormal
    # flushing in the MFMA path, exact decode, exact store.
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7C00) != 0x7C00
    bits = np.where(finite, bits, 0).astype(np.uint16)
    B = bits.view(np.float16).reshape(256, 256)
    A = np.eye(256, dtype=np.float16)
    for idx in configs_for(lib, 256, 256, 256, "none"):
        got = run(lib, A, B, None, "none", config=idx)
        assert np.array_equal(got.view(np.uint16) & 0x7FFF, B.view(np.uint16) & 0x7FFF), lib.config_info(idx)
        nz = (B.view(np.uint16) & 0x7FFF) != 0
        assert np.array_equal(got.view(np.uint16)[nz], B.view(np.uint16)[nz])


def test_rank1_round_to_nearest_even(lib):
    # C = fp16(u_i * v_j) (exact products), including exact ties that separate
    # round-to-nearest-even from truncation.
    rng = np.random.default_rng(5)
    M, N, K = 64, 64, 64
    u = rng.uniform(-2, 2, M).astype(np.float16)
    v = rng.uniform(-2, 2, N).astype(np.float16)
    u[0], v[0] = np.float16(1 + 2 ** -10), np.float16(1.5)
    A = np.zeros((M, K), np.float16)
    A[:, 7] = u
    B = workloads.random_f16(6, (K, N))
    B[7, :] = v
    ref = np.outer(u.astype(np.float64), v.astype(np.float64)).astype(np.float16)
    for idx in configs_for(lib, M, N, K, "none"):
        got = run(lib, A, B, None, "none", config=idx)
        assert np.array_equal(got.view(np.uint16), ref.view(np.uint16)), lib.config_info(idx)
    assert float(got[0, 0]) == 1.5 + 2 * 2 ** -10


def test_bias_only_exact(lib):
    # A = 0: C = bias broadcast, and gelu(bias) within one fp16 ulp of the oracle
    M, N, K = 100, 264, 64
    A = np.zeros((M, K), np.float16)
    B = workloads.random_f16(7, (K, N))
    bias = workloads.random_f16(8, (N,), -6, 6)
    got = run(lib, A, B, bias, "bias")
    assert np.array_equal(got.astype(np.float64), np.broadcast_to(bias.astype(np.float64), (M, N)))
    got = run(lib, A, B, bias, "bias_gelu")
    ref = oracle.gemm(A, B, bias, "bias_gelu")
    assert ulp_distance(got, ref).max() <= 1


@pytest.mark.parametrize("M", [16, 256, 72])
def test_gelu_epilogue_every_finite_fp16(lib, M):
    # A = 0, so C[i][j] = gelu(bias[j]) with bias = every finite binary16 value:
    # the fused GELU of each path (skinny M = 16, DMA tile M = 256, register
    # tile M = 72 with K = 8) against the oracle, within one fp16 ulp, and
    # bit-identical on at least 99.5% of the values.
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7C00) != 0x7C00]                       # 63488 finite patterns
    bias = bits.view(np.float16)
    N = bias.shape[0]
    K = 8 if M == 72 else 64
    A = np.zeros((M, K), np.float16)
    B = workloads.random_f16(11, (K, N))
    ref = oracle.gemm(A[:1], B, bias, "bias_gelu")[0]
    got = run(lib, A, B, bias, "bias_gelu")
    for i in (0, M - 1):
        u = ulp_distance(got[i], ref)
        assert u.max() <= 1, (M, i, int(u.argmax()), float(bias[u.argmax()]))
        assert np.mean(u == 0) >= 0.995, (M, i, float(np.mean(u == 0)))
    assert np.array_equal(got[0].view(np.uint16), got[M - 1].view(np.uint16))


@pytest.mark.parametrize("shape", [(16, 264, 64), (256, 520, 128), (72, 264, 8)])
def test_epilogues_on_non_finite_sums(lib, shape):
    # Rows whose fp32 sum is +inf, -inf, NaN (a NaN input; inf - inf) or past the fp16 range (+-131008), among
    # finite rows, through every epilogue of every path able to run the shape.  Against the oracle: GELU(+inf)
    # = +inf, GELU(-inf) = NaN (x Phi(x) is -inf * 0 there), NaN stays NaN, +131008 rounds to +inf and
    # GELU(-131008) underflows to -0.  Non-NaN results of the special rows must match bit for bit (zeros of
    # either sign), NaN positions exactly, and the finite rows keep the usual bar.
    import dense_tiled_gemm_04_amd as g

    M, N, K = shape
    rng = np.random.default_rng(41)
    A = rng.uniform(-1, 1, (M, K)).astype(np.float16)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float16)
    B[0] = 1.0
    if K > 1:
        B[1] = 1.0
    bias = workloads.random_f16(12, (N,), -3, 3)
    rows = [0, 1, M // 2, M // 2 + 1, M - 2, M - 1]
    A[rows[0], 0] = np.inf
    A[rows[1], 0] = -np.inf
    A[rows[2], 0] = np.nan
    A[rows[3], 0], A[rows[3], 1] = np.inf, -np.inf
    A[rows[4], 0], A[rows[4], 1] = 65504.0, 65504.0
    A[rows[5], 0], A[rows[5], 1] = -65504.0, -65504.0
    keep = np.setdiff1d(np.arange(M), rows)
    Bt = np.ascontiguousarray(B.T)
    for epi in ("none", "bias", "bias_gelu"):
        b = None if epi == "none" else bias
        ref = oracle.gemm(A, B, b, epi)
        assert np.isnan(ref[rows[1]]).all() == (epi == "bias_gelu") and np.isnan(ref[rows[2:4]]).all()
        calls = [(False, idx) for idx in configs_for(lib, M, N, K, epi) + [None]]
        calls += [(True, c["idx"]) for c in lib.configs() if c["b_transposed"]] + [(True, None)]
        for bt, idx in calls:
            try:
                out = g.gemm_f16(dev(A), dev(Bt) if bt else dev(B), None if b is None else dev(b), epi,
                                 b_transposed=bt, config=idx)
            except g.GemmError as e:
                assert bt and idx is not None and e.status == 6, e  # a Bt config that does not take this shape
                continue
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            name = (epi, bt, "default" if idx is None else lib.config_info(idx)["name"])
            assert_parity(got[keep], ref[keep], name)
            gs, rs = got[rows], ref[rows]
            assert np.array_equal(np.isnan(gs), np.isnan(rs)), name
            fin = ~np.isnan(rs)
            assert np.array_equal(gs[fin].astype(np.float64), rs[fin].astype(np.float64)), name
            assert np.array_equal(np.signbit(gs[fin]), np.signbit(rs[fin])), name


# ---------------------------------------------------------------------------
# edges: canaries, misaligned views, degenerate sizes, determinism
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(300, 520, 256), (16, 1032, 384), (333, 277, 100)])
def test_canaries_untouched(lib, shape):
    M, N, K = shape
    A, B, bias = workloads.make_inputs("ragged_4095x3001x1000", M=M, N=N, K=K)
    ref = oracle.gemm(A, B, bias, "bias")
    pad = 4096
    buf = torch.full((M * N + 2 * pad,), -7.0, dtype=torch.float16, device="cuda")
    out = buf[pad:pad + M * N].view(M, N)
    import dense_tiled_gemm_04_amd as g
    g.gemm_f16(dev(A), dev(B), dev(bias), "bias", out=out)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:pad] == np.float16(-7.0)) and np.all(host[pad + M * N:] == np.float16(-7.0))
    assert_parity(host[pad:pad + M * N].reshape(M, N), ref, shape)


def test_misaligned_views(lib):
    M, N, K = 130, 136, 72
    A, B, bias = workloads.make_inputs("ragged_4095x3001x1000", M=M, N=N, K=K)
    ref = oracle.gemm(A, B, bias, "bias_gelu")
    ab = torch.zeros(M * K + 1, dtype=torch.float16, device="cuda")
    bb = torch.zeros(K * N + 1, dtype=torch.float16, device="cuda")
    cb = torch.zeros(M * N + 1, dtype=torch.float16, device="cuda")
    ab[1:] = dev(A).reshape(-1)
    bb[1:] = dev(B).reshape(-1)
    import dense_tiled_gemm_04_amd as g
    Av, Bv, Cv = ab[1:].view(M, K), bb[1:].view(K, N), cb[1:].view(M, N)
    cfg = g.config_info(g.select_config(Av, Bv, dev(bias), "bias_gelu", out=Cv))
    assert cfg["loader"] == "buf"
    g.gemm_f16(Av, Bv, dev(bias), "bias_gelu", out=Cv)
    torch.cuda.synchronize()
    assert_parity(Cv.cpu().numpy(), ref, "misaligned")
    # every configuration that accepts the misaligned views
    for c in lib.configs():
        if c["kind"] != "tile" or c["loader"] == "dma" or c["b_transposed"]:
            continue
        Cv.zero_()
        g.gemm_f16(Av, Bv, dev(bias), "bias_gelu", out=Cv, config=c["idx"])
        torch.cuda.synchronize()
        assert_parity(Cv.cpu().numpy(), ref, ("misaligned", c["name"]))


# ---------------------------------------------------------------------------
# buffer LDS-DMA loader: unaligned rows, K tails, odd N and the end of B
# ---------------------------------------------------------------------------
def _buf_configs(lib):
    out = [c["idx"] for c in lib.configs() if c["kind"] == "tile" and c["loader"] == "buf" and not c["b_transposed"]]
    assert out
    return out


@pytest.mark.parametrize("shape", [(333, 277, 104), (259, 129, 1000), (130, 3001, 200), (1, 1, 8), (17, 33, 8),
                                   (300, 515, 64), (513, 7, 40)])
def test_buffer_loader_shapes(lib, shape):
    M, N, K = shape
    A, B, bias = workloads.make_inputs("ragged_4095x3001x1000", M=M, N=N, K=K)
    ref = oracle.gemm(A, B, bias, "bias")
    for idx in _buf_configs(lib):
        got = run(lib, A, B, bias, "bias", config=idx)
        m = assert_parity(got, ref, (shape, lib.config_info(idx)["name"]))
        assert m["frac_exact"] > 0.97, m


@pytest.mark.parametrize("shape", [(70, 301, 200), (5, 3, 8), (260, 2049, 64)])
def test_buffer_loader_last_element_of_B(lib, shape):
    # B is zero except its last element, so C[:, N-1] = A[:, K-1] * B[K-1][N-1] and every other column is 0.
    # With odd N the chunk holding that element may start off the dword grid of B's end.
    M, N, K = shape
    A, _, _ = workloads.make_inputs("ragged_4095x3001x1000", M=M, N=N, K=K)
    B = np.zeros((K, N), np.float16)
    B[K - 1, N - 1] = np.float16(1.5)
    ref = oracle.gemm(A, B)
    for idx in _buf_configs(lib):
        got = run(lib, A, B, None, "none", config=idx)
        assert np.array_equal(got.view(np.uint16), ref.view(np.uint16)), lib.config_info(idx)["name"]


def test_buffer_loader_B_end_on_page_boundary(lib):
    # Odd N with B ending exactly on a 4 KiB boundary: the buffer loader's 2-byte pad would cross into the
    # next page, so the dispatcher must pick another loader, and a forced buffer config is refused.
    import dense_tiled_gemm_04_amd as g
    M, N, K = 100, 301, 64
    A, B, bias = workloads.make_inputs("ragged_4095x3001x1000", M=M, N=N, K=K)
    ref = oracle.gemm(A, B, bias, "bias")
    store = torch.zeros(K * N + 8192, dtype=torch.float16, device="cuda")
    end = store.data_ptr() + store.numel() * 2
    end_page = (end // 4096) * 4096
    first = (end_page - K * N * 2 - store.data_ptr()) // 2
    assert first >= 0
    Bv = store[first:first + K * N].view(K, N)
    assert (Bv.data_ptr() + K * N * 2) % 4096 == 0
    Bv.copy_(dev(B))
    cfg = g.config_info(g.select_config(dev(A), Bv, dev(bias), "bias"))
    assert cfg["loader"] == "reg"
    got = g.gemm_f16(dev(A), Bv, dev(bias), "bias")
    torch.cuda.synchronize()
    assert_parity(got.cpu().numpy(), ref, "page-end B")
    with pytest.raises(Exception):
        g.gemm_f16(dev(A), Bv, dev(bias), "bias", config=_buf_configs(lib)[0])


def test_k_tail_does_not_read_next_row(lib):
    # Infinities in column 0 of some rows of A.  A loader that let the next row's first elements into the
    # K tail of a row (multiplied by the zero rows of B past K) would turn that row into NaN.
    M, N, K = 130, 264, 200
    A, B, bias = workloads.make_inputs("ragged_4095x3001x1000", M=M, N=N, K=K)
    B[0] = np.where(B[0] == 0, np.float16(0.5), B[0])
    inf_rows = [1, 64, 65, 129]
    A[inf_rows, 0] = np.float16(np.inf)
    ref = oracle.gemm(A, B, bias, "bias")
    keep = np.setdiff1d(np.arange(M), inf_rows)
    cfgs = configs_for(lib, M, N, K, "bias") + [None]
    for idx in cfgs:
        got = run(lib, A, B, bias, "bias", config=idx)
        name = lib.config_info(idx)["name"] if idx is not None else "default"
        assert_parity(got[keep], ref[keep], ("finite rows", name))
        assert np.array_equal(got[inf_rows].view(np.uint16), ref[inf_rows].view(np.uint16)), name


def test_degenerate_sizes(lib):
    import dense_tiled_gemm_04_amd as g
    bias = workloads.random_f16(9, (40,), -3, 3)
    for epi in ("none", "bias", "bias_gelu"):
        A = torch.zeros((30, 0), dtype=torch.float16, device="cuda")
        B = torch.zeros((0, 40), dtype=torch.float16, device="cuda")
        out = torch.full((30, 40), 5.0, dtype=torch.float16, device="cuda")
        g.gemm_f16(A, B, dev(bias) if epi != "none" else None, epi, out=out)
        torch.cuda.synchronize()
        ref = oracle.gemm(np.zeros((30, 0), np.float16), np.zeros((0, 40), np.float16),
                          bias if epi != "none" else None, epi)
        assert np.array_equal(out.cpu().numpy().view(np.uint16), ref.view(np.uint16))
    e = g.gemm_f16(torch.zeros((0, 8), dtype=torch.float16, device="cuda"),
                   torch.zeros((8, 8), dtype=torch.float16, device="cuda"))
    assert tuple(e.shape) == (0, 8)


@pytest.mark.parametrize("name", ["gemm_4096", "skinny_16x16384x8192", "ragged_4095x3001x1000"])
def test_determinism(lib, name):
    w = workloads.WORKLOADS[name]
    A, B, bias = workloads.make_inputs(w)
    a, b = dev(A), dev(B)
    bb = dev(bias) if bias is not None else None
    import dense_tiled_gemm_04_amd as g
    c1 = g.gemm_f16(a, b, bb, w.epilogue)
    c2 = g.gemm_f16(a, b, bb, w.epilogue)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


def test_torch_front_end_errors(lib):
    import dense_tiled_gemm_04_amd as g
    a = torch.zeros((4, 8), dtype=torch.float16, device="cuda")
    b = torch.zeros((8, 4), dtype=torch.float16, device="cuda")
    with pytest.raises(TypeError):
        g.gemm_f16(a.float(), b)
    with pytest.raises(ValueError):
        g.gemm_f16(a, torch.zeros((7, 4), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        g.gemm_f16(a, b, None, "bias")
    with pytest.raises(ValueError):
        g.gemm_f16(a.t(), b.t())


def _same_f32_bits(x, y):
    x, y = np.asarray(x, np.float32), np.asarray(y, np.float32)
    both_nan = np.isnan(x) & np.isnan(y)
    return bool(np.all(both_nan | (x.view(np.uint32) == y.view(np.uint32))))


@pytest.mark.parametrize("n", [1, 7, 1024, 1000003, 64 * 1024 * 1024 + 5])
def test_vector_add_matches_oracle(lib, n):
    # The pages' first kernel: float32 C = A + B, every element the IEEE binary32 sum, so bit-exact.
    import dense_tiled_gemm_04_amd as g
    a, b = workloads.make_vector_add_inputs(n, seed=12 + n % 97)
    k = min(n, 4096)  # a block of arbitrary bit patterns: subnormals, infinities, NaNs, ties
    a[:k] = workloads.random_f32_bits(1, k)
    b[:k] = workloads.random_f32_bits(2, k)
    ref = oracle.vector_add(a, b)
    z = g.vector_add(dev(a), dev(b))
    torch.cuda.synchronize()
    assert _same_f32_bits(z.cpu().numpy(), ref)


def test_vector_add_unaligned_views(lib):
    # views 4 bytes off the 16-byte grid take the scalar kernel; still bit-exact against the oracle
    import dense_tiled_gemm_04_amd as g
    x, y = workloads.make_vector_add_inputs(100_003, seed=13)
    x[:2048] = workloads.random_f32_bits(3, 2048)
    dx = dev(x)
    z = g.vector_add(dx[1:], dx[:-1])
    torch.cuda.synchronize()
    assert _same_f32_bits(z.cpu().numpy(), oracle.vector_add(x[1:], x[:-1]))


# ---------------------------------------------------------------------------
# the event-median timing helper
# ---------------------------------------------------------------------------
def test_gemm_f16_time_median_and_result(lib):
    import dense_tiled_gemm_04_amd as g
    M = N = K = 2048
    A, B, _ = workloads.make_inputs("gemm_4096", M=M, N=N, K=K)
    dA, dB = dev(A), dev(B)
    dC = torch.empty((M, N), dtype=torch.float16, device="cuda")
    sh = torch.cuda.current_stream().cuda_stream
    st, med = g.gemm_f16_time_raw(M, N, K, dA.data_ptr(), dB.data_ptr(), None, dC.data_ptr(), 0, 51, sh)
    assert st == 0 and med > 0
    # the output of the timed launches is the product
    r = np.arange(0, M, 37)
    c = (r * 13) % N
    ref = oracle.gemm_points(A, B, None, "none", r, c)
    assert_parity(dC.cpu().numpy()[r, c][None, :], ref[None, :], "gemm_f16_time output")
    # against the benchmark's way of timing: one event pair around back-to-back launches
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    e0.record(stream)
    for _ in range(51):
        assert g.gemm_f16_raw(M, N, K, dA.data_ptr(), dB.data_ptr(), None, dC.data_ptr(), 0, sh) == 0
    e1.record(stream)
    torch.cuda.synchronize()
    avg = e0.elapsed_time(e1) / 51
    assert 0.5 < med / avg < 2.0, (med, avg)
    # a forced configuration, and the empty call
    idx = g.select_config_raw(M, N, K, dA.data_ptr(), dB.data_ptr(), None, dC.data_ptr(), 0)
    st, med2 = g.gemm_f16_time_raw(M, N, K, dA.data_ptr(), dB.data_ptr(), None, dC.data_ptr(), 0, 5, sh, config=idx)
    assert st == 0 and med2 > 0
    assert g.gemm_f16_time_raw(0, N, K, None, None, None, None, 0, 5, sh) == (0, 0.0)


def test_gemm_f16_time_rejects_bad_arguments(lib):
    import dense_tiled_gemm_04_amd as g
    a = torch.zeros((64, 64), dtype=torch.float16, device="cuda")
    p = a.data_ptr()
    assert g.gemm_f16_time_raw(64, 64, 64, p, p, None, p, 0, 0)[0] == 1           # iters < 1
    assert g.gemm_f16_time_raw(64, 64, 64, p, p, None, p, 0, 100001)[0] == 1      # iters too large
    assert g.gemm_f16_time_raw(64, 64, 64, p, p, None, p, 0, 5, config=g.num_configs())[0] == 5
    assert g.gemm_f16_time_raw(-1, 64, 64, p, p, None, p, 0, 5)[0] == 1
    assert g.gemm_f16_time_raw(64, 64, 64, p, p, None, p, 7, 5)[0] == 3


# ---------------------------------------------------------------------------
# strided layouts: A, B and C as column slices of wider row-major arrays
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(300, 520, 256), (333, 277, 104), (16, 1032, 384), (257, 136, 192), (45, 200, 136)])
@pytest.mark.parametrize("pad", [24, 5])
def test_strided_submatrices_every_config(lib, shape, pad):
    import dense_tiled_gemm_04_amd as g
    M, N, K = shape
    A, B, bias = workloads.make_inputs("ragged_4095x3001x1000", M=M, N=N, K=K)
    ref = oracle.gemm(A, B, bias, "bias_gelu")
    lda, ldb, ldc = K + pad, N + pad, N + pad + 8
    Abuf = torch.zeros((M, lda), dtype=torch.float16, device="cuda")
    Bbuf = torch.zeros((K, ldb), dtype=torch.float16, device="cuda")
    Abuf[:, pad:pad + K] = dev(A)
    Bbuf[:, 0:N] = dev(B)
    Av, Bv = Abuf[:, pad:pad + K], Bbuf[:, 0:N]
    assert Av.stride() == (lda, 1) and Bv.stride() == (ldb, 1)
    db = dev(bias)
    ran = []
    for c in lib.configs() + [None]:
        Cbuf = torch.full((M, ldc), -7.0, dtype=torch.float16, device="cuda")
        Cv = Cbuf[:, 8:8 + N]
        try:
            g.gemm_f16(Av, Bv, db, "bias_gelu", out=Cv, config=None if c is None else c["idx"])
        except g.GemmError as e:
            assert c is not None and e.status == 6, e   # only "this config cannot run this call"
            continue
        torch.cuda.synchronize()
        host = Cbuf.cpu().numpy()
        name = "default" if c is None else c["name"]
        assert np.all(host[:, :8] == np.float16(-7.0)) and np.all(host[:, 8 + N:] == np.float16(-7.0)), name
        assert_parity(host[:, 8:8 + N], ref, (shape, pad, name))
        ran.append(name)
    assert "default" in ran and len(ran) >= 3, ran


# ---------------------------------------------------------------------------
# B given transposed: Bt [N][K] (a linear layer's weight layout), C = A . Bt^T
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(300, 520, 256), (333, 277, 104), (16, 1032, 384), (257, 136, 192),
                                   (130, 264, 200), (5, 3001, 7), (64, 64, 64)])
@pytest.mark.parametrize("epi", ["none", "bias_gelu"])
def test_b_transposed_every_config(lib, shape, epi):
    import dense_tiled_gemm_04_amd as g
    M, N, K = shape
    A, B, bias = workloads.make_inputs("mlp_up_8192x16384x4096", M=M, N=N, K=K)
    if epi == "none":
        bias = None
    ref = oracle.gemm(A, B, bias, epi)
    Bt = dev(np.ascontiguousarray(B.T))
    dA, db = dev(A), (dev(bias) if bias is not None else None)
    ran = []
    for c in [c for c in lib.configs() if c["b_transposed"]] + [None]:
        try:
            out = g.gemm_f16(dA, Bt, db, epi, b_transposed=True, config=None if c is None else c["idx"])
        except g.GemmError as e:
            assert c is not None and e.status == 6, e
            continue
        torch.cuda.synchronize()
        name = "default" if c is None else c["name"]
        m = assert_parity(out.cpu().numpy(), ref, (shape, epi, name))
        assert m["frac_exact"] > 0.97, (name, m)
        ran.append(name)
    assert "default" in ran and len(ran) >= 2, ran


def test_b_transposed_strided_and_k_tail_isolation(lib):
    # Bt as a column slice of a wider array, K not a multiple of the K-block, and infinities in column 0 of some
    # Bt rows: a loader that let the next Bt row into the K tail of a row (times the zeroed A tail) would turn
    # a whole output column into NaN.
    import dense_tiled_gemm_04_amd as g
    M, N, K = 130, 264, 200
    A, B, bias = workloads.make_inputs("ragged_4095x3001x1000", M=M, N=N, K=K)
    A[:, 0] = np.where(A[:, 0] == 0, np.float16(0.5), A[:, 0])
    Bt = np.ascontiguousarray(B.T)
    inf_cols = [1, 64, 65, 263]
    Bt[inf_cols, 0] = np.float16(np.inf)
    ref = oracle.gemm(A, np.ascontiguousarray(Bt.T), bias, "bias")
    keep = np.setdiff1d(np.arange(N), inf_cols)
    buf = torch.zeros((N, K + 40), dtype=torch.float16, device="cuda")
    buf[:, 8:8 + K] = dev(Bt)
    Btv = buf[:, 8:8 + K]
    for c in [c for c in lib.configs() if c["b_transposed"]] + [None]:
        try:
            out = g.gemm_f16(dev(A), Btv, dev(bias), "bias", b_transposed=True,
                             config=None if c is None else c["idx"])
        except g.GemmError as e:
            assert c is not None and e.status == 6, e
            continue
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        name = "default" if c is None else c["name"]
        assert_parity(got[:, keep], ref[:, keep], ("finite columns", name))
        assert np.array_equal(got[:, inf_cols].view(np.uint16), ref[:, inf_cols].view(np.uint16)), name


# ---------------------------------------------------------------------------
# skinny M with B given transposed (decode through a linear layer's weight)
# ---------------------------------------------------------------------------
def test_b_transposed_skinny_workload_full(lib):
    import dense_tiled_gemm_04_amd as g
    w = workloads.WORKLOADS["skinny_16x16384x8192"]
    A, B, bias = workloads.make_inputs(w)
    ref = oracle.gemm(A, B, bias, w.epilogue)
    out = g.gemm_f16(dev(A), dev(np.ascontiguousarray(B.T)), dev(bias), w.epilogue, b_transposed=True)
    torch.cuda.synchronize()
    m = assert_parity(out.cpu().numpy(), ref, w.name + " (Bt)")
    assert m["frac_exact"] > 0.97


@pytest.mark.parametrize("M", [1, 7, 16, 17, 32, 33, 64])
def test_b_transposed_skinny_shapes_and_k_tail_isolation(lib, M):
    # every skinny Bt config (and the default) on K with a tail past the 128-deep stage, Bt as a column slice of a
    # wider array, and infinities in column 0 of some Bt rows: a k-chunk past K that read the next Bt row would
    # put an infinity into the zeroed A tail's product and turn a whole output column into NaN.
    import dense_tiled_gemm_04_amd as g
    N, K = 264, 200
    A, B, bias = workloads.make_inputs("skinny_16x16384x8192", M=M, N=N, K=K)
    A[:, 0] = np.where(A[:, 0] == 0, np.float16(0.5), A[:, 0])
    Bt = np.ascontiguousarray(B.T)
    inf_cols = [1, 64, 65, 263]
    Bt[inf_cols, 0] = np.float16(np.inf)
    ref = oracle.gemm(A, np.ascontiguousarray(Bt.T), bias, "bias_gelu")
    keep = np.setdiff1d(np.arange(N), inf_cols)
    buf = torch.zeros((N, K + 40), dtype=torch.float16, device="cuda")
    buf[:, 8:8 + K] = dev(Bt)
    Btv = buf[:, 8:8 + K]
    ran = []
    for c in [c for c in lib.configs() if c["b_transposed"] and c["kind"] == "skinny"] + [None]:
        try:
            out = g.gemm_f16(dev(A), Btv, dev(bias), "bias_gelu", b_transposed=True,
                             config=None if c is None else c["idx"])
        except g.GemmError as e:
            assert c is not None and e.status == 6, e
            continue
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        name = "default" if c is None else c["name"]
        assert_parity(got[:, keep], ref[:, keep], (M, "finite columns", name))
        assert np.array_equal(got[:, inf_cols].view(np.uint16), ref[:, inf_cols].view(np.uint16)), (M, name)
        ran.append(name)
    assert "default" in ran and (M > 32 or len(ran) >= 2), ran


def test_mfma16_configs_agree_bitwise(lib):
    # Every configuration on the 16x16x32 MFMA sums each output's K products in the same order (k-steps of 32 in
    # increasing k, the MFMA's own order inside a step), whatever its tile width, loader, LDS-staged epilogue or B
    # layout, and feeds the MFMA the same values in the same lanes.  With the bias epilogue (one fp32 add: nothing
    # for the compiler to contract) their outputs must be bit-identical, and each matches the oracle.
    import dense_tiled_gemm_04_amd as g
    M, N, K = 600, 776, 320  # several 256-row and 192/256-column tiles, ragged M and N, K a multiple of 64
    A, B, bias = workloads.make_inputs("ragged_4095x3001x1000", M=M, N=N, K=K)
    Bt = np.ascontiguousarray(B.T)
    ref = oracle.gemm(A, B, bias, "bias")
    outs = {}
    for c in lib.configs():
        if c["kind"] != "tile" or c["mfma"] != 16:
            continue
        try:
            if c["b_transposed"]:
                out = g.gemm_f16(dev(A), dev(Bt), dev(bias), "bias", b_transposed=True, config=c["idx"])
            else:
                out = g.gemm_f16(dev(A), dev(B), dev(bias), "bias", config=c["idx"])
        except g.GemmError as e:
            assert e.status == 6, (c["name"], e)
            continue
        torch.cuda.synchronize()
        outs[c["name"]] = out.cpu().numpy()
    names = sorted(outs)
    assert len(names) >= 4, names
    assert_parity(outs[names[0]], ref, names[0])
    for n in names[1:]:
        assert np.array_equal(outs[n].view(np.uint16), outs[names[0]].view(np.uint16)), (n, names[0])


# ---------------------------------------------------------------------------
# the MFMA throughput calibration kernel
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [16, 32])
def test_mfma_calibration_runs_and_stamps(lib, shape):
    import dense_tiled_gemm_04_amd as g
    wgs = 8
    stamps = torch.zeros((wgs, 4), dtype=torch.int64, device="cuda")
    sink = torch.full((wgs * 512,), float("nan"), dtype=torch.float32, device="cuda")
    assert g.mfma_calibration_raw(shape, 200, wgs, stamps.data_ptr(), sink.data_ptr()) == 0
    torch.cuda.synchronize()
    st = stamps.cpu().numpy()
    assert np.all(st[:, 1] > st[:, 0]) and np.all(st[:, 3] > st[:, 2])
    # the shader clock the loop saw lies between 0.5 and 3 GHz
    clk = (st[:, 1] - st[:, 0]) / ((st[:, 3] - st[:, 2]) / 100e6)
    assert np.all((clk > 0.5e9) & (clk < 3.0e9)), clk
    assert bool(torch.isfinite(sink).all())
    per_mfma = 2 * 16 * 16 * 32 if shape == 16 else 2 * 32 * 32 * 16
    assert g.mfma_calibration_flops(shape, 200, wgs) == per_mfma * 8 * 8 * 200 * wgs
