"""GPU parity of the row softmax (through the C ABI) against the CPU oracle.

Every kernel path is covered: rows held in the registers of 16 to 64 threads
(cols <= 4096) or of 2 or 4 waves (cols <= 16384), and the two-pass online
kernel (longer rows), with 1 to 8 chunks per thread, at shapes with ragged chunk tails, plus IEEE special values,
in-place calls, misaligned views, canaries around the output and the three
softmax workloads at full size.  The bar is the GEMM's (relative Frobenius
error <= 2e-3, max |y - ref| / (1 + |ref|) <= 1e-2, NaN exactly where the
oracle has NaN), and in addition at most 1 fp16 ulp from the oracle: the fp32
arithmetic is accurate to a few fp32 ulps, so only values within that distance
of a rounding midpoint can land one fp16 ulp away.
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


def run(lib, X, out=None):
    y = lib.softmax_f16(dev(X) if isinstance(X, np.ndarray) else X, out=out)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check(got, ref, what):
    m = assert_parity(got, ref, what)
    assert m["max_ulp"] <= 1, (what, m)
    return m


SHAPES = [
    # register path, a row within one wave: 16, 32 and 64 threads per row, 1..8 chunks per thread
    (1, 1), (5, 7), (64, 64), (33, 129), (257, 256), (33, 500), (30, 513), (130, 1000), (17, 2048), (40, 3001),
    (9, 4096),
    # register path, a row over 2 or 4 waves
    (7, 4097), (5, 8193), (3, 12000), (4, 16384),
    # online path
    (3, 16385), (2, 40000), (2, 100003),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_shapes_every_path(lib, shape):
    rows, cols = shape
    X = workloads.make_softmax_input("softmax_4095x3001", rows=rows, cols=cols)
    ref = oracle.softmax_rows(X)
    got = run(lib, X)
    m = check(got, ref, (shape, lib.softmax_path(rows, cols)))
    assert m["frac_exact"] > 0.98, m


@pytest.mark.parametrize("cols", [6, 500, 3001, 20000])
def test_special_values(lib, cols):
    # per path: -inf entries, an all -inf row, a +inf entry, a NaN entry, a huge-magnitude row
    rng = np.random.default_rng(cols)
    X = (rng.standard_normal((6, cols)) * 2).astype(np.float16)
    X[0, ::3] = -np.inf
    X[1, :] = -np.inf
    X[2, cols // 2] = np.inf
    X[3, cols - 1] = np.nan
    X[4, :] = np.float16(-65504.0)
    X[4, cols // 3] = np.float16(65504.0)
    X[5, :] = np.float16(60000.0)
    ref = oracle.softmax_rows(X)
    got = run(lib, X)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    check(got[ok].reshape(1, -1), ref[ok].reshape(1, -1), ("special", cols))
    assert np.all(got[0, ::3] == 0)
    assert np.all(np.isnan(got[1])) and np.all(np.isnan(got[2])) and np.all(np.isnan(got[3]))


@pytest.mark.parametrize("cols", [300, 3001, 20000])
def test_in_place(lib, cols):
    X = workloads.make_softmax_input("softmax_8192x16384", rows=37, cols=cols)
    ref = oracle.softmax_rows(X)
    t = dev(X)
    lib.softmax_f16(t, out=t)
    torch.cuda.synchronize()
    check(t.cpu().numpy(), ref, ("in place", cols))


@pytest.mark.parametrize("cols", [300, 3001, 20000])
def test_misaligned_views_and_canaries(lib, cols):
    rows = 19
    X = workloads.make_softmax_input("softmax_4095x3001", rows=rows, cols=cols)
    ref = oracle.softmax_rows(X)
    pad = 4099  # odd: both views start 2 bytes off any 4-byte boundary of the allocation
    xb = torch.zeros(rows * cols + 2 * pad, dtype=torch.float16, device="cuda")
    yb = torch.full((rows * cols + 2 * pad,), -7.0, dtype=torch.float16, device="cuda")
    xb[pad:pad + rows * cols] = dev(X).reshape(-1)
    Xv = xb[pad:pad + rows * cols].view(rows, cols)
    Yv = yb[pad:pad + rows * cols].view(rows, cols)
    lib.softmax_f16(Xv, out=Yv)
    torch.cuda.synchronize()
    host = yb.cpu().numpy()
    assert np.all(host[:pad] == np.float16(-7.0)) and np.all(host[pad + rows * cols:] == np.float16(-7.0))
    check(host[pad:pad + rows * cols].reshape(rows, cols), ref, ("misaligned", cols))


def test_empty_and_errors(lib):
    import dense_tiled_gemm_04_amd as g
    e = g.softmax_f16(torch.zeros((0, 8), dtype=torch.float16, device="cuda"))
    assert tuple(e.shape) == (0, 8)
    e = g.softmax_f16(torch.zeros((8, 0), dtype=torch.float16, device="cuda"))
    assert tuple(e.shape) == (8, 0)
    with pytest.raises(TypeError):
        g.softmax_f16(torch.zeros((4, 4), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        g.softmax_f16(torch.zeros((4, 4), dtype=torch.float16, device="cuda"),
                      out=torch.zeros((4, 5), dtype=torch.float16, device="cuda"))


@pytest.mark.parametrize("name", list(workloads.SOFTMAX_WORKLOADS))
def test_workloads_full(lib, name):
    w = workloads.SOFTMAX_WORKLOADS[name]
    X = workloads.make_softmax_input(w)
    ref = oracle.softmax_rows(X)
    got = run(lib, X)
    m = check(got, ref, name)
    assert m["frac_exact"] > 0.99, m


def test_determinism(lib):
    import dense_tiled_gemm_04_amd as g
    X = dev(workloads.make_softmax_input("softmax_8192x16384", rows=512))
    a, b = g.softmax_f16(X), g.softmax_f16(X)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("shape", [(22400, 3001), (65536, 1024)])
def test_streaming_loads_large_matrix(lib, shape):
    # 128 MiB and more: the register path reads X with non-temporal loads
    rows, cols = shape
    assert rows * cols * 2 >= 128 << 20
    X = workloads.make_softmax_input("softmax_8192x16384", rows=rows, cols=cols)
    ref = oracle.softmax_rows(X)
    got = run(lib, X)
    m = check(got, ref, shape)
    assert m["frac_exact"] > 0.99, m
