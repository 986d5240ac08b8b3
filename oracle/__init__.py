"""CPU oracle for the fp16 GEMM + fused bias / bias+GELU epilogue, the row-wise
softmax, the attention forward pass and the fp32 vector add (Python side).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code with
the GPU library and never imports it.

The arithmetic lives in ``gemm_oracle.c`` (plain fp64 loops, own binary16 codec,
libm ``erf``); this module only builds that file with gcc and marshals numpy
arrays into it.  See the C file's header for the definition it follows
(TileLang tutorial pages: blog post "Designing High-Performance GPU Kernels with
TileLang", section "Step 4"; news article on TileLang kernel design, paragraphs
on the tiled GEMM and on the fused bias + GELU epilogue).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

EPILOGUES = {"none": 0, "bias": 1, "bias_gelu": 2}

_lib = None


def build(force: bool = True) -> str:
    """Compile gemm_oracle.c into liboracle.so next to it (gcc, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_gemm_f16.argtypes = [i64, i64, i64, p, p, p, p, p, ctypes.c_int, ctypes.c_int]
    lib.oracle_gemm_f16.restype = ctypes.c_int
    lib.oracle_gemm_f16_points.argtypes = [i64, i64, i64, p, p, p, ctypes.c_int, i64, p, p, p, p, ctypes.c_int]
    lib.oracle_gemm_f16_points.restype = ctypes.c_int
    lib.oracle_f16_decode_n.argtypes = [p, p, i64]
    lib.oracle_f16_encode_n.argtypes = [p, p, i64]
    lib.oracle_gelu_n.argtypes = [p, p, i64]
    lib.oracle_f16_encode.argtypes = [ctypes.c_double]
    lib.oracle_f16_encode.restype = ctypes.c_uint16
    lib.oracle_f16_decode.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_decode.restype = ctypes.c_double
    lib.oracle_gelu.argtypes = [ctypes.c_double]
    lib.oracle_gelu.restype = ctypes.c_double
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_softmax_rows_f16.argtypes = [i64, i64, p, p, p, ctypes.c_int]
    lib.oracle_softmax_rows_f16.restype = ctypes.c_int
    lib.oracle_attention_f16.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, p, ctypes.c_int, ctypes.c_double,
                                         ctypes.c_int]
    lib.oracle_attention_f16.restype = ctypes.c_int
    lib.oracle_attention_f16_rows.argtypes = [i64, i64, i64, i64, i64, p, p, p, ctypes.c_int, ctypes.c_double, i64,
                                              p, p, p, ctypes.c_int]
    lib.oracle_attention_f16_rows.restype = ctypes.c_int
    lib.oracle_vector_add_f32.argtypes = [i64, p, p, p]
    lib.oracle_vector_add_f32.restype = ctypes.c_int
    _lib = lib
    return lib


def _bits(x) -> np.ndarray:
    """fp16 array (or uint16 bit pattern array) -> contiguous uint16 bits."""
    x = np.asarray(x)
    if x.dtype == np.float16:
        x = x.view(np.uint16)
    if x.dtype != np.uint16:
        raise TypeError("expected float16 or uint16 bits, got %s" % x.dtype)
    return np.ascontiguousarray(x)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def gemm(A, B, bias=None, epilogue: str = "none", want_y: bool = False, threads: int = 0):
    """C = fp16(epilogue(A @ B [+ bias])) in fp64; returns float16 array (and fp64 Y)."""
    lib = _load()
    A16, B16 = _bits(A), _bits(B)
    if A16.ndim != 2 or B16.ndim != 2 or A16.shape[1] != B16.shape[0]:
        raise ValueError("shape mismatch")
    M, K = A16.shape
    N = B16.shape[1]
    epi = EPILOGUES[epilogue]
    b16 = _bits(bias).reshape(-1) if bias is not None else None
    if epi != 0 and (b16 is None or b16.shape[0] != N):
        raise ValueError("bias of length N required")
    C = np.empty((M, N), dtype=np.uint16)
    Y = np.empty((M, N), dtype=np.float64) if want_y else None
    rc = lib.oracle_gemm_f16(M, N, K, _ptr(A16), _ptr(B16), _ptr(b16), _ptr(C), _ptr(Y), epi, threads)
    if rc != 0:
        raise RuntimeError("oracle_gemm_f16 failed (%d)" % rc)
    C = C.view(np.float16)
    return (C, Y) if want_y else C


def gemm_points(A, B, bias, epilogue: str, rows, cols, want_y: bool = False, threads: int = 0):
    """C[rows[t], cols[t]] for each t, computed one dot product at a time."""
    lib = _load()
    A16, B16 = _bits(A), _bits(B)
    M, K = A16.shape
    N = B16.shape[1]
    epi = EPILOGUES[epilogue]
    b16 = _bits(bias).reshape(-1) if bias is not None else None
    r = np.ascontiguousarray(rows, dtype=np.int64)
    c = np.ascontiguousarray(cols, dtype=np.int64)
    if r.shape != c.shape:
        raise ValueError("rows/cols length mismatch")
    out = np.empty(r.shape[0], dtype=np.uint16)
    Y = np.empty(r.shape[0], dtype=np.float64) if want_y else None
    rc = lib.oracle_gemm_f16_points(M, N, K, _ptr(A16), _ptr(B16), _ptr(b16), epi, r.shape[0],
                                    _ptr(r), _ptr(c), _ptr(out), _ptr(Y), threads)
    if rc != 0:
        raise RuntimeError("oracle_gemm_f16_points failed (%d)" % rc)
    out = out.view(np.float16)
    return (out, Y) if want_y else out


def softmax_rows(X, want_y: bool = False, threads: int = 0):
    """Row-wise softmax of an fp16 matrix in fp64, rounded once to fp16 (see the C file)."""
    lib = _load()
    X16 = _bits(X)
    if X16.ndim != 2:
        raise ValueError("expected a 2-D matrix")
    rows, cols = X16.shape
    Y = np.empty((rows, cols), dtype=np.uint16)
    Yd = np.empty((rows, cols), dtype=np.float64) if want_y else None
    rc = lib.oracle_softmax_rows_f16(rows, cols, _ptr(X16), _ptr(Y), _ptr(Yd), threads)
    if rc != 0:
        raise RuntimeError("oracle_softmax_rows_f16 failed (%d)" % rc)
    Y = Y.view(np.float16)
    return (Y, Yd) if want_y else Y


def attention(Q, K, V, causal: bool = False, scale: float | None = None, want_y: bool = False,
              threads: int = 0):
    """Attention forward in fp64, rounded once to fp16.  Q [B,H,Nq,D], K and V [B,H,Nkv,D] (fp16).
    scale defaults to 1/sqrt(D); causal masks keys j > i (top-left aligned)."""
    lib = _load()
    Q16, K16, V16 = _bits(Q), _bits(K), _bits(V)
    if Q16.ndim != 4 or K16.shape != V16.shape or K16.ndim != 4:
        raise ValueError("expected Q [B,H,Nq,D] and K, V [B,H,Nkv,D]")
    Bn, Hn, Nq, D = Q16.shape
    if K16.shape[0] != Bn or K16.shape[1] != Hn or K16.shape[3] != D:
        raise ValueError("Q, K, V shapes disagree")
    Nkv = K16.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    O = np.empty(Q16.shape, dtype=np.uint16)
    Od = np.empty(Q16.shape, dtype=np.float64) if want_y else None
    rc = lib.oracle_attention_f16(Bn, Hn, Nq, Nkv, D, _ptr(Q16), _ptr(K16), _ptr(V16), _ptr(O), _ptr(Od),
                                  1 if causal else 0, float(scale), threads)
    if rc != 0:
        raise RuntimeError("oracle_attention_f16 failed (%d)" % rc)
    O = O.view(np.float16)
    return (O, Od) if want_y else O


def attention_rows(Q, K, V, rows, causal: bool = False, scale: float | None = None, want_y: bool = False,
                   threads: int = 0):
    """Selected output rows of attention(): rows are flat indices (b*H + h)*Nq + i; returns [len(rows), D]."""
    lib = _load()
    Q16, K16, V16 = _bits(Q), _bits(K), _bits(V)
    Bn, Hn, Nq, D = Q16.shape
    Nkv = K16.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    O = np.empty((r.shape[0], D), dtype=np.uint16)
    Od = np.empty((r.shape[0], D), dtype=np.float64) if want_y else None
    rc = lib.oracle_attention_f16_rows(Bn, Hn, Nq, Nkv, D, _ptr(Q16), _ptr(K16), _ptr(V16), 1 if causal else 0,
                                       float(scale), r.shape[0], _ptr(r), _ptr(O), _ptr(Od), threads)
    if rc != 0:
        raise RuntimeError("oracle_attention_f16_rows failed (%d)" % rc)
    O = O.view(np.float16)
    return (O, Od) if want_y else O


def vector_add(a, b) -> np.ndarray:
    """C = A + B on float32 vectors, each element the correctly rounded binary32 sum (see the C file)."""
    lib = _load()
    a = np.ascontiguousarray(a, dtype=np.float32).reshape(-1)
    b = np.ascontiguousarray(b, dtype=np.float32).reshape(-1)
    if a.shape != b.shape:
        raise ValueError("length mismatch")
    c = np.empty_like(a)
    rc = lib.oracle_vector_add_f32(a.shape[0], _ptr(a), _ptr(b), _ptr(c))
    if rc != 0:
        raise RuntimeError("oracle_vector_add_f32 failed (%d)" % rc)
    return c


def f16_decode(bits) -> np.ndarray:
    lib = _load()
    h = np.ascontiguousarray(bits, dtype=np.uint16).reshape(-1)
    out = np.empty(h.shape[0], dtype=np.float64)
    lib.oracle_f16_decode_n(_ptr(h), _ptr(out), h.shape[0])
    return out


def f16_encode(x) -> np.ndarray:
    """fp64 values -> binary16 bit patterns (uint16), RNE."""
    lib = _load()
    d = np.ascontiguousarray(x, dtype=np.float64).reshape(-1)
    out = np.empty(d.shape[0], dtype=np.uint16)
    lib.oracle_f16_encode_n(_ptr(d), _ptr(out), d.shape[0])
    return out


def gelu(x) -> np.ndarray:
    lib = _load()
    d = np.ascontiguousarray(x, dtype=np.float64).reshape(-1)
    out = np.empty(d.shape[0], dtype=np.float64)
    lib.oracle_gelu_n(_ptr(d), _ptr(out), d.shape[0])
    return out
