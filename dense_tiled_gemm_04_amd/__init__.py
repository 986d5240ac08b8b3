"""Python binding of the MI355X (gfx950) fp16 GEMM library.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libgemm_f16.so`` (built from ``csrc/`` by ``build.py``), reached
through the C ABI in ``include/gemm_f16.h``.  PyTorch supplies device memory and
the current stream.  If the shared library is missing, every entry point
raises: there is no CPU or PyTorch fallback.

Computes C = fp16(epi(A @ B)), epi in {none, bias, bias_gelu} with GELU in its
exact erf form, fp32 accumulation (TileLang tutorial: blog post "Designing
High-Performance GPU Kernels with TileLang", section "Step 4"; news article on
TileLang kernel design, paragraphs on the tiled GEMM and the fused epilogue),
the row-wise softmax of an fp16 matrix (same news article, the closing
sentences of the fused-epilogue paragraph) and the attention forward pass
(same news article, paragraph on FlashAttention).
"""
from __future__ import annotations

import ctypes
import json
import os

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libgemm_f16.so")

EPILOGUES = {"none": 0, "bias": 1, "bias_gelu": 2}
STATUS = {
    0: "GEMM_OK", 1: "GEMM_ERR_INVALID_DIM", 2: "GEMM_ERR_NULL_POINTER", 3: "GEMM_ERR_BAD_EPILOGUE",
    4: "GEMM_ERR_LAUNCH", 5: "GEMM_ERR_NO_CONFIG", 6: "GEMM_ERR_UNSUPPORTED", 7: "GEMM_ERR_MISALIGNED",
}
# every symbol the headers under include/ declare
EXPORTS = [
    "gemm_f16", "gemm_f16_status_string", "gemm_f16_num_configs", "gemm_f16_config_info",
    "gemm_f16_select_config", "gemm_f16_with_config", "vector_add_f32",
    "gemm_f16_ex", "gemm_f16_select_config_ex", "gemm_f16_with_config_ex",
    "gemm_f16_bt", "gemm_f16_bt_select_config", "gemm_f16_bt_with_config",
    "softmax_rows_f16", "softmax_rows_f16_path", "flash_attn_fwd_f16", "flash_attn_fwd_f16_kernel",
    "gemm_status_string", "gemm_f16_time",
    "mfma_f16_calibration", "mfma_f16_calibration_flops",
]
SOFTMAX_PATHS = {0: "none", 1: "wave", 2: "workgroup", 3: "online"}

_lib = None


class GemmError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(status_string(status))


def load():
    """Load libgemm_f16.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libgemm_f16.so is not built; run `python -m dense_tiled_gemm_04_amd.build` "
                           "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.gemm_f16.argtypes = [i64, i64, i64, vp, vp, vp, vp, i32, vp]
    lib.gemm_f16.restype = i32
    lib.gemm_f16_with_config.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, i32, vp]
    lib.gemm_f16_with_config.restype = i32
    lib.gemm_f16_select_config.argtypes = [i64, i64, i64, vp, vp, vp, vp, i32]
    lib.gemm_f16_select_config.restype = i32
    lib.gemm_f16_ex.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, vp, i64, i32, vp]
    lib.gemm_f16_ex.restype = i32
    lib.gemm_f16_with_config_ex.argtypes = [i32, i64, i64, i64, vp, i64, vp, i64, vp, vp, i64, i32, vp]
    lib.gemm_f16_with_config_ex.restype = i32
    lib.gemm_f16_select_config_ex.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, vp, i64, i32]
    lib.gemm_f16_select_config_ex.restype = i32
    lib.gemm_f16_bt.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, vp, i64, i32, vp]
    lib.gemm_f16_bt.restype = i32
    lib.gemm_f16_bt_with_config.argtypes = [i32, i64, i64, i64, vp, i64, vp, i64, vp, vp, i64, i32, vp]
    lib.gemm_f16_bt_with_config.restype = i32
    lib.gemm_f16_bt_select_config.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, vp, i64, i32]
    lib.gemm_f16_bt_select_config.restype = i32
    lib.gemm_f16_status_string.argtypes = [i32]
    lib.gemm_f16_status_string.restype = ctypes.c_char_p
    lib.gemm_status_string.argtypes = [i32]
    lib.gemm_status_string.restype = ctypes.c_char_p
    lib.gemm_f16_time.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, i32, vp, i32, ctypes.POINTER(ctypes.c_float)]
    lib.gemm_f16_time.restype = i32
    lib.mfma_f16_calibration.argtypes = [i32, i64, i64, vp, vp, vp]
    lib.mfma_f16_calibration.restype = i32
    lib.mfma_f16_calibration_flops.argtypes = [i32, i64, i64]
    lib.mfma_f16_calibration_flops.restype = i64
    lib.gemm_f16_num_configs.argtypes = []
    lib.gemm_f16_num_configs.restype = i32
    lib.gemm_f16_config_info.argtypes = [i32, ctypes.c_char_p, i32]
    lib.gemm_f16_config_info.restype = i32
    lib.vector_add_f32.argtypes = [i64, vp, vp, vp, vp]
    lib.vector_add_f32.restype = i32
    lib.softmax_rows_f16.argtypes = [i64, i64, vp, vp, vp]
    lib.softmax_rows_f16.restype = i32
    lib.softmax_rows_f16_path.argtypes = [i64, i64]
    lib.softmax_rows_f16_path.restype = i32
    lib.flash_attn_fwd_f16.argtypes = [i64, i64, i64, i64, i64, vp, vp, vp, vp, i32, ctypes.c_float, vp]
    lib.flash_attn_fwd_f16.restype = i32
    lib.flash_attn_fwd_f16_kernel.argtypes = [i64, i64, i64, i64, i64, vp, vp, vp, vp, i32, ctypes.c_float, i32, vp]
    lib.flash_attn_fwd_f16_kernel.restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().gemm_f16_status_string(int(status)).decode()


def num_configs() -> int:
    return int(load().gemm_f16_num_configs())


def config_info(idx: int) -> dict:
    buf = ctypes.create_string_buffer(1024)
    n = load().gemm_f16_config_info(int(idx), buf, 1024)
    if n < 0:
        raise GemmError(-n)
    return json.loads(buf.value.decode())


def configs() -> list[dict]:
    return [config_info(i) for i in range(num_configs())]


# ---------------------------------------------------------------------------
# raw-pointer entry points (ints are device addresses; stream is a hipStream_t)
# ---------------------------------------------------------------------------
def gemm_f16_raw(M, N, K, A, B, bias, C, epilogue: int, stream=0, config: int | None = None) -> int:
    lib = load()
    if config is None:
        return int(lib.gemm_f16(M, N, K, A, B, bias, C, epilogue, stream))
    return int(lib.gemm_f16_with_config(config, M, N, K, A, B, bias, C, epilogue, stream))


def select_config_raw(M, N, K, A, B, bias, C, epilogue: int) -> int:
    return int(load().gemm_f16_select_config(M, N, K, A, B, bias, C, epilogue))


def gemm_f16_ex_raw(M, N, K, A, lda, B, ldb, bias, C, ldc, epilogue: int, stream=0,
                    config: int | None = None) -> int:
    lib = load()
    if config is None:
        return int(lib.gemm_f16_ex(M, N, K, A, lda, B, ldb, bias, C, ldc, epilogue, stream))
    return int(lib.gemm_f16_with_config_ex(config, M, N, K, A, lda, B, ldb, bias, C, ldc, epilogue, stream))


def select_config_ex_raw(M, N, K, A, lda, B, ldb, bias, C, ldc, epilogue: int) -> int:
    return int(load().gemm_f16_select_config_ex(M, N, K, A, lda, B, ldb, bias, C, ldc, epilogue))


def gemm_f16_bt_raw(M, N, K, A, lda, Bt, ldb, bias, C, ldc, epilogue: int, stream=0,
                    config: int | None = None) -> int:
    lib = load()
    if config is None:
        return int(lib.gemm_f16_bt(M, N, K, A, lda, Bt, ldb, bias, C, ldc, epilogue, stream))
    return int(lib.gemm_f16_bt_with_config(config, M, N, K, A, lda, Bt, ldb, bias, C, ldc, epilogue, stream))


def select_config_bt_raw(M, N, K, A, lda, Bt, ldb, bias, C, ldc, epilogue: int) -> int:
    return int(load().gemm_f16_bt_select_config(M, N, K, A, lda, Bt, ldb, bias, C, ldc, epilogue))


def gemm_f16_time_raw(M, N, K, A, B, bias, C, epilogue: int, iters: int, stream=0, config: int = -1):
    """(status, median ms per launch) of gemm_f16_time: `iters` event-bracketed launches after one untimed."""
    out = ctypes.c_float(-1.0)
    st = int(load().gemm_f16_time(config, M, N, K, A, B, bias, C, epilogue, stream, iters, ctypes.byref(out)))
    return st, float(out.value)


def mfma_calibration_raw(shape: int, iters: int, workgroups: int, stamps, sink, stream=0) -> int:
    """Launch the register-only MFMA loop (include/calibration_f16.h); stamps and sink are device pointers."""
    return int(load().mfma_f16_calibration(shape, iters, workgroups, stamps, sink, stream))


def mfma_calibration_flops(shape: int, iters: int, workgroups: int) -> int:
    return int(load().mfma_f16_calibration_flops(shape, iters, workgroups))


def softmax_rows_raw(rows, cols, X, Y, stream=0) -> int:
    return int(load().softmax_rows_f16(rows, cols, X, Y, stream))


def softmax_path(rows: int, cols: int) -> str:
    """Which softmax kernel a call of this shape runs: none, wave, workgroup or online."""
    return SOFTMAX_PATHS[int(load().softmax_rows_f16_path(rows, cols))]


# ---------------------------------------------------------------------------
# torch front end
# ---------------------------------------------------------------------------
def _check(t, name, ndim):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != torch.float16:
        raise TypeError("%s must be float16, got %s" % (name, t.dtype))
    if t.dim() != ndim:
        raise ValueError("%s must be %d-D" % (name, ndim))
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous (row-major)" % name)


def _check_rows(t, name):
    """A 2-D float16 GPU matrix stored row-major with unit column stride (possibly a
    sub-matrix of a wider array); returns its leading dimension."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != torch.float16:
        raise TypeError("%s must be float16, got %s" % (name, t.dtype))
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    rows, cols = t.shape
    if rows > 1 and cols > 1 and t.stride(1) != 1:
        raise ValueError("%s must be row-major with unit column stride" % name)
    ld = t.stride(0) if rows > 1 else cols
    if rows > 1 and ld < cols:
        raise ValueError("%s rows overlap (stride %d < %d columns)" % (name, ld, cols))
    return max(ld, cols)


def _stream_handle():
    import torch
    return torch.cuda.current_stream().cuda_stream


def gemm_f16(A, B, bias=None, epilogue: str = "none", out=None, config: int | None = None,
             b_transposed: bool = False):
    """C = fp16(epi(A @ B [+ bias])) on the current stream; returns C (torch.float16 [M, N]).
    With b_transposed, B is given as Bt [N, K] (a linear layer's weight) and C = epi(A @ Bt^T).
    A, B and out may be row-major sub-matrices of wider arrays (unit column stride)."""
    import torch
    if epilogue not in EPILOGUES:
        raise ValueError("epilogue must be one of %s" % list(EPILOGUES))
    lda = _check_rows(A, "A")
    ldb = _check_rows(B, "B")
    M, K = A.shape
    N, K2 = B.shape if b_transposed else B.shape[::-1]
    if K != K2:
        raise ValueError("inner dimensions differ: A is %s, B is %s" % (tuple(A.shape), tuple(B.shape)))
    if A.device != B.device:
        raise ValueError("A and B on different devices")
    epi = EPILOGUES[epilogue]
    if epi != 0:
        if bias is None:
            raise ValueError("epilogue %r needs a bias" % epilogue)
        _check(bias, "bias", 1)
        if bias.shape[0] != N:
            raise ValueError("bias must have N=%d elements" % N)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=A.device)
    else:
        if tuple(out.shape) != (M, N):
            raise ValueError("out must be [%d, %d]" % (M, N))
    ldc = _check_rows(out, "out")
    with torch.cuda.device(A.device):
        fn = gemm_f16_bt_raw if b_transposed else gemm_f16_ex_raw
        st = fn(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, bias.data_ptr() if epi != 0 else None,
                out.data_ptr(), ldc, epi, _stream_handle(), config)
    if st != 0:
        raise GemmError(st)
    return out


def select_config(A, B, bias=None, epilogue: str = "none", out=None, b_transposed: bool = False) -> int:
    """Index of the configuration gemm_f16 would launch (-1 for an empty output)."""
    M, K = A.shape
    N = B.shape[0] if b_transposed else B.shape[1]
    epi = EPILOGUES[epilogue]
    optr = out.data_ptr() if out is not None else 256  # a 256-byte-aligned stand-in address
    ldc = _check_rows(out, "out") if out is not None else N
    fn = select_config_bt_raw if b_transposed else select_config_ex_raw
    r = fn(M, N, K, A.data_ptr(), _check_rows(A, "A"), B.data_ptr(), _check_rows(B, "B"),
           bias.data_ptr() if bias is not None else None, optr, ldc, epi)
    if r < -1:
        raise GemmError(-r)
    return r


def softmax_f16(X, out=None):
    """Row-wise softmax of a contiguous float16 GPU matrix on the current stream; returns Y.
    out may be X itself (in place)."""
    import torch
    _check(X, "X", 2)
    rows, cols = X.shape
    if out is None:
        out = torch.empty_like(X)
    else:
        _check(out, "out", 2)
        if tuple(out.shape) != (rows, cols):
            raise ValueError("out must be [%d, %d]" % (rows, cols))
    with torch.cuda.device(X.device):
        st = softmax_rows_raw(rows, cols, X.data_ptr(), out.data_ptr(), _stream_handle())
    if st != 0:
        raise GemmError(st)
    return out


# kernels of the attention forward pass (include/attention_f16.h)
ATTN_KERNEL_AUTO, ATTN_KERNEL_BLOCK_SERIAL, ATTN_KERNEL_PIPELINED = 0, 1, 2


def flash_attn_raw(B, H, Nq, Nkv, D, Q, K, V, O, causal: bool, scale: float, stream=0, kernel=None) -> int:
    if kernel is None:
        return int(load().flash_attn_fwd_f16(B, H, Nq, Nkv, D, Q, K, V, O, 1 if causal else 0, float(scale), stream))
    return int(load().flash_attn_fwd_f16_kernel(B, H, Nq, Nkv, D, Q, K, V, O, 1 if causal else 0, float(scale),
                                                int(kernel), stream))


def flash_attn(Q, K, V, causal: bool = False, scale: float | None = None, out=None, kernel=None):
    """Attention forward on contiguous float16 GPU tensors Q [B,H,Nq,D], K and V [B,H,Nkv,D] on the current
    stream; D is 64 or 128, scale defaults to 1/sqrt(D), causal masks keys j > i.  Returns O [B,H,Nq,D].
    `kernel` (an ATTN_KERNEL_* value) forces one of the kernels; None is the default dispatch."""
    import math
    import torch
    for t, n in ((Q, "Q"), (K, "K"), (V, "V")):
        _check(t, n, 4)
    Bn, Hn, Nq, D = Q.shape
    if tuple(K.shape) != tuple(V.shape) or K.shape[0] != Bn or K.shape[1] != Hn or K.shape[3] != D:
        raise ValueError("K and V must be [B, H, Nkv, D] matching Q [B, H, Nq, D]")
    Nkv = K.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(Q)
    else:
        _check(out, "out", 4)
        if tuple(out.shape) != tuple(Q.shape):
            raise ValueError("out must have Q's shape")
    with torch.cuda.device(Q.device):
        st = flash_attn_raw(Bn, Hn, Nq, Nkv, D, Q.data_ptr(), K.data_ptr(), V.data_ptr(), out.data_ptr(), causal,
                            scale, _stream_handle(), kernel)
    if st != 0:
        raise GemmError(st)
    return out


def vector_add(a, b, out=None):
    """out = a + b for contiguous float32 GPU tensors (the HBM calibration kernel)."""
    import torch
    for t, n in ((a, "a"), (b, "b")):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise TypeError("%s must be a contiguous float32 GPU tensor" % n)
    if a.numel() != b.numel():
        raise ValueError("size mismatch")
    if out is None:
        out = torch.empty_like(a)
    with torch.cuda.device(a.device):
        st = int(load().vector_add_f32(a.numel(), a.data_ptr(), b.data_ptr(), out.data_ptr(), _stream_handle()))
    if st != 0:
        raise GemmError(st)
    return out
