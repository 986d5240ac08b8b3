"""Seeded synthetic inputs for the fp16 GEMM workloads.

This module only draws random numbers and rounds them to fp16; it holds none of
the GEMM's arithmetic.  Both the GPU library's tests/benchmark and the CPU
oracle take their inputs from here, so both sides see the same bits.

Recipe (the pages fix only the shapes and the 4096^3 fp16 headline, see the
TileLang blog post, sections "performance" and "Step 4"; the distributions
below are this project's workload definitions):
  * ``rng = numpy.random.default_rng(seed)`` (PCG64);
  * draw A, then B, then bias, each as float64, in that order;
  * ``N(0, v)`` means variance v (std = sqrt(v)); ``U[-1,1)`` is
    ``rng.uniform(-1, 1)``;
  * cast each array once to fp16 with numpy's round-to-nearest-even.
Numpy's Generator streams are not promised stable across numpy versions, so
``input_digest`` records a sha256 of the bits actually used.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    seed: int
    epilogue: str          # "none" | "bias" | "bias_gelu"
    a_dist: tuple          # ("uniform", lo, hi) or ("normal", variance)
    b_dist: tuple
    bias_dist: tuple | None
    note: str = ""

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> int:
        """A, B, bias (if used) and C, each moved once, fp16."""
        b = 2 * (self.M * self.K + self.K * self.N + self.M * self.N)
        if self.epilogue != "none":
            b += 2 * self.N
        return b


WORKLOADS = {
    w.name: w
    for w in [
        Workload("gemm_256", 256, 256, 256, 0, "none", ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0), None,
                 "small square GEMM, no epilogue"),
        Workload("gemm_4096", 4096, 4096, 4096, 1, "none", ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0), None,
                 "the pages' 4096^3 fp16 headline shape"),
        Workload("mlp_up_8192x16384x4096", 8192, 16384, 4096, 2, "bias_gelu", ("normal", 1.0),
                 ("normal", 1.0 / 4096), ("normal", 0.1), "fused MLP up-projection, GELU(A.B + bias)"),
        Workload("ragged_4095x3001x1000", 4095, 3001, 1000, 3, "bias", ("uniform", -1.0, 1.0),
                 ("uniform", -1.0, 1.0), ("normal", 0.1), "no dimension a multiple of any tile size"),
        Workload("skinny_16x16384x8192", 16, 16384, 8192, 4, "bias_gelu", ("normal", 1.0),
                 ("normal", 1.0 / 8192), ("normal", 0.1), "skinny M, HBM-bound"),
    ]
}
ORDER = list(WORKLOADS)


def _draw(rng: np.random.Generator, dist: tuple, shape) -> np.ndarray:
    if dist[0] == "uniform":
        return rng.uniform(dist[1], dist[2], size=shape)
    if dist[0] == "normal":
        return rng.standard_normal(size=shape) * math.sqrt(dist[1])
    raise ValueError(dist)


def make_inputs(w: Workload | str, M: int | None = None, N: int | None = None, K: int | None = None):
    """Return (A, B, bias) as float16 numpy arrays (bias None without epilogue).

    M/N/K override the workload's shape (same distributions and seed), which
    lets tests draw small instances with the same value statistics.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    rng = np.random.default_rng(w.seed)
    A = _draw(rng, w.a_dist, (M, K)).astype(np.float16)
    B = _draw(rng, w.b_dist, (K, N)).astype(np.float16)
    bias = _draw(rng, w.bias_dist, (N,)).astype(np.float16) if w.bias_dist is not None else None
    return A, B, bias


@dataclasses.dataclass(frozen=True)
class SoftmaxWorkload:
    """Row-wise softmax of an fp16 [rows][cols] matrix (the pages give no shapes for it)."""
    name: str
    rows: int
    cols: int
    seed: int
    dist: tuple            # ("normal", variance) or ("uniform", lo, hi)
    note: str = ""

    @property
    def algorithmic_bytes(self) -> int:
        """X read once and Y written once, fp16."""
        return 2 * 2 * self.rows * self.cols


SOFTMAX_WORKLOADS = {
    w.name: w
    for w in [
        SoftmaxWorkload("softmax_8192x16384", 8192, 16384, 5, ("normal", 4.0),
                        "row softmax over the MLP up-projection's output shape; logits N(0, 2^2)"),
        SoftmaxWorkload("softmax_4095x3001", 4095, 3001, 6, ("normal", 4.0),
                        "ragged rows: neither dimension a multiple of a chunk or a workgroup"),
        SoftmaxWorkload("softmax_65536x256", 65536, 256, 7, ("normal", 4.0),
                        "short rows: one wave per row"),
    ]
}


def make_softmax_input(w: SoftmaxWorkload | str, rows: int | None = None, cols: int | None = None) -> np.ndarray:
    """X as a float16 numpy array, drawn as for the GEMM inputs (rows/cols override the shape)."""
    if isinstance(w, str):
        w = SOFTMAX_WORKLOADS[w]
    rows = w.rows if rows is None else rows
    cols = w.cols if cols is None else cols
    rng = np.random.default_rng(w.seed)
    return _draw(rng, w.dist, (rows, cols)).astype(np.float16)


@dataclasses.dataclass(frozen=True)
class AttentionWorkload:
    """Attention forward: Q [B,H,Nq,D], K and V [B,H,Nkv,D], fp16 (the pages give no shapes for it)."""
    name: str
    B: int
    H: int
    Nq: int
    Nkv: int
    D: int
    causal: bool
    seed: int
    note: str = ""

    @property
    def pairs(self) -> int:
        """(query, key) pairs the softmax runs over: Nq*Nkv, or the top-left causal triangle."""
        if not self.causal:
            return self.Nq * self.Nkv
        n = min(self.Nq, self.Nkv)
        return n * (n + 1) // 2 + max(0, self.Nq - self.Nkv) * self.Nkv

    @property
    def flops(self) -> int:
        """2 * D for Q.K plus 2 * D for P.V per allowed pair, per (batch, head)."""
        return 4 * self.B * self.H * self.D * self.pairs

    @property
    def algorithmic_bytes(self) -> int:
        return 2 * self.B * self.H * self.D * (2 * self.Nq + 2 * self.Nkv)


ATTENTION_WORKLOADS = {
    w.name: w
    for w in [
        AttentionWorkload("attn_b4_h32_n4096_d128", 4, 32, 4096, 4096, 128, False, 8,
                          "non-causal self-attention, 32 heads of 128 at sequence 4096"),
        AttentionWorkload("attn_b4_h32_n4096_d128_causal", 4, 32, 4096, 4096, 128, True, 9,
                          "causal self-attention, 32 heads of 128 at sequence 4096"),
        AttentionWorkload("attn_b2_h16_n1000_d64_causal", 2, 16, 1000, 1000, 64, True, 10,
                          "ragged causal self-attention, head dimension 64"),
        AttentionWorkload("attn_b1_h8_q777_kv1500_d128", 1, 8, 777, 1500, 128, False, 11,
                          "cross-attention, ragged query and key lengths"),
    ]
}


def make_attention_inputs(w: AttentionWorkload | str, B=None, H=None, Nq=None, Nkv=None):
    """Q, K, V as float16 numpy arrays, each N(0, 1), drawn in that order (shape overrides allowed)."""
    if isinstance(w, str):
        w = ATTENTION_WORKLOADS[w]
    B = w.B if B is None else B
    H = w.H if H is None else H
    Nq = w.Nq if Nq is None else Nq
    Nkv = w.Nkv if Nkv is None else Nkv
    rng = np.random.default_rng(w.seed)
    Q = rng.standard_normal((B, H, Nq, w.D)).astype(np.float16)
    K = rng.standard_normal((B, H, Nkv, w.D)).astype(np.float16)
    V = rng.standard_normal((B, H, Nkv, w.D)).astype(np.float16)
    return Q, K, V


def random_f16(seed: int, shape, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    """Plain uniform fp16 draws for ad-hoc test shapes."""
    rng = np.random.default_rng(seed)
    return rng.uniform(lo, hi, size=shape).astype(np.float16)


def random_f32_bits(seed: int, n: int) -> np.ndarray:
    """n float32 values with uniformly random bit patterns (every class: normal, subnormal, zero, inf, NaN)."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32).view(np.float32)


def make_vector_add_inputs(n: int, seed: int = 12):
    """Two float32 vectors ~ N(0, 1) of length n for the vector add (the pages' first kernel adds two float32
    vectors; they give no distribution)."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(n).astype(np.float32)
    b = rng.standard_normal(n).astype(np.float32)
    return a, b


def input_digest(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        if a is not None:
            h.update(np.ascontiguousarray(a).view(np.uint8).tobytes())
    return h.hexdigest()
