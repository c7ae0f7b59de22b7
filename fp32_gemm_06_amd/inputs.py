"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module only draws numbers; it holds none of the GEMM arithmetic.  Both
the HIP path and the CPU oracle receive the same host arrays from it.

Generator: numpy ``Generator(PCG64(seed))``; draw order A, then B, then C0.
Uniform entries are drawn on [-1, 1) in float64 and cast to float32 (the cast
may round to +-1.0, which is inside the closed interval).  Normal entries use
``standard_normal(dtype=float32)``; "N(0, 0.02)" is read as standard deviation
0.02 (the usual weight-initialisation scale).

The workloads are the ones the pages measure or describe:
  * the square 4092 x 4092 fp32 product of the worklog benchmark ("CUDA 矩阵
    乘法优化：从朴素 Kernel 到接近 cuBLAS", the table at the top of the page
    and section "第一性原理"), which is not a tile multiple;
  * the aligned 4096 cube, a small 128 cube, a prefill-shaped product and the
    small-M decode product ("GPU GEMM 优化完全拆解（一）", section "LLM 推理
    本质上是 GEMM 的串联": prefill is a large matrix-matrix product, decode a
    matrix-vector product with M = batch).
The pages do not say which values filled their matrices; the distributions
below stand in for them.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    alpha: float
    beta: float
    dist: str          # "uniform" | "normal" | "prefill" | "decode"
    seed: int


WORKLOADS = {
    "sgemm_128_uniform": Workload("sgemm_128_uniform", 128, 128, 128, 1.0, 0.5, "uniform", 101),
    "sgemm_4092_uniform": Workload("sgemm_4092_uniform", 4092, 4092, 4092, 1.0, 0.0, "uniform", 102),
    "sgemm_4096_normal": Workload("sgemm_4096_normal", 4096, 4096, 4096, 0.5, 1.0, "normal", 103),
    "prefill_2048x4096x11008": Workload("prefill_2048x4096x11008", 2048, 11008, 4096, 1.0, 0.0,
                                        "prefill", 104),
    "decode_m1_4096": Workload("decode_m1_4096", 1, 4096, 4096, 1.0, 0.0, "decode", 106),
    "decode_m4_4096": Workload("decode_m4_4096", 4, 4096, 4096, 1.0, 0.0, "decode", 109),
    "decode_m8_4096": Workload("decode_m8_4096", 8, 4096, 4096, 1.0, 0.0, "decode", 113),
}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def uniform(g: np.random.Generator, shape) -> np.ndarray:
    return g.uniform(-1.0, 1.0, size=shape).astype(np.float32)


def normal(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def make(w: Workload | str):
    """Return (A, B, C0) host arrays for a named workload (row-major, packed)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    g = rng(w.seed)
    if w.dist == "uniform":
        A, B, C0 = uniform(g, (w.M, w.K)), uniform(g, (w.K, w.N)), uniform(g, (w.M, w.N))
    elif w.dist == "normal":
        A, B, C0 = normal(g, (w.M, w.K)), normal(g, (w.K, w.N)), normal(g, (w.M, w.N))
    elif w.dist in ("prefill", "decode"):
        A = normal(g, (w.M, w.K))
        B = normal(g, (w.K, w.N), std=0.02)
        C0 = np.zeros((w.M, w.N), dtype=np.float32)
    else:
        raise ValueError(w.dist)
    return A, B, C0


def random_case(seed: int, M: int, N: int, K: int, kind: str = "uniform",
                lda: int | None = None, ldb: int | None = None, ldc: int | None = None,
                pad_value: float = np.nan):
    """A, B, C0 for an arbitrary shape, optionally embedded in wider rows.

    When a leading dimension exceeds the row length the extra columns are
    filled with ``pad_value`` (NaN by default) so that a kernel reading past
    the row end shows up as a NaN in its output.  Returned arrays are views of
    shape (rows, cols) whose row stride is the leading dimension.
    kinds: "uniform" (U[-1,1)), "normal" (N(0,1)), "int" (integers in
    [-4, 4], exact in fp32 for every partial sum while 16 K < 2**24).
    """
    g = rng(seed)

    def draw(r, c):
        if kind == "uniform":
            return uniform(g, (r, c))
        if kind == "normal":
            return normal(g, (r, c))
        if kind == "int":
            return g.integers(-4, 5, size=(r, c)).astype(np.float32)
        raise ValueError(kind)

    def embed(x, ld):
        r, c = x.shape
        ld = c if ld is None else ld
        if ld < max(1, c):
            raise ValueError("leading dimension shorter than the row")
        buf = np.full((max(r, 1), max(ld, 1)), pad_value, dtype=np.float32)
        buf[:r, :c] = x
        return buf[:r, :c]

    A = embed(draw(M, K), lda)
    B = embed(draw(K, N), ldb)
    C0 = embed(draw(M, N), ldc)
    return A, B, C0


def identity(n: int) -> np.ndarray:
    return np.eye(n, dtype=np.float32)


def ones(r: int, c: int) -> np.ndarray:
    return np.ones((r, c), dtype=np.float32)
