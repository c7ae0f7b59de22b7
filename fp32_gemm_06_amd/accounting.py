"""Work and traffic accounting for the benchmark (no GEMM arithmetic).

FLOPs: a multiply-add counts as two operations, so an M x N x K product is
2 M N K; the alpha/beta update adds M N, which the pages call negligible
("GPU GEMM 优化完全拆解（一）", section "什么是 GEMM").  Throughput is reported
with 2 M N K.

Algorithmic bytes: what any implementation must move between HBM and the
chip with an unbounded cache: read A and B once, write C once, and read C
once more only when beta != 0 ("CUDA 矩阵乘法优化：从朴素 Kernel 到接近
cuBLAS", section "第一性原理" counts A, B and C read plus C written).

Tile traffic: with BM x BN output tiles every K-slice of A is re-read N/BN
times and of B M/BN times, so operand traffic is 4 M N K (1/BM + 1/BN) bytes
("GPU GEMM 优化完全拆解（一）", section "收益：全局内存流量降了一个量级").
Arithmetic intensity of one square tile TILE (one output per thread,
"GPU 基础原理", section "4.7 片上计算阶段") is 2 TILE^3 / (8 TILE^2) = TILE/4.
"""
from __future__ import annotations

import math

FP32 = 4

# MI355X published peaks (dense, no sparsity).
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBPS = 8000.0
CUS = 256
XCDS = 8
SCLK_GHZ = 2.4


def flops(M: int, N: int, K: int, with_update: bool = False) -> int:
    f = 2 * M * N * K
    return f + M * N if with_update else f


def algorithmic_bytes(M: int, N: int, K: int, beta: float) -> int:
    b = FP32 * (M * K + K * N + M * N)
    if beta != 0.0:
        b += FP32 * M * N
    return b


def tile_operand_bytes(M: int, N: int, K: int, BM: int, BN: int) -> float:
    """Operand bytes fetched by a tiled kernel with BM x BN output tiles."""
    return FP32 * M * N * K * (1.0 / BM + 1.0 / BN)


def naive_bytes(M: int, N: int, K: int) -> int:
    """One thread per output reading its whole row of A, column of B and C."""
    return FP32 * M * N * (2 * K + 1)


def tile_intensity(tile: int) -> float:
    return (2 * tile ** 3) / (2 * FP32 * tile ** 2)


def l2_intensity(BM: int, BN: int) -> float:
    """FLOPs per operand byte of a BM x BN tile: BM BN / (2 (BM + BN))."""
    return BM * BN / (2.0 * (BM + BN))


def grid(M: int, N: int, BM: int, BN: int):
    return math.ceil(M / BM), math.ceil(N / BN)


def valid_in_last_block(size: int, block: int) -> int:
    r = size % block
    return block if r == 0 else r
