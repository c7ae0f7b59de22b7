"""Bit-exact cases: results that no summation order or fp32 rounding can change.

* B = I (or A = I): C = alpha A + beta C0 with alpha = 1, beta in {0, 0.5}:
  the products are exact, the sums with zeros are exact, and the update
  rounds once.  With full-mantissa data this also exposes any conversion of
  the operands to a narrower format (it would change A's low bits).
* All-ones operands: C = alpha K + beta C0, exact for K < 2**24.
* Integer entries in [-4, 4]: every partial sum is an integer below 2**24,
  so any order gives the same exact result; this pins indexing, edges,
  leading dimensions and races independently of rounding.
Expected values: the oracle's double result rounded once to fp32.
"""
import numpy as np
import pytest

import fp32_gemm_06_amd as fg
import oracle
from fp32_gemm_06_amd import inputs
from gpu_util import assert_bitexact, require_gpu, run_hip

pytestmark = pytest.mark.gpu

EDGE_SHAPES = [
    (9, 9, 9), (16, 16, 16), (17, 15, 33), (31, 33, 32), (32, 32, 31), (33, 31, 65),
    (63, 64, 65), (64, 65, 63), (65, 63, 64), (127, 128, 129), (128, 129, 127),
    (129, 127, 128), (255, 256, 257), (256, 257, 255), (257, 255, 256),
    (300, 77, 50), (77, 300, 9), (513, 260, 17), (260, 513, 100), (12, 700, 300),
    (700, 12, 300), (1, 1, 1), (2, 3, 4), (5, 6, 7), (8, 40, 33), (9, 41, 34),
]


@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_integers_auto(shape):
    require_gpu()
    M, N, K = shape
    A, B, C0 = inputs.random_case(hash(shape) % 1000, M, N, K, kind="int")
    got, canary = run_hip(A, B, C0, 1.0, 0.5, guard=64)
    assert canary, "write outside C"
    assert_bitexact(got, oracle.sgemm(A, B, C0, 1.0, 0.5), f"int {shape}")


def test_integers_every_config_ragged():
    require_gpu()
    for (M, N, K) in [(257, 255, 129), (100, 300, 61), (33, 520, 12)]:
        A, B, C0 = inputs.random_case(M + N + K, M, N, K, kind="int")
        ref = oracle.sgemm(A, B, C0, 1.0, 0.5)
        for cfg in range(fg.fp32gemm_num_configs(0)):
            got, canary = run_hip(A, B, C0, 1.0, 0.5, config=cfg, family="gemm", guard=64)
            assert canary, f"write outside C, config {fg.fp32gemm_config_name(0, cfg)}"
            assert_bitexact(got, ref, f"int {(M, N, K)} {fg.fp32gemm_config_name(0, cfg)}")


def test_integers_every_config_short_k_128bit_path():
    """Aligned shapes (the 128-bit DMA path) with K from one slice to five:
    the deeper-pipelined tiles fetch up to three slices ahead, so these cover
    prefetches that start past the end of K and ragged last slices."""
    require_gpu()
    for K in (4, 28, 32, 36, 64, 68, 96, 100, 132):
        M, N = 136, 196
        A, B, C0 = inputs.random_case(900 + K, M, N, K, kind="int")
        ref = oracle.sgemm(A, B, C0, 1.0, 0.5)
        for cfg in range(fg.fp32gemm_num_configs(0)):
            got, canary = run_hip(A, B, C0, 1.0, 0.5, config=cfg, family="gemm", guard=64)
            assert canary, f"write outside C, K={K} {fg.fp32gemm_config_name(0, cfg)}"
            assert_bitexact(got, ref, f"int K={K} {fg.fp32gemm_config_name(0, cfg)}")


@pytest.mark.parametrize("beta", [0.0, 0.5])
@pytest.mark.parametrize("shape", [(128, 128), (300, 260), (4092, 4092)], ids=str)
def test_identity_b(shape, beta):
    """B = I: catches any narrowing of A (a TF32/bf16-like conversion drops
    A's low mantissa bits) and any row/column mix-up."""
    require_gpu()
    M, n = shape
    g = inputs.rng(M + n)
    A, C0 = inputs.uniform(g, (M, n)), inputs.uniform(g, (M, n))
    got, _ = run_hip(A, inputs.identity(n), C0, 1.0, beta)
    want = A.astype(np.float64) + beta * C0.astype(np.float64)
    assert_bitexact(got, want, f"B=I {shape} beta={beta}")


def test_identity_a():
    """A = I: C = B + 0.5 C0 exactly (pins B's path the same way)."""
    require_gpu()
    n, N = 300, 333
    g = inputs.rng(5)
    B, C0 = inputs.uniform(g, (n, N)), inputs.uniform(g, (n, N))
    got, _ = run_hip(inputs.identity(n), B, C0, 1.0, 0.5)
    assert_bitexact(got, B.astype(np.float64) + 0.5 * C0.astype(np.float64), "A=I")


@pytest.mark.parametrize("shape", [(128, 128, 128), (4092, 4092, 4092), (4096, 4096, 4096),
                                   (1, 4096, 4096), (8, 100, 5000)], ids=str)
def test_all_ones(shape):
    require_gpu()
    M, N, K = shape
    C0 = inputs.uniform(inputs.rng(3), (M, N))
    got, _ = run_hip(inputs.ones(M, K), inputs.ones(K, N), C0, 2.0, 0.5)
    want = np.float64(2.0 * K) + 0.5 * C0.astype(np.float64)
    assert_bitexact(got, want, f"ones {shape}")



@pytest.mark.parametrize("layout", [(0, 0), (0, 1), (1, 0), (1, 1)], ids=str)
def test_beta_zero_path_keeps_the_k_order(layout):
    """With beta = 0 the tiled kernels finish their last K slice one row of
    blocks at a time and store it at once; with beta != 0 they take the
    plain epilogue.  Both must sum every element in the same order: on
    full-mantissa data, C from beta = 0 equals C from beta = 1 over C0 = 0
    bit for bit (adding beta * 0 is exact).  Every configuration for
    op(A) op(B) = A B, the library's choice for the transposed layouts; the
    aligned (128-bit) and the 4-byte aligned (32-bit) operand paths."""
    torch = require_gpu()
    ta, tb = layout
    for (M, N, K, off) in [(300, 520, 260, 0), (129, 67, 97, 1)]:
        A, B, _ = inputs.random_case(M + N + K + off, M, N, K, kind="uniform")
        sa = np.ascontiguousarray(A.T) if ta else A
        sb = np.ascontiguousarray(B.T) if tb else B
        lda, ldb = (M if ta else K), (K if tb else N)
        # an offset of one float leaves the operands only 4-byte aligned
        fa = torch.zeros(sa.size + 4, device="cuda")
        fa[off:off + sa.size] = torch.from_numpy(sa.reshape(-1)).cuda()
        fb = torch.zeros(sb.size + 4, device="cuda")
        fb[off:off + sb.size] = torch.from_numpy(sb.reshape(-1)).cuda()
        pa, pb = fa.data_ptr() + 4 * off, fb.data_ptr() + 4 * off
        cfgs = range(fg.fp32gemm_num_configs(0)) if layout == (0, 0) else [None]
        for cfg in cfgs:
            outs = []
            for beta in (0.0, 1.0):
                C = torch.full((M, N), float("nan") if beta == 0.0 else 0.0, device="cuda")
                if cfg is None:
                    rc = fg.sgemm_ex(ta, tb, M, N, K, 1.0, pa, lda, pb, ldb, beta, C, N)
                else:
                    rc = fg.fp32gemm_sgemm_with_config(cfg, M, N, K, 1.0, pa, lda, pb, ldb, beta, C, N)
                assert rc == 0, fg.strerror(rc)
                outs.append(C)
            torch.cuda.synchronize()
            name = "auto" if cfg is None else fg.fp32gemm_config_name(0, cfg)
            assert torch.equal(outs[0], outs[1]), (layout, (M, N, K, off), name)
