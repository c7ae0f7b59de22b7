"""The small-M (decode) kernel: every batch size 1..8, both load paths, every
configuration, ragged N and K, padded leading dimensions."""
import numpy as np
import pytest

import fp32_gemm_06_amd as fg
import oracle
from fp32_gemm_06_amd import inputs
from gpu_util import assert_bitexact, assert_parity, require_gpu, run_hip

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M", range(1, 9))
def test_every_batch_size_every_config(M):
    require_gpu()
    # N = 1000: float4 path with a partial last column block; N = 333: 32-bit path
    for (N, K) in [(1000, 777), (333, 4099), (16, 5000)]:
        A, B, C0 = inputs.random_case(M * 31 + N, M, N, K, kind="int")
        ref = oracle.sgemm(A, B, C0, 1.0, 0.5)
        for cfg in range(fg.fp32gemm_num_configs(1)):
            got, canary = run_hip(A, B, C0, 1.0, 0.5, config=cfg, family="gemv", guard=32)
            assert canary, f"write outside C (M={M} N={N} {fg.fp32gemm_config_name(1, cfg)})"
            assert_bitexact(got, ref, f"M={M} N={N} K={K} {fg.fp32gemm_config_name(1, cfg)}")


@pytest.mark.parametrize("lds", [(3, 4, 5), (4, 8, 4)], ids=str)
def test_padded(lds):
    require_gpu()
    M, N, K = 5, 700, 900
    A, B, C0 = inputs.random_case(11, M, N, K, kind="normal", lda=K + lds[0], ldb=N + lds[1],
                                  ldc=N + lds[2])
    got, canary = run_hip(A, B, C0, -0.5, 1.5, guard=16)
    assert canary
    assert_parity(got, oracle.sgemm(A, B, C0, -0.5, 1.5), oracle.bound(A, B, C0, -0.5, 1.5),
                  f"padded {lds}")


def test_decode_sizes_normal():
    """The decode workloads' distributions (x ~ N(0,1), W ~ 0.02 N(0,1)) at
    every batch size, full output against the oracle."""
    require_gpu()
    for M in range(1, 9):
        g = inputs.rng(200 + M)
        X = inputs.normal(g, (M, 4096))
        W = inputs.normal(g, (4096, 4096), std=0.02)
        Y0 = np.zeros((M, 4096), np.float32)
        got, _ = run_hip(X, W, Y0, 1.0, 0.0)
        assert_parity(got, oracle.sgemm(X, W, Y0, 1.0, 0.0), oracle.bound(X, W, Y0, 1.0, 0.0),
                      f"decode M={M}")


@pytest.mark.parametrize("M", range(1, 9))
def test_transposed_x(M):
    """op(A) = A^T (A stored K x M) through sgemm_ex: the same kernel reads X
    with strides swapped.  K = 5000 spans an odd number of passes."""
    from test_transpose_batched import _case, run_batched
    N, K = 530, 5000
    As, Bs, Cs = _case(7000 + M, M, N, K)
    (got,), ok = run_batched(1, 0, As, Bs, Cs, 1.0, 0.5, pads=(5, 4, 3), offset=1)
    assert ok, "write outside C"
    assert_bitexact(got, oracle.sgemm(As[0], Bs[0], Cs[0], 1.0, 0.5), f"M={M} op(A)=A^T")


@pytest.mark.parametrize("tb", (0, 1))
def test_transposed_x_huge_lda_falls_back(tb):
    """lda beyond the GEMV kernels' X-offset range sends op(A) = A^T to the
    tiled kernel, which gives the same exact result."""
    from test_transpose_batched import _case, run_batched
    M, N, K = 2, 50, 3
    As, Bs, Cs = _case(7100 + tb, M, N, K)
    (got,), ok = run_batched(1, tb, As, Bs, Cs, 1.0, 0.5, pads=(140000 - M, 0, 0))
    assert ok
    assert_bitexact(got, oracle.sgemm(As[0], Bs[0], Cs[0], 1.0, 0.5), f"huge lda tb={tb}")
