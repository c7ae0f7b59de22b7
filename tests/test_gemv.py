"""The small-M (decode) kernels: every batch size 1..8, both load paths, every
configuration, ragged N and K, padded leading dimensions; M = 9..128 on every
configuration that takes it (vector-ALU row capacities up to 32, the skinny
MFMA kernel up to 128), routed through sgemm, with op(A) = A^T, with the weight
stored transposed and in strided batches."""
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


WIDE_M = [9, 12, 13, 16, 17, 24, 25, 32, 33, 40, 48, 49, 64, 65, 80, 96, 97, 100, 128]


@pytest.mark.parametrize("M", WIDE_M)
def test_wide_rows_every_config(M):
    """M = 9..128: every configuration of the GEMV family that runs this M
    (vector-ALU stripes on row capacities up to 32, the skinny MFMA kernel on
    16/32/64-column stripes up to 128/128/64 rows; rows past M masked), both
    load paths, bit-exact, nothing written outside C; the configurations
    whose row limit is below M are refused."""
    require_gpu()
    names = fg.config_names(fg.KIND_SGEMV)
    rows = [fg.fp32gemm_config_max_rows(fg.KIND_SGEMV, c) for c in range(len(names))]
    assert any(r >= M for r in rows)
    for (N, K) in [(1000, 777), (333, 4099), (16, 5000)]:
        A, B, C0 = inputs.random_case(M * 37 + N, M, N, K, kind="int")
        ref = oracle.sgemm(A, B, C0, 1.0, 0.5)
        for cfg in range(len(names)):
            if rows[cfg] < M:
                with pytest.raises(fg.Fp32GemmError):
                    run_hip(A, B, C0, 1.0, 0.5, config=cfg, family="gemv")
                continue
            got, canary = run_hip(A, B, C0, 1.0, 0.5, config=cfg, family="gemv", guard=32)
            assert canary, f"write outside C (M={M} N={N} {names[cfg]})"
            assert_bitexact(got, ref, f"M={M} N={N} K={K} {names[cfg]}")


@pytest.mark.parametrize("M", [9, 16, 24, 32, 48, 64, 96, 128])
def test_wide_rows_routed(M):
    """sgemm with M = 9..128 (the skinny kernel where it pays, the tiled
    kernel where it has 256 tiles or more or where K < 5 M), and sgemv
    (always the skinny kernel), against the oracle."""
    require_gpu()
    for (N, K) in [(4096, 1024), (24576, 256), (530, 130)]:
        A, B, C0 = inputs.random_case(M + N, M, N, K, kind="uniform")
        ref = oracle.sgemm(A, B, C0, 0.75, -1.0)
        bnd = oracle.bound(A, B, C0, 0.75, -1.0)
        for family in ("auto", "gemv"):
            got, canary = run_hip(A, B, C0, 0.75, -1.0, family=family, guard=16)
            assert canary
            assert_parity(got, ref, bnd, f"M={M} N={N} K={K} {family}")


@pytest.mark.parametrize("M", [10, 20, 32, 48, 80, 100])
def test_wide_rows_transposed_x(M):
    """op(A) = A^T with M = 9..128: the skinny kernel reads X with swapped strides
    (M = 48 and 80 round up to 4 and 8 row blocks: 3 and 5 take op(A) = A only)."""
    from test_transpose_batched import _case, run_batched
    N, K = 530, 3001
    As, Bs, Cs = _case(7200 + M, M, N, K)
    (got,), ok = run_batched(1, 0, As, Bs, Cs, 1.0, 0.5, pads=(5, 4, 3), offset=1)
    assert ok, "write outside C"
    assert_bitexact(got, oracle.sgemm(As[0], Bs[0], Cs[0], 1.0, 0.5), f"M={M} op(A)=A^T")


@pytest.mark.parametrize("ta", (0, 1))
@pytest.mark.parametrize("M", [9, 16, 33, 48, 64, 80, 96, 100, 128])
def test_wide_rows_weight_transposed(ta, M):
    """op(B) = B^T (weight stored N x K) with M = 9..128: the skinny kernel's
    stored-row path, with 16-byte loads along k (aligned, K % 4 == 0) and
    with 4-byte loads (K odd, and operands off 16-byte alignment)."""
    from test_transpose_batched import _case, run_batched
    for (N, K, offset) in [(530, 3000, 0), (530, 3001, 0), (47, 1024, 1)]:
        As, Bs, Cs = _case(7400 + M + K, M, N, K)
        (got,), ok = run_batched(ta, 1, As, Bs, Cs, 1.0, 0.5, pads=(3, 4, 5), offset=offset)
        assert ok, "write outside C"
        assert_bitexact(got, oracle.sgemm(As[0], Bs[0], Cs[0], 1.0, 0.5),
                        f"M={M} N={N} K={K} ta={ta} op(B)=B^T")


def test_wide_rows_batched():
    """Strided batches of M = 16, 27, 45 and 70 entries in one skinny grid,
    both weight layouts (K = 700: the skinny kernel's side of K = 5 M)."""
    from test_transpose_batched import _case, run_batched
    for M in (16, 27, 45, 70):
        for tb in (0, 1):
            As, Bs, Cs = _case(7300 + M, M, 200, 700, batch=3)
            outs, ok = run_batched(0, tb, As, Bs, Cs, 1.0, 1.0, pads=(1, 2, 3), gaps=(7, 5, 3))
            assert ok, "write outside C"
            for b in range(3):
                assert_bitexact(outs[b], oracle.sgemm(As[b], Bs[b], Cs[b], 1.0, 1.0),
                                f"M={M} tb={tb} entry {b}")


@pytest.mark.parametrize("tb", (0, 1))
@pytest.mark.parametrize("M,offset", [(48, 0), (80, 0), (48, 1), (80, 1)])
def test_wide_rows_batched_wide_stripes(tb, M, offset):
    """Four entries of M x 4096 x 700: the grid of 16-column stripes takes four
    rounds, so the skinny kernel runs 64-column stripes (M = 48, W stored
    K x N) or 32-column ones; one float off a 16-byte boundary, the weight is
    read a float at a time (stored N x K) or on 16-column stripes (K x N)."""
    from test_transpose_batched import _case, run_batched
    As, Bs, Cs = _case(7500 + M + tb + offset, M, 4096, 700, batch=4)
    outs, ok = run_batched(0, tb, As, Bs, Cs, 1.0, 0.5, offset=offset)
    assert ok, "write outside C"
    for b in range(4):
        assert_bitexact(outs[b], oracle.sgemm(As[b], Bs[b], Cs[b], 1.0, 0.5),
                        f"M={M} tb={tb} offset={offset} entry {b}")


@pytest.mark.parametrize("tb,M,N", [(1, 9, 530), (1, 12, 4096), (1, 16, 1000), (0, 9, 12288),
                                    (0, 16, 12288)])
def test_one_row_block_x_in_registers(tb, M, N):
    """One row block with op(A) = A on aligned rows: over W stored N x K, and on
    64-column stripes over W stored K x N, the skinny kernel loads X straight
    into registers (no LDS staging, no per-pass barrier).  K = 1028 ends in a
    partial pass; rows past M and k past K read zeros."""
    from test_transpose_batched import _case, run_batched
    As, Bs, Cs = _case(7600 + M + N + tb, M, N, 1028)
    (got,), ok = run_batched(0, tb, As, Bs, Cs, 1.0, 0.5)
    assert ok, "write outside C"
    assert_bitexact(got, oracle.sgemm(As[0], Bs[0], Cs[0], 1.0, 0.5), f"M={M} N={N} tb={tb}")
