"""The fused epilogue (sgemm_fused): C <- act(alpha op(A) op(B) + beta C +
bias[j]) against the oracle's sgemm_fused.

Integer data and integer biases keep every value exact, so these cases are
bit-exact; uniform data use the standard tolerance with the bias added to the
scale.  Shapes reach the 64x64, 128x128 and 256x256 tiles, both GEMV kernels
(M <= 8 with B as given and stored transposed), the skinny MFMA kernel
(M = 9..128 with K >= 5 M), and the alpha = 0 path.
"""
import itertools

import numpy as np
import pytest

import fp32_gemm_06_amd as fg
import oracle
from fp32_gemm_06_amd import inputs
from gpu_util import assert_bitexact, assert_parity, require_gpu
from test_transpose_batched import SENTINEL, _store

pytestmark = pytest.mark.gpu


def run_fused(ta, tb, A, B, C0, alpha, beta, bias, act, pads=(0, 0, 0), offset=0):
    """A, B, C0: the op() operands (host).  Returns (C float64, untouched
    outside C)."""
    torch = require_gpu()
    M, K = A.shape
    N = B.shape[1]
    a_st = np.ascontiguousarray(A.T) if ta else A
    b_st = np.ascontiguousarray(B.T) if tb else B
    lda, ldb, ldc = a_st.shape[1] + pads[0], b_st.shape[1] + pads[1], N + pads[2]
    dA, oa = _store(torch, [a_st], lda, 0, offset, 8)
    dB, ob = _store(torch, [b_st], ldb, 0, offset, 8)
    dC, oc = _store(torch, [C0], ldc, 0, offset, 64)
    dbias = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias)).cuda()
    rc = fg.sgemm_fused(ta, tb, M, N, K, alpha, dA.data_ptr() + 4 * oa, lda,
                        dB.data_ptr() + 4 * ob, ldb, beta, dC.data_ptr() + 4 * oc, ldc, dbias, act)
    if rc:
        raise fg.Fp32GemmError(rc)
    torch.cuda.synchronize()
    host = dC.cpu().numpy()
    got = host[oc: oc + M * ldc].reshape(M, ldc)[:, :N].astype(np.float64)
    ok = bool(np.all(host[:oc] == SENTINEL) and np.all(host[oc + M * ldc:][
        ~np.isnan(host[oc + M * ldc:])] == SENTINEL))
    return got, ok


def _ints(seed, M, N, K):
    g = inputs.rng(seed)
    A, B, C0 = (g.integers(-4, 5, size=s).astype(np.float32) for s in ((M, K), (K, N), (M, N)))
    bias = g.integers(-40, 41, size=N).astype(np.float32)
    return A, B, C0, bias


SHAPES = [(300, 260, 130), (257, 255, 129), (2000, 2000, 64), (4092, 4092, 40), (5, 300, 500),
          (8, 1000, 777), (1, 64, 33), (48, 530, 700), (100, 257, 1001)]


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("shape", SHAPES, ids=str)
def test_bitexact(shape, act):
    M, N, K = shape
    for ta, tb in itertools.product((0, 1), (0, 1)):
        if M > 1000 and (ta, tb) != (0, 0) and act == 0:
            continue   # the large tiles' layouts are covered once with act = 1
        A, B, C0, bias = _ints(M + N + K + ta + 2 * tb, M, N, K)
        got, ok = run_fused(ta, tb, A, B, C0, 1.0, 0.5, bias, act, pads=(4, 0, 4))
        assert ok, "write outside C"
        want = oracle.sgemm_fused(A, B, C0, 1.0, 0.5, bias, act)
        if M * N <= 1 << 20:
            assert_bitexact(got, want, f"{shape} op {ta}{tb} act {act}")
        else:
            rows = np.array([0, 1, M // 2, M - 1])
            assert_bitexact(got[rows], want[rows], f"{shape} op {ta}{tb} act {act} rows")


@pytest.mark.parametrize("act", [0, 1])
def test_no_bias_and_misaligned(act):
    M, N, K = 130, 98, 99
    A, B, C0, _ = _ints(11 + act, M, N, K)
    got, ok = run_fused(0, 0, A, B, C0, 2.0, -1.0, None, act, offset=1)
    assert ok
    assert_bitexact(got, oracle.sgemm_fused(A, B, C0, 2.0, -1.0, None, act), f"no bias act {act}")


@pytest.mark.parametrize("K", [0, 7])
def test_alpha_zero_or_k_zero_applies_the_epilogue(K):
    """The quick-return path (C <- beta C) still adds the bias and applies
    the activation."""
    M, N = 70, 90
    A, B, C0, bias = _ints(20 + K, M, N, max(K, 1))
    A, B = A[:, :K], B[:K]
    alpha = 0.0 if K else 1.0
    got, ok = run_fused(0, 0, A, B, C0, alpha, 0.5, bias, 1, pads=(1, 0, 0))
    assert ok
    assert_bitexact(got, oracle.sgemm_fused(A, B, C0, alpha, 0.5, bias, 1, K=K),
                    f"quick return K={K}")


def test_special_values_in_c():
    """beta = 1 carries NaN and infinities of C into the epilogue: NaN stays
    NaN through the ReLU, -inf becomes 0."""
    M, N, K = 64, 64, 32
    A, B, C0, bias = _ints(30, M, N, K)
    C0[0, 0], C0[1, 1], C0[2, 2] = np.nan, -np.inf, np.inf
    got, ok = run_fused(0, 0, A, B, C0, 1.0, 1.0, bias, 1)
    want = oracle.sgemm_fused(A, B, C0, 1.0, 1.0, bias, 1)
    assert np.isnan(got[0, 0]) and got[1, 1] == 0.0 and got[2, 2] == np.inf
    mask = np.ones_like(got, dtype=bool)
    mask[0, 0] = False
    assert np.array_equal(got[mask], want[mask])


@pytest.mark.parametrize("shape", [(1024, 768, 1000), (8, 4096, 4096)], ids=str)
def test_uniform_tolerance(shape):
    M, N, K = shape
    g = inputs.rng(M + N)
    A, B, C0 = inputs.uniform(g, (M, K)), inputs.uniform(g, (K, N)), inputs.uniform(g, (M, N))
    bias = inputs.uniform(g, (N,))
    got, ok = run_fused(0, 1, A, B, C0, 0.75, -1.25, bias, 1)
    assert ok
    assert_parity(got, oracle.sgemm_fused(A, B, C0, 0.75, -1.25, bias, 1),
                  oracle.bound_fused(A, B, C0, 0.75, -1.25, bias), f"uniform {shape}")
