"""Products the tiled kernel runs as two launches over column or row ranges of C.

When the 256x256 tiles overflow whole rounds of 256, the dispatcher may run
the columns (or rows) that fill exact rounds in that tile and the rest as a
second product.  These cases check that the two launches together compute the
same product as the oracle: sampled full rows and columns, including the ones
on both sides of the split point and the ragged last ones, for every operand
layout, the fused epilogue and strided batches.
"""
import numpy as np
import pytest

import fp32_gemm_06_amd as fg
import oracle
from fp32_gemm_06_amd import inputs
from gpu_util import assert_parity, require_gpu

pytestmark = pytest.mark.gpu


def _lines(n, first, g, extra=10):
    """Indices 0, 1, the split point's neighbours, the last two, and a few random."""
    fixed = [0, 1, first - 2, first - 1, first, first + 1, n - 2, n - 1] if first else [0, n - 1]
    return sorted(set(i for i in fixed + list(g.integers(0, n, extra)) if 0 <= i < n))


def _entries(M, N, first, dim, seed):
    g = np.random.default_rng(seed)
    rows = _lines(M, first if dim == 2 else 0, g)
    cols = _lines(N, first if dim == 1 else 0, g)
    r1, c1 = np.repeat(rows, N), np.tile(np.arange(N), len(rows))
    r2, c2 = np.tile(np.arange(M), len(cols)), np.repeat(cols, M)
    return np.concatenate([r1, r2]).astype(np.int32), np.concatenate([c1, c2]).astype(np.int32)


def _check(got, opA, opB, C0, alpha, beta, dim, first, seed, bias=None, act=oracle.ACT_NONE,
           what=""):
    M, N = got.shape
    rows, cols = _entries(M, N, first, dim, seed)
    if bias is None and act == oracle.ACT_NONE:
        ref = oracle.sgemm_entries(rows, cols, opA, opB, C0, alpha, beta)
        bnd = oracle.bound_entries(rows, cols, opA, opB, C0, alpha, beta)
    else:
        ref = oracle.sgemm_fused_entries(rows, cols, opA, opB, C0, alpha, beta, bias, act)
        bnd = oracle.bound_fused_entries(rows, cols, opA, opB, C0, alpha, beta, bias)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    return assert_parity(got[rows, cols], ref, bnd, what)


CASES = [
    # (M, N, K, transA, transB, expected split dimension)
    (2048, 11008, 512, 0, 0, 1),
    (2048, 11008, 384, 1, 1, 1),
    (2048, 11008, 256, 0, 1, 1),
    (2816, 8192, 1024, 0, 0, 2),
    (2816, 8192, 1056, 1, 0, 2),
    (2816, 8192, 1024, 1, 1, 2),
]


@pytest.mark.parametrize("M,N,K,ta,tb,dim", CASES, ids=lambda v: str(v))
def test_split_layouts(M, N, K, ta, tb, dim):
    torch = require_gpu()
    got_dim, first = fg.fp32gemm_round_split(M, N, K, 1)
    assert got_dim == dim, (got_dim, first)
    seed = M + N + K + 2 * ta + tb
    g = inputs.rng(seed)
    opA, opB, C0 = inputs.uniform(g, (M, K)), inputs.uniform(g, (K, N)), inputs.uniform(g, (M, N))
    sA = np.ascontiguousarray(opA.T) if ta else opA
    sB = np.ascontiguousarray(opB.T) if tb else opB
    dA, dB, dC = (torch.from_numpy(x).cuda() for x in (sA, sB, C0))
    rc = fg.sgemm_ex(ta, tb, M, N, K, 0.75, dA, sA.shape[1], dB, sB.shape[1], -0.5, dC, N)
    assert rc == 0, fg.fp32gemm_strerror(rc)
    torch.cuda.synchronize()
    got = dC.cpu().numpy().astype(np.float64)
    print(M, N, K, ta, tb, "split", dim, first,
          _check(got, opA, opB, C0, 0.75, -0.5, dim, first, seed, what=f"{M}x{N}x{K} {ta}{tb}"))


@pytest.mark.parametrize("act", [oracle.ACT_NONE, oracle.ACT_RELU])
def test_split_fused_bias(act):
    torch = require_gpu()
    M, N, K = 2048, 11008, 256
    dim, first = fg.fp32gemm_round_split(M, N, K, 1)
    assert dim == 1
    g = inputs.rng(77 + act)
    A, B, C0 = inputs.uniform(g, (M, K)), inputs.uniform(g, (K, N)), inputs.uniform(g, (M, N))
    bias = inputs.uniform(g, (N,))
    dA, dB, dC, dbias = (torch.from_numpy(x).cuda() for x in (A, B, C0, bias))
    rc = fg.sgemm_fused(0, 0, M, N, K, 1.0, dA, K, dB, N, 0.5, dC, N, dbias, act)
    assert rc == 0, fg.fp32gemm_strerror(rc)
    torch.cuda.synchronize()
    got = dC.cpu().numpy().astype(np.float64)
    _check(got, A, B, C0, 1.0, 0.5, dim, first, 78, bias=bias, act=act, what=f"fused act={act}")


def test_split_batched():
    """256 entries of 256 x 300: 256 columns of every entry fill one round of
    256x256 tiles; the other 44 columns run as the second product."""
    torch = require_gpu()
    M, N, K, batch = 256, 300, 256, 256
    dim, first = fg.fp32gemm_round_split(M, N, K, batch)
    assert (dim, first) == (1, 256)
    g = inputs.rng(91)
    A = inputs.uniform(g, (batch, M, K))
    B = inputs.uniform(g, (batch, K, N))
    C0 = inputs.uniform(g, (batch, M, N))
    dA, dB, dC = (torch.from_numpy(x).cuda() for x in (A, B, C0))
    rc = fg.sgemm_strided_batched(0, 0, M, N, K, 1.0, dA, K, M * K, dB, N, K * N, 1.0, dC, N,
                                  M * N, batch)
    assert rc == 0, fg.fp32gemm_strerror(rc)
    torch.cuda.synchronize()
    got = dC.cpu().numpy().astype(np.float64)
    for b in (0, 1, 127, 254, 255):
        _check(got[b], A[b], B[b], C0[b], 1.0, 1.0, dim, first, 92 + b, what=f"entry {b}")
