"""Small-M products with the weight stored transposed (op(B) = B^T, B stored
N x K, the layout of a linear layer's weight), which sgemm_ex sends to the
row-dot kernel, against the CPU oracle.

Integer inputs make the expected values exact (bit-exact cases); uniform
inputs use the standard tolerance.  Shapes cover every M from 1 to 8, ragged
N (not a multiple of the rows a workgroup owns) and ragged K (a partial last
K chunk), both layouts of A, the 128-bit and the 32-bit weight paths, and the
decode sizes of a 4096-wide model.
"""
import numpy as np
import pytest

import oracle
from fp32_gemm_06_amd import inputs
from gpu_util import assert_bitexact, assert_parity, require_gpu
from test_transpose_batched import _case, run_batched

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M", range(1, 9))
@pytest.mark.parametrize("ta", (0, 1))
def test_every_m_ragged_bitexact(M, ta):
    N, K = 301, 1500          # 1500 = one full 1024-float chunk + a ragged one
    As, Bs, Cs = _case(1000 + 10 * M + ta, M, N, K)
    (got,), ok = run_batched(ta, 1, As, Bs, Cs, 1.0, 0.5, pads=(3, 4, 2))
    assert ok, "write outside C"
    assert_bitexact(got, oracle.sgemm(As[0], Bs[0], Cs[0], 1.0, 0.5), f"M={M} ta={ta}")


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_misaligned_weight_scalar_path(offset):
    """Weights off a 16-byte boundary (and K % 4 != 0) take the 32-bit loads."""
    M, N, K = 3, 200, 777
    As, Bs, Cs = _case(2000 + offset, M, N, K)
    (got,), ok = run_batched(0, 1, As, Bs, Cs, 2.0, -1.0, offset=offset)
    assert ok
    assert_bitexact(got, oracle.sgemm(As[0], Bs[0], Cs[0], 2.0, -1.0), f"offset {offset}")


@pytest.mark.parametrize("N", [1, 3, 4, 5, 7, 8, 9, 4095, 16390])
@pytest.mark.parametrize("M", [2, 5])
def test_ragged_n_both_rows_per_wave(M, N):
    """N around a workgroup's 4 rows (M = 2: one row per wave) and 8 rows
    (M = 5: two rows per wave)."""
    K = 260
    As, Bs, Cs = _case(3000 + N + M, M, N, K)
    (got,), ok = run_batched(0, 1, As, Bs, Cs, 1.0, 0.5, pads=(0, 4, 0))
    assert ok
    assert_bitexact(got, oracle.sgemm(As[0], Bs[0], Cs[0], 1.0, 0.5), f"N={N}")


@pytest.mark.parametrize("K", [1, 3, 4, 255, 256, 1024, 1025])
def test_k_edges(K):
    M, N = 5, 130
    As, Bs, Cs = _case(4000 + K, M, N, K)
    (got,), ok = run_batched(1, 1, As, Bs, Cs, 1.0, 0.5)
    assert ok
    assert_bitexact(got, oracle.sgemm(As[0], Bs[0], Cs[0], 1.0, 0.5), f"K={K}")


def test_beta_zero_ignores_nan_c():
    M, N, K = 4, 96, 300
    As, Bs, _ = _case(5000, M, N, K)
    Cs = [np.full((M, N), np.nan, np.float32)]
    (got,), ok = run_batched(0, 1, As, Bs, Cs, 1.0, 0.0)
    assert ok
    assert_bitexact(got, oracle.sgemm(As[0], Bs[0], None, 1.0, 0.0), "beta = 0 over NaN")


@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (4, 4096, 4096), (8, 4096, 4096),
                                   (1, 11008, 4096), (8, 4096, 11008)], ids=str)
def test_decode_shapes_uniform(M, N, K):
    """Decode-time projections of a 4096-wide model with 11008-wide FFN."""
    g = inputs.rng(M * 31 + N + K)
    A = inputs.uniform(g, (M, K))
    B = inputs.uniform(g, (K, N))
    C = inputs.uniform(g, (M, N))
    (got,), ok = run_batched(0, 1, [A], [B], [C], 1.0, -0.5)
    assert ok
    assert_parity(got, oracle.sgemm(A, B, C, 1.0, -0.5), oracle.bound(A, B, C, 1.0, -0.5),
                  f"decode {M}x{N}x{K}")


def test_deterministic():
    """The fixed reduction order gives the same bits on every call."""
    torch = require_gpu()
    import fp32_gemm_06_amd as fg
    M, N, K = 8, 2048, 3000
    g = inputs.rng(6000)
    A = torch.from_numpy(inputs.uniform(g, (M, K))).cuda()
    W = torch.from_numpy(inputs.uniform(g, (N, K))).cuda()
    outs = []
    for _ in range(3):
        C = torch.zeros(M, N, device="cuda")
        assert fg.sgemm_ex(0, 1, M, N, K, 1.0, A, K, W, K, 0.0, C, N) == 0
        outs.append(C)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


@pytest.mark.parametrize("M", [1, 3, 4, 8])
@pytest.mark.parametrize("K", [64, 128, 200, 500])
def test_short_rows_share_wave_instructions(M, K):
    """Rows shorter than 512 floats: four rows per wave instruction (16 lanes
    each), K chunks of 256; N ragged against the 4 (or 8) rows a wave owns."""
    N = 301
    for ta in (0, 1):
        As, Bs, Cs = _case(8000 + 10 * M + K + ta, M, N, K)
        (got,), ok = run_batched(ta, 1, As, Bs, Cs, 1.0, 0.5, pads=(2, 4, 3))
        assert ok, "write outside C"
        assert_bitexact(got, oracle.sgemm(As[0], Bs[0], Cs[0], 1.0, 0.5), f"M={M} K={K} ta={ta}")


def test_short_rows_scalar_path():
    M, N, K = 2, 257, 130     # K % 4 != 0: 32-bit weight loads
    As, Bs, Cs = _case(8100, M, N, K)
    (got,), ok = run_batched(0, 1, As, Bs, Cs, 2.0, -1.0, offset=1)
    assert ok
    assert_bitexact(got, oracle.sgemm(As[0], Bs[0], Cs[0], 2.0, -1.0), "short rows, 32-bit")
