"""Edges of the contract: leading dimensions, alignment, read conventions, quick
returns, argument errors and determinism."""
import numpy as np
import pytest

import fp32_gemm_06_amd as fg
import oracle
from fp32_gemm_06_amd import inputs
from gpu_util import assert_bitexact, assert_parity, require_gpu, run_hip

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("lds", [(0, 0, 0), (4, 8, 12), (1, 3, 5), (129, 1, 7)], ids=str)
@pytest.mark.parametrize("shape", [(70, 90, 110), (257, 129, 65), (6, 300, 200)], ids=str)
def test_leading_dims(shape, lds):
    """Padded rows (filled with NaN on the device) must be neither read nor written."""
    require_gpu()
    M, N, K = shape
    A, B, C0 = inputs.random_case(1, M, N, K, kind="int", lda=K + lds[0], ldb=N + lds[1],
                                  ldc=N + lds[2])
    got, canary = run_hip(A, B, C0, 1.0, 0.5, guard=32)
    assert canary, "write outside C or into its row padding"
    assert_bitexact(got, oracle.sgemm(A, B, C0, 1.0, 0.5), f"ld {shape} {lds}")


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_misaligned_pointers(offset):
    """Operands not 16-byte aligned take the 32-bit load path; same result."""
    require_gpu()
    for (M, N, K) in [(130, 260, 68), (5, 300, 64)]:
        A, B, C0 = inputs.random_case(offset, M, N, K, kind="int")
        got, canary = run_hip(A, B, C0, 1.0, 0.5, guard=16, offset=offset)
        assert canary
        assert_bitexact(got, oracle.sgemm(A, B, C0, 1.0, 0.5), f"offset {offset}")


def test_beta_zero_does_not_read_c():
    require_gpu()
    for (M, N, K) in [(200, 300, 100), (4, 500, 300)]:
        A, B, _ = inputs.random_case(2, M, N, K, kind="uniform")
        nanC = np.full((M, N), np.nan, dtype=np.float32)
        got, _ = run_hip(A, B, nanC, 1.0, 0.0)
        assert np.all(np.isfinite(got))
        ref = oracle.sgemm(A, B, None, 1.0, 0.0)
        assert_parity(got, ref, oracle.bound(A, B, None, 1.0, 0.0), "beta=0")


def test_alpha_zero_and_k_zero():
    require_gpu()
    torch = pytest.importorskip("torch")
    M, N, K = 50, 60, 70
    g = inputs.rng(9)
    C0 = inputs.uniform(g, (M, N))
    nanA = np.full((M, K), np.nan, dtype=np.float32)
    nanB = np.full((K, N), np.nan, dtype=np.float32)
    got, _ = run_hip(nanA, nanB, C0, 0.0, -2.0)
    assert_bitexact(got, -2.0 * C0.astype(np.float64), "alpha=0")
    got, _ = run_hip(nanA, nanB, C0, 0.0, 0.0)
    assert np.all(got == 0.0)
    # K = 0: C = beta C, A and B are NULL
    C = torch.from_numpy(C0.copy()).cuda()
    assert fg.sgemm(M, N, 0, 1.0, None, 1, None, N, 0.5, C, N) == 0
    torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy(), (0.5 * C0.astype(np.float64)).astype(np.float32))
    # beta = 1 with alpha = 0 leaves C alone
    assert fg.sgemm(M, N, K, 0.0, None, K, None, N, 1.0, C, N) == 0
    # M = 0 / N = 0 do nothing even with NULL pointers
    assert fg.sgemm(0, N, K, 1.0, None, K, None, N, 0.0, None, N) == 0
    assert fg.sgemm(M, 0, K, 1.0, None, K, None, 1, 0.0, None, 1) == 0


def test_argument_errors():
    require_gpu()
    torch = pytest.importorskip("torch")
    A = torch.zeros(16, 16, device="cuda")
    cases = [
        ((-1, 4, 4, 1.0, A, 4, A, 4, 0.0, A, 4), -1),
        ((4, -1, 4, 1.0, A, 4, A, 4, 0.0, A, 4), -2),
        ((4, 4, -1, 1.0, A, 4, A, 4, 0.0, A, 4), -3),
        ((4, 4, 4, 1.0, None, 4, A, 4, 0.0, A, 4), -5),
        ((4, 4, 8, 1.0, A, 4, A, 4, 0.0, A, 4), -6),
        ((4, 4, 4, 1.0, A, 4, None, 4, 0.0, A, 4), -7),
        ((4, 8, 4, 1.0, A, 4, A, 4, 0.0, A, 8), -8),
        ((4, 4, 4, 1.0, A, 4, A, 4, 0.0, None, 4), -10),
        ((4, 8, 4, 1.0, A, 4, A, 8, 0.0, A, 4), -11),
    ]
    for args, code in cases:
        assert fg.sgemm(*args) == code, (args, code)
        assert "invalid argument" in fg.strerror(code)
    assert fg.sgemv(129, 4, 4, 1.0, A, 4, A, 4, 0.0, A, 4) == -1
    assert fg.sgemv(0, 4, 4, 1.0, A, 4, A, 4, 0.0, A, 4) == -1
    assert fg.fp32gemm_sgemm_with_config(10 ** 6, 4, 4, 4, 1.0, A, 4, A, 4, 0.0, A, 4) == -100
    assert fg.fp32gemm_sgemv_with_config(10 ** 6, 4, 4, 4, 1.0, A, 4, A, 4, 0.0, A, 4) == -100


def test_deterministic_and_stream_independent():
    """Repeated calls are bit-identical (no float atomics, fixed reduction
    order), also on a second stream."""
    torch = require_gpu()
    for (M, N, K) in [(4092, 4092, 4092), (1, 4096, 4096), (8, 4096, 4096), (600, 700, 900)]:
        A, B, _ = inputs.random_case(M, M, N, K, kind="normal")
        dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        first = fg.gemm(dA, dB).clone()
        for _ in range(3):
            assert torch.equal(fg.gemm(dA, dB), first)
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            other = fg.gemm(dA, dB)
        s.synchronize()
        assert torch.equal(other, first)


def test_gemm_wrapper_views_and_epilogue():
    """gemm() maps transposed torch views onto sgemm_ex and bias/act onto
    sgemm_fused; bit-exact on integer data."""
    torch = require_gpu()
    import fp32_gemm_06_amd as fg
    M, N, K = 70, 90, 110
    g = inputs.rng(77)
    A = g.integers(-4, 5, size=(M, K)).astype(np.float32)
    B = g.integers(-4, 5, size=(K, N)).astype(np.float32)
    C0 = g.integers(-4, 5, size=(M, N)).astype(np.float32)
    bias = g.integers(-9, 10, size=N).astype(np.float32)
    dA = torch.from_numpy(A).cuda()
    dAt = torch.from_numpy(np.ascontiguousarray(A.T)).cuda().t()     # a transposed view
    dBt = torch.from_numpy(np.ascontiguousarray(B.T)).cuda().t()     # W.t() of an N x K weight
    want = oracle.sgemm(A, B, C0, 1.0, 0.5)
    for a in (dA, dAt):
        C = torch.from_numpy(C0).cuda()
        fg.gemm(a, dBt, C, beta=0.5)
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy().astype(np.float64), want)
    C = torch.from_numpy(C0).cuda()
    fg.gemm(dAt, dBt, C, beta=0.5, bias=torch.from_numpy(bias).cuda(), act="relu")
    torch.cuda.synchronize()
    assert np.array_equal(C.cpu().numpy().astype(np.float64),
                          oracle.sgemm_fused(A, B, C0, 1.0, 0.5, bias, oracle.ACT_RELU))
    with pytest.raises(ValueError):
        fg.gemm(dA, dBt, config=0)


def test_host_query_before_torch_import():
    """A host-only call (the configuration query) made before torch is
    imported loads the library first.  The binding imports torch before the
    library, so the process keeps one HIP runtime and the next product still
    finds the GPU (a second runtime reported no device).  In a fresh process."""
    import os
    import subprocess
    import sys
    import textwrap
    require_gpu()
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = textwrap.dedent(f"""
        import sys
        sys.path.insert(0, {root!r})
        import fp32_gemm_06_amd as fg
        assert fg.fp32gemm_select_config(0, 1536, 1536, 256) >= 0
        import torch
        A = torch.ones(64, 32, device="cuda")
        B = torch.ones(32, 48, device="cuda")
        C = torch.zeros(64, 48, device="cuda")
        rc = fg.sgemm(64, 48, 32, 1.0, A, 32, B, 48, 0.0, C, 48)
        torch.cuda.synchronize()
        assert rc == 0, fg.strerror(rc)
        assert bool((C == 32).all())
        print("product ok")
    """)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0 and "product ok" in r.stdout, r.stdout + r.stderr
