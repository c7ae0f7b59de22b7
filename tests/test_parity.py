"""HIP path vs the CPU oracle on the benchmark workloads and across tile configurations.

Tolerance (every element): |C - C_ref| <= 1e-4 * (|alpha| (|A||B|) + |beta| |C0|),
no NaN/Inf unless the reference has one.
"""
import numpy as np
import pytest

import fp32_gemm_06_amd as fg
import oracle
from fp32_gemm_06_amd import inputs
from gpu_util import assert_parity, require_gpu, run_hip

pytestmark = pytest.mark.gpu


def _sample(M, N, seed, nrand=24):
    g = np.random.default_rng(seed)
    rows = sorted(set([0, 1, M // 2, M - 2, M - 1] + list(g.integers(0, M, nrand))))
    cols = sorted(set([0, 1, N // 2, N - 2, N - 1] + list(g.integers(0, N, nrand))))
    r1 = np.repeat(rows, N)
    c1 = np.tile(np.arange(N), len(rows))
    r2 = np.tile(np.arange(M), len(cols))
    c2 = np.repeat(cols, M)
    return np.concatenate([r1, r2]).astype(np.int32), np.concatenate([c1, c2]).astype(np.int32)


@pytest.mark.parametrize("name", ["sgemm_128_uniform", "decode_m1_4096", "decode_m4_4096",
                                  "decode_m8_4096"])
def test_workload_full(name):
    """Small workloads: every element against the oracle."""
    require_gpu()
    w = inputs.WORKLOADS[name]
    A, B, C0 = inputs.make(w)
    got, _ = run_hip(A, B, C0, w.alpha, w.beta)
    ref = oracle.sgemm(A, B, C0, w.alpha, w.beta)
    bnd = oracle.bound(A, B, C0, w.alpha, w.beta)
    print(name, "worst ratio", assert_parity(got, ref, bnd, name))


@pytest.mark.parametrize("name", ["sgemm_4092_uniform", "sgemm_4096_normal",
                                  "prefill_2048x4096x11008"])
def test_workload_sampled(name):
    """Full-size workloads, same launch as the benchmark: sampled full rows and
    columns (including the last, ragged ones) against the oracle."""
    require_gpu()
    w = inputs.WORKLOADS[name]
    A, B, C0 = inputs.make(w)
    got, _ = run_hip(A, B, C0, w.alpha, w.beta)
    rows, cols = _sample(w.M, w.N, w.seed)
    ref = oracle.sgemm_entries(rows, cols, A, B, C0, w.alpha, w.beta)
    bnd = oracle.bound_entries(rows, cols, A, B, C0, w.alpha, w.beta)
    print(name, "worst ratio", assert_parity(got[rows, cols], ref, bnd, name))
    assert np.all(np.isfinite(got)), "non-finite output"


def test_every_gemm_config_medium():
    """Each SGEMM configuration on a shape that spans several tiles with ragged
    tails in M, N and K, every element against the oracle."""
    require_gpu()
    M, N, K = 300, 520, 260
    A, B, C0 = inputs.random_case(7, M, N, K, kind="uniform")
    ref = oracle.sgemm(A, B, C0, 1.25, -0.75)
    bnd = oracle.bound(A, B, C0, 1.25, -0.75)
    for cfg in range(fg.fp32gemm_num_configs(0)):
        got, _ = run_hip(A, B, C0, 1.25, -0.75, config=cfg, family="gemm")
        assert_parity(got, ref, bnd, fg.fp32gemm_config_name(0, cfg))


def test_every_gemv_config():
    require_gpu()
    for M in (1, 3, 8):
        N, K = 1000, 777
        A, B, C0 = inputs.random_case(70 + M, M, N, K, kind="normal")
        ref = oracle.sgemm(A, B, C0, 0.5, 2.0)
        bnd = oracle.bound(A, B, C0, 0.5, 2.0)
        for cfg in range(fg.fp32gemm_num_configs(1)):
            got, _ = run_hip(A, B, C0, 0.5, 2.0, config=cfg, family="gemv")
            assert_parity(got, ref, bnd, f"M={M} {fg.fp32gemm_config_name(1, cfg)}")
