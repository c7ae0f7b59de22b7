"""HIP path vs the CPU oracle on the benchmark workloads and across tile configurations.

Tolerance (every element): |C - C_ref| <= 1e-4 * (|alpha| (|A||B|) + |beta| |C0|);
a non-finite reference value must be matched exactly (same NaN / same-signed Inf).
"""
import numpy as np
import pytest

import fp32_gemm_06_amd as fg
import oracle
from fp32_gemm_06_amd import inputs
from gpu_util import assert_parity, require_gpu, run_hip

pytestmark = pytest.mark.gpu


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
def test_workload_every_element(name):
    """Full-size workloads in the launch configuration the benchmark uses:
    every element of C against the oracle.  The prefill product runs as two
    launches (whole rounds of 256x256 tiles over the first columns, the rest
    on its own tile), so both launches and their seam are covered."""
    require_gpu()
    w = inputs.WORKLOADS[name]
    A, B, C0 = inputs.make(w)
    got, _ = run_hip(A, B, C0, w.alpha, w.beta)
    ref = oracle.sgemm(A, B, C0, w.alpha, w.beta)
    bnd = oracle.bound(A, B, C0, w.alpha, w.beta)
    print(name, "worst ratio", assert_parity(got, ref, bnd, name),
          "round split", fg.fp32gemm_round_split(w.M, w.N, w.K))
    assert np.all(np.isfinite(got)), "non-finite output"


def test_prefill_runs_as_two_launches():
    """The every-element prefill check above covers both launches of the
    round split; this pins that the split is what runs."""
    require_gpu()
    dim, first = fg.fp32gemm_round_split(2048, 11008, 4096)
    assert dim == 1 and 0 < first < 11008 and first % 256 == 0


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
