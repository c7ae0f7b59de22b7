"""The split-K GEMV (W stored K x N, 256-column blocks x K chunks, partial
sums added in chunk order by the last workgroup of each column block).

Its scratch-free form (one workgroup per column block walking the chunks)
adds the same partial sums in the same order, so the two must agree bit for
bit: a partial sum read before it was published, a counter left non-zero by
an earlier call, or two streams sharing scratch would all show as a
difference.  Both are also checked against the oracle."""
import numpy as np
import pytest

import fp32_gemm_06_amd as fg
import oracle
from fp32_gemm_06_amd import inputs
from gpu_util import assert_bitexact, assert_parity, require_gpu, run_hip

pytestmark = pytest.mark.gpu

SHAPES = [(1, 4096, 4096), (4, 4096, 4096), (8, 4096, 4096), (3, 1000, 777), (5, 333, 4099),
          (2, 16, 5000), (8, 11008, 4096), (7, 4100, 300), (1, 2048, 64), (6, 512, 2049)]


def _cfg(name):
    names = fg.config_names(fg.KIND_SGEMV)
    return names.index(name)


VARIANTS = ["split256_w4_u4", "split256_w8_u4"]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("shape", SHAPES, ids=str)
def test_split_matches_scratch_free_form_and_oracle(shape, variant):
    require_gpu()
    M, N, K = shape
    A, B, C0 = inputs.random_case(M * 1000 + N + K, M, N, K, kind="normal")
    split, canary = run_hip(A, B, C0, 0.75, -0.5, config=_cfg(variant), family="gemv",
                            guard=32)
    assert canary, "write outside C"
    serial, _ = run_hip(A, B, C0, 0.75, -0.5, config=_cfg(variant + "_serial"),
                        family="gemv")
    assert np.array_equal(split, serial), f"{shape}: split and scratch-free forms differ"
    assert_parity(split, oracle.sgemm(A, B, C0, 0.75, -0.5), oracle.bound(A, B, C0, 0.75, -0.5),
                  f"split {shape}")


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("shape", [(1, 4096, 4096), (8, 1000, 777), (4, 333, 4099)], ids=str)
def test_split_integer_exact(shape, variant):
    require_gpu()
    M, N, K = shape
    A, B, C0 = inputs.random_case(M + N + K, M, N, K, kind="int")
    got, canary = run_hip(A, B, C0, 1.0, 0.5, config=_cfg(variant), family="gemv", guard=32)
    assert canary
    assert_bitexact(got, oracle.sgemm(A, B, C0, 1.0, 0.5), f"int {shape}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_repeated_calls_reset_the_counters(variant):
    """Calls back to back on one stream with new inputs each time, shapes
    with different chunk counts in between: each equals the scratch-free form."""
    torch = require_gpu()
    dev = torch.device("cuda:0")
    split, serial = _cfg(variant), _cfg(variant + "_serial")
    for i, (M, N, K) in enumerate([(1, 4096, 4096), (8, 4096, 4096), (2, 1000, 777),
                                   (1, 4096, 4096), (5, 2048, 8192), (1, 4096, 4096)] * 2):
        g = inputs.rng(500 + i)
        X = torch.from_numpy(inputs.normal(g, (M, K))).to(dev)
        W = torch.from_numpy(inputs.normal(g, (K, N))).to(dev)
        outs = []
        for cfg in (split, serial):
            Y = torch.zeros(M, N, device=dev)
            rc = fg.fp32gemm_sgemv_with_config(cfg, M, N, K, 1.0, X, K, W, N, 0.0, Y, N)
            assert rc == 0, fg.strerror(rc)
            outs.append(Y)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1]), f"call {i} {(M, N, K)}"


@pytest.mark.parametrize("variant", VARIANTS)
def test_more_streams_than_scratch_slots(variant):
    """Twelve streams (the library keeps scratch for eight per device) run
    the product at once on different inputs; the streams without scratch
    take the scratch-free form.  Every result equals the scratch-free form
    computed alone."""
    torch = require_gpu()
    dev = torch.device("cuda:0")
    split, serial = _cfg(variant), _cfg(variant + "_serial")
    M, N, K = 4, 4096, 4096
    streams = [torch.cuda.Stream() for _ in range(12)]
    Xs, Ws, Ys = [], [], []
    for i in range(len(streams)):
        g = inputs.rng(900 + i)
        Xs.append(torch.from_numpy(inputs.normal(g, (M, K))).to(dev))
        Ws.append(torch.from_numpy(inputs.normal(g, (K, N))).to(dev))
        Ys.append(torch.zeros(M, N, device=dev))
    torch.cuda.synchronize()
    for rep in range(3):
        for i, st in enumerate(streams):
            rc = fg.fp32gemm_sgemv_with_config(split, M, N, K, 1.0, Xs[i], K, Ws[i], N, 0.0,
                                               Ys[i], N, st)
            assert rc == 0, fg.strerror(rc)
        torch.cuda.synchronize()
        for i in range(len(streams)):
            want = torch.zeros(M, N, device=dev)
            rc = fg.fp32gemm_sgemv_with_config(serial, M, N, K, 1.0, Xs[i], K, Ws[i], N, 0.0,
                                               want, N)
            assert rc == 0
            torch.cuda.synchronize()
            assert torch.equal(Ys[i], want), f"stream {i}, round {rep}"
