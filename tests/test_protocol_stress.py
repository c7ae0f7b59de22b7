"""The in-kernel cross-workgroup protocols under many interleaved calls.

The split GEMV and stream-K keep arrival counters in per-stream device
memory that every call must leave at zero, and they share each stream's slot
across shapes with different counter counts.  Two streams each run 60 rounds
of a mixed sequence (split GEMV at M = 1, 4 and 8 with 16, 5 and 32 chunks;
stream-K on both tiles with plans that share tiles, including one with its
counters in the workspace; the no-allocation split-K), back to back with no
host synchronisation inside a round.  Integer-valued inputs make every sum
exact, so every call must reproduce the oracle bit for bit."""
import numpy as np
import pytest

import fp32_gemm_06_amd as fg
import oracle
from fp32_gemm_06_amd import inputs
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu

ROUNDS = 60


def _gemv_case(torch, seed, M, N, K):
    A, B, C0 = inputs.random_case(seed, M, N, K, kind="int")
    want = oracle.sgemm(A, B, C0, 1.0, 0.5)
    return dict(kind="gemv", M=M, N=N, K=K, A=torch.from_numpy(A).cuda(),
                B=torch.from_numpy(B).cuda(), C0=torch.from_numpy(C0).cuda(), want=want)


def _sk_case(torch, seed, M, N, K, tile, groups):
    A, B, C0 = inputs.random_case(seed, M, N, K, kind="int")
    want = oracle.sgemm(A, B, C0, 1.0, 0.5)
    wsb = fg.fp32gemm_streamk_plan(M, N, K, tile, groups)[0]
    return dict(kind="sk", M=M, N=N, K=K, tile=tile, groups=groups, wsb=wsb,
                A=torch.from_numpy(A).cuda(), B=torch.from_numpy(B).cuda(),
                C0=torch.from_numpy(C0).cuda(), want=want)


def _noalloc_case(torch, seed, M, N, K, splits):
    A, B, C0 = inputs.random_case(seed, M, N, K, kind="int")
    want = oracle.sgemm(A, B, C0, 1.0, 0.5)
    return dict(kind="noalloc", M=M, N=N, K=K, splits=splits, A=torch.from_numpy(A).cuda(),
                B=torch.from_numpy(B).cuda(), C0=torch.from_numpy(C0).cuda(), want=want)


def test_interleaved_calls_on_two_streams_stay_exact():
    torch = require_gpu()
    split = {fg.fp32gemm_config_name(1, i): i for i in range(fg.fp32gemm_num_configs(1))}
    cases = [
        _gemv_case(torch, 11, 1, 4096, 4096),     # 16 column blocks x 16 chunks
        _sk_case(torch, 12, 300, 520, 1000, 0, 7),
        _gemv_case(torch, 13, 4, 11008, 1024),    # many column blocks, few chunks
        _sk_case(torch, 14, 4160, 4160, 96, 1, 0),  # > 4096 tiles: counters in the workspace
        _gemv_case(torch, 15, 8, 2048, 8192),     # 32 chunks
        _noalloc_case(torch, 16, 256, 256, 8192, 16),
        _sk_case(torch, 17, 129, 67, 4099, 1, 5),
    ]
    # the split GEMV runs through its forced configuration (the 8-wave form for M = 8)
    for c in cases:
        if c["kind"] == "gemv":
            c["cfg"] = split["split256_w8_u4" if c["M"] > 4 else "split256_w4_u4"]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = {}
    for s_i, st in enumerate(streams):
        for c_i, c in enumerate(cases):
            outs[s_i, c_i] = torch.empty(c["M"], c["N"], device="cuda")
            if c["kind"] == "sk":
                c.setdefault("ws", {})[s_i] = torch.empty(max(c["wsb"], 4) // 4, device="cuda")
    torch.cuda.synchronize()

    def launch(s_i, st, c_i, c):
        Y = outs[s_i, c_i]
        Y.copy_(c["C0"])
        M, N, K = c["M"], c["N"], c["K"]
        if c["kind"] == "gemv":
            rc = fg.fp32gemm_sgemv_with_config(c["cfg"], M, N, K, 1.0, c["A"], K, c["B"], N, 0.5,
                                               Y, N, st)
        elif c["kind"] == "sk":
            rc = fg.fp32gemm_streamk_with_config(c["tile"], c["groups"], 0, 0, M, N, K, 1.0,
                                                 c["A"], K, c["B"], N, 0.5, Y, N, c["ws"][s_i],
                                                 c["wsb"], st)
        else:
            rc = fg.sgemm_splitk_noalloc(0, 0, M, N, K, 1.0, c["A"], K, c["B"], N, 0.5, Y, N,
                                         c["splits"], st)
        assert rc == 0, (c["kind"], fg.strerror(rc))

    for rnd in range(ROUNDS):
        for s_i, st in enumerate(streams):
            with torch.cuda.stream(st):
                # the no-allocation split-K shares one scratch per device: only
                # stream 0 runs it, so calls on the two streams never overlap in it
                for c_i, c in enumerate(cases):
                    if c["kind"] == "noalloc" and s_i != 0:
                        continue
                    launch(s_i, st, c_i, c)
        if rnd % 15 == 14 or rnd == ROUNDS - 1:
            torch.cuda.synchronize()
            for (s_i, c_i), Y in outs.items():
                c = cases[c_i]
                if c["kind"] == "noalloc" and s_i != 0:
                    continue
                got = Y.cpu().numpy().astype(np.float64)
                assert np.array_equal(got, c["want"]), (rnd, s_i, c["kind"], c["M"], c["N"], c["K"])
