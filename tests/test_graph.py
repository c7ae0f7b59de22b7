"""The entry points under HIP graph capture (torch.cuda.CUDAGraph).

The library launches kernels only (no allocation, no memset), so a captured
sequence replays the same work.  Each replay runs on new input contents
copied into the captured buffers, with eager work and synchronisations in
between, and must give bit-identical results to the same calls run eagerly
(every kernel here has a fixed summation order).
"""
import numpy as np
import pytest

import fp32_gemm_06_amd as fg
from fp32_gemm_06_amd import inputs
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


def test_captured_sequence_replays_bit_identically():
    torch = require_gpu()
    dev = torch.device("cuda:0")
    M, N, K = 520, 780, 1000          # tiled kernel with ragged tiles
    m, n, k = 4, 3000, 2048           # GEMV (column stripes and row dots)
    H, S, D = 8, 1024, 128            # batched decode attention scores
    A = torch.empty(M, K, device=dev)
    B = torch.empty(K, N, device=dev)
    bias = torch.empty(N, device=dev)
    x = torch.empty(m, k, device=dev)
    W = torch.empty(k, n, device=dev)
    Wt = torch.empty(n, k, device=dev)
    q = torch.empty(H, 1, D, device=dev)
    kc = torch.empty(H, S, D, device=dev)
    wsb = fg.sgemm_splitk_workspace_size(M, N, K, 4)
    ws = torch.empty(wsb // 4, device=dev)
    # stream-K: the library's plan, and a forced one whose workgroups span
    # several tiles and cut tiles into many segments
    skb = fg.sgemm_streamk_workspace_size(M, N, K)
    skw = torch.empty(skb // 4, device=dev)
    skb2 = fg.fp32gemm_streamk_plan(M, N, K, 1, 37)[0]
    skw2 = torch.empty(skb2 // 4, device=dev)
    outs = {name: torch.empty(shape, device=dev) for name, shape in (
        ("sgemm", (M, N)), ("fused", (M, N)), ("splitk", (M, N)), ("streamk", (M, N)),
        ("streamk_forced", (M, N)), ("gemv", (m, n)),
        ("rows", (m, n)), ("scores", (H, 1, S)))}

    def fill(seed):
        g = inputs.rng(seed)
        for t in (A, B, bias, x, W, Wt, q, kc):
            t.copy_(torch.from_numpy(inputs.uniform(g, tuple(t.shape))))
        for t in outs.values():
            t.fill_(1.0)      # beta = 0.5 below reads C

    def calls():
        o = outs
        rcs = [
            fg.sgemm(M, N, K, 1.0, A, K, B, N, 0.5, o["sgemm"], N),
            fg.sgemm_fused(0, 0, M, N, K, 1.0, A, K, B, N, 0.5, o["fused"], N, bias, fg.ACT_RELU),
            fg.sgemm_splitk(0, 0, M, N, K, 1.0, A, K, B, N, 0.5, o["splitk"], N, 4, ws, wsb),
            fg.sgemm_streamk(0, 0, M, N, K, 1.0, A, K, B, N, 0.5, o["streamk"], N, skw, skb),
            fg.fp32gemm_streamk_with_config(1, 37, 0, 0, M, N, K, 1.0, A, K, B, N, 0.5,
                                            o["streamk_forced"], N, skw2, skb2),
            fg.sgemv(m, n, k, 1.0, x, k, W, n, 0.5, o["gemv"], n),
            fg.sgemm_ex(0, 1, m, n, k, 1.0, x, k, Wt, k, 0.5, o["rows"], n),
            fg.sgemm_strided_batched(0, 1, 1, S, D, 0.088, q, D, D, kc, D, S * D, 0.5,
                                     o["scores"], S, S, H),
        ]
        assert all(rc == 0 for rc in rcs), rcs

    # eager reference results for three input sets
    want = []
    for seed in (1, 2, 3):
        fill(seed)
        calls()
        torch.cuda.synchronize()
        want.append({name: t.clone() for name, t in outs.items()})

    # capture once (warm the side stream first, as graph capture requires)
    fill(1)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    fill(1)
    with torch.cuda.graph(graph):
        calls()

    for i, seed in enumerate((1, 2, 3)):
        fill(seed)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t in outs.items():
            assert torch.equal(t, want[i][name]), f"replay {i}: {name} differs from the eager result"
        # unrelated eager work between replays
        torch.matmul(A, B)
        torch.cuda.synchronize()
