"""Fused against unfused epilogue: sgemm_fused (bias + ReLU applied in
registers before C is stored once) against sgemm followed by the same
elementwise chain as separate kernels (torch's in-place add of the bias row
and ReLU, each of which reads and writes C).

This is the measurement behind the operator-fusion argument of "GPU 基础原
理" (a translation of "Basic facts about GPUs"), section "4.1 算子融合": the
unfused chain moves the intermediate through HBM.  Same device buffers, fp32,
alpha = 1, beta = 0; weights stored N x K (y = x W^T + b, a linear layer) and
as given.

    python -m fp32_gemm_06_amd.epilogue_sweep --out sweep.jsonl --md table.md
"""
from __future__ import annotations

import argparse
import json

# (M, N, K, transB): prefill projections, the square benchmark, decode
SHAPES = [(2048, 11008, 4096, 1), (2048, 4096, 4096, 1), (4092, 4092, 4092, 0),
          (512, 11008, 4096, 1), (1, 11008, 4096, 1), (8, 11008, 4096, 1), (1, 4096, 4096, 0)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", required=True)
    ap.add_argument("--md", default=None)
    a = ap.parse_args()

    import torch

    import fp32_gemm_06_amd as fg

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def timed(fn, target_ms=40.0):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        one = max(e0.elapsed_time(e1), 1e-3)
        n = max(20, min(2000, int(target_ms / one)))
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3

    def check(rc):
        if rc:
            raise fg.Fp32GemmError(rc)

    big = torch.randn(4096, 4096, device=dev)   # warm the clock
    for _ in range(60):
        torch.matmul(big, big)
    del big
    recs = []
    with open(a.out, "w") as out:
        for (M, N, K, tb) in SHAPES:
            X = torch.randn(M, K, device=dev)
            W = torch.randn(N, K, device=dev) if tb else torch.randn(K, N, device=dev)
            ldb = K if tb else N
            bias = torch.randn(N, device=dev)
            C = torch.empty(M, N, device=dev)
            C2 = torch.empty(M, N, device=dev)

            def fused():
                check(fg.sgemm_fused(0, tb, M, N, K, 1.0, X, K, W, ldb, 0.0, C, N, bias,
                                     fg.ACT_RELU, sp))

            def unfused():
                check(fg.sgemm_ex(0, tb, M, N, K, 1.0, X, K, W, ldb, 0.0, C2, N, sp))
                C2.add_(bias)
                C2.relu_()

            def plain():
                check(fg.sgemm_ex(0, tb, M, N, K, 1.0, X, K, W, ldb, 0.0, C2, N, sp))

            rec = {"M": M, "N": N, "K": K, "transB": tb,
                   "plain_us": round(timed(plain), 3), "fused_us": round(timed(fused), 3),
                   "unfused_us": round(timed(unfused), 3)}
            fused()
            unfused()
            torch.cuda.synchronize()
            rec["max_abs_diff"] = float((C - C2).abs().max())
            rec["c_bytes"] = 4 * M * N
            print(json.dumps(rec), flush=True)
            out.write(json.dumps(rec) + "\n")
            recs.append(rec)
            del X, W, bias, C, C2
    if a.md:
        lines = ["| M x N x K | W stored | GEMM alone | fused bias + ReLU | GEMM, then add + ReLU kernels "
                 "| saved | C size | max fused - unfused |", "|---" * 8 + "|"]
        for r in recs:
            lines.append(f"| {r['M']} x {r['N']} x {r['K']} | {'N x K' if r['transB'] else 'K x N'} "
                         f"| {r['plain_us']:.1f} us | {r['fused_us']:.1f} us | {r['unfused_us']:.1f} us "
                         f"| {r['unfused_us'] - r['fused_us']:.1f} us | {r['c_bytes'] / 1e6:.1f} MB "
                         f"| {r['max_abs_diff']:.1e} |")
        with open(a.md, "w") as f:
            f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
