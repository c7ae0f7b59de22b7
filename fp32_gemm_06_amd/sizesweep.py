"""Square-size sweep of sgemm against the vendor library, as context.

The worklog compares its final kernel with the vendor BLAS across square
sizes and notes the vendor library's lead at small sizes, where too few
blocks fill the GPU ("CUDA 矩阵乘法优化：从朴素 Kernel 到接近 cuBLAS",
section "10. cuBLAS 领先的性能差异与全尺寸 Benchmark").  This repeats that
measurement on MI355X: sgemm through the C ABI against torch.matmul (which
calls the vendor library) on the same device buffers, alpha = 1, beta = 0,
fp32 with TF32 disabled.

    python -m fp32_gemm_06_amd.sizesweep --out sweep.jsonl
    python -m fp32_gemm_06_amd.sizesweep --out llm.jsonl --shapes 2048x11008x4096 ...

`--shapes` takes M x N x K products (row-major, op = nn) instead of squares.
"""
from __future__ import annotations

import argparse
import json

SIZES = [128, 256, 384, 512, 768, 1024, 1536, 2048, 3072, 4092, 4096]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", required=True)
    ap.add_argument("--sizes", type=int, nargs="*", default=SIZES)
    ap.add_argument("--ops", nargs="*", default=["nn"], choices=["nn", "nt", "tn", "tt"],
                    help="operand layouts: n = as given, t = stored transposed")
    ap.add_argument("--shapes", nargs="*", default=None,
                    help="MxNxK products to time instead of the squares (nn only)")
    ap.add_argument("--md", default=None, help="also write a markdown table here")
    a = ap.parse_args()

    import torch

    import fp32_gemm_06_amd as fg

    torch.backends.cuda.matmul.allow_tf32 = False
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def timed(fn, target_ms=60.0):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        one = max(e0.elapsed_time(e1), 1e-3)
        n = max(10, min(2000, int(target_ms / one)))
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3

    def describe(M, N, K):
        """The configuration sgemm runs: one tile, or two launches (round split)."""
        dim, first = fg.fp32gemm_round_split(M, N, K, 1)
        if dim == 0:
            return fg.fp32gemm_config_name(0, fg.fp32gemm_select_config(0, M, N, K))
        if dim == 1:
            rest = fg.fp32gemm_select_config(0, M, N - first, K)
            where = f"cols <{first}"
        else:
            rest = fg.fp32gemm_select_config(0, M - first, N, K)
            where = f"rows <{first}"
        return f"{where}: 256x256x32_w128x64_g8; rest: {fg.fp32gemm_config_name(0, rest)}"

    if a.shapes:
        cases = [tuple(int(v) for v in sh.lower().split("x")) + ("nn",) for sh in a.shapes]
    else:
        cases = [(n, n, n, op) for n in a.sizes for op in a.ops]

    # warm the clock before the first size
    big = torch.randn(4096, 4096, device=dev)
    for _ in range(60):
        torch.matmul(big, big)
    del big
    recs = []
    with open(a.out, "w") as out:
        for (M, N, K, op) in cases:
            ta, tb = int(op[0] == "t"), int(op[1] == "t")
            # storage: op(A) = A^T reads A stored K x M, op(B) = B^T reads B stored N x K
            A = torch.randn(K, M, device=dev) if ta else torch.randn(M, K, device=dev)
            B = torch.randn(N, K, device=dev) if tb else torch.randn(K, N, device=dev)
            C = torch.empty(M, N, device=dev)
            opA = A.t() if ta else A
            opB = B.t() if tb else B

            def ours():
                rc = fg.sgemm_ex(ta, tb, M, N, K, 1.0, A, A.shape[1], B, B.shape[1], 0.0, C, N,
                                 stream.cuda_stream)
                if rc:
                    raise fg.Fp32GemmError(rc)

            us_ours = timed(ours)
            us_vendor = timed(lambda: torch.matmul(opA, opB))
            ref = torch.matmul(opA.double(), opB.double())
            err = float(((C.double() - ref).abs() /
                         (opA.abs().double() @ opB.abs().double())).max())
            flop = 2.0 * M * N * K
            rec = {"M": M, "N": N, "K": K, "op": op, "us": round(us_ours, 3),
                   "tflops": round(flop / us_ours / 1e6, 3),
                   "vendor_us": round(us_vendor, 3),
                   "vendor_tflops": round(flop / us_vendor / 1e6, 3),
                   "ratio": round(us_vendor / us_ours, 3), "max_rel_err": err,
                   "config": describe(M, N, K)}
            print(json.dumps(rec), flush=True)
            out.write(json.dumps(rec) + "\n")
            recs.append(rec)
            del A, B, C, ref
    if a.md:
        lines = ["| M x N x K | op | sgemm us | sgemm TFLOP/s | vendor TFLOP/s | vendor time / ours "
                 "| max_rel_err | config |", "|---" * 8 + "|"]
        for r in recs:
            shape = f"{r['M']} x {r['N']} x {r['K']}"
            lines.append(f"| {shape} | {r['op']} | {r['us']} | {r['tflops']} | {r['vendor_tflops']} "
                         f"| {r['ratio']} | {r['max_rel_err']:.1e} | {r['config']} |")
        with open(a.md, "w") as f:
            f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
