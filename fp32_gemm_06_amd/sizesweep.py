"""Square-size sweep of sgemm against the vendor library, as context.

The worklog compares its final kernel with the vendor BLAS across square
sizes and notes the vendor library's lead at small sizes, where too few
blocks fill the GPU ("CUDA 矩阵乘法优化：从朴素 Kernel 到接近 cuBLAS",
section "10. cuBLAS 领先的性能差异与全尺寸 Benchmark").  This repeats that
measurement on MI355X: sgemm through the C ABI against torch.matmul (which
calls the vendor library) on the same device buffers, alpha = 1, beta = 0,
fp32 with TF32 disabled.

    python -m fp32_gemm_06_amd.sizesweep --out sweep.jsonl
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

    # warm the clock before the first size
    big = torch.randn(4096, 4096, device=dev)
    for _ in range(60):
        torch.matmul(big, big)
    del big
    recs = []
    with open(a.out, "w") as out:
        for n in a.sizes:
            for op in a.ops:
                ta, tb = int(op[0] == "t"), int(op[1] == "t")
                # storage: A is n x n either way; op(A) = A^T reads it transposed
                A = torch.randn(n, n, device=dev)
                B = torch.randn(n, n, device=dev)
                C = torch.empty(n, n, device=dev)
                opA = A.t() if ta else A
                opB = B.t() if tb else B

                def ours():
                    rc = fg.sgemm_ex(ta, tb, n, n, n, 1.0, A, n, B, n, 0.0, C, n, stream.cuda_stream)
                    if rc:
                        raise fg.Fp32GemmError(rc)

                us_ours = timed(ours)
                us_vendor = timed(lambda: torch.matmul(opA, opB))
                ref = torch.matmul(opA.double(), opB.double())
                err = float(((C.double() - ref).abs() /
                             (opA.abs().double() @ opB.abs().double())).max())
                rec = {"n": n, "op": op, "us": round(us_ours, 3),
                       "tflops": round(2 * n ** 3 / us_ours / 1e6, 3),
                       "vendor_us": round(us_vendor, 3),
                       "vendor_tflops": round(2 * n ** 3 / us_vendor / 1e6, 3),
                       "ratio": round(us_vendor / us_ours, 3), "max_rel_err": err,
                       "config": fg.fp32gemm_config_name(0, fg.fp32gemm_select_config(0, n, n, n))}
                print(json.dumps(rec), flush=True)
                out.write(json.dumps(rec) + "\n")
                recs.append(rec)
                del A, B, C
    if a.md:
        lines = ["| n | op | sgemm us | sgemm TFLOP/s | vendor TFLOP/s | vendor time / ours "
                 "| max_rel_err | config |", "|---" * 8 + "|"]
        for r in recs:
            lines.append(f"| {r['n']} | {r['op']} | {r['us']} | {r['tflops']} | {r['vendor_tflops']} "
                         f"| {r['ratio']} | {r['max_rel_err']:.1e} | {r['config']} |")
        with open(a.md, "w") as f:
            f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
