"""Decode-batch sweep: the product of M token rows (M = 1..256, several
sequences decoded at once) with a weight matrix, for both weight layouts,
against the vendor library.

The decode GEMMs of an LLM stream the weights once per step ("GPU GEMM 优化完
全拆解（一）", section "LLM 推理本质上是 GEMM 的串联"), so their time is the
weight read until M is large.  Each call cycles through 8 copies of the weight
(more than the Infinity Cache holds), so every call reads it from HBM.  The
library routes by M: the GEMV kernels up to 8 rows, the skinny MFMA kernel up
to 128 where it pays, the tiled kernel beyond.  `nn`: W stored K x N
(`sgemm`); `nt`: W stored N x K (`sgemm_ex(N, T)`, a linear layer's weight).
The vendor library is torch.matmul on the same buffers (x @ W and x @ W_t.t()),
fp32 with TF32 disabled.

    python -m fp32_gemm_06_amd.decode_sweep --out sweep.jsonl --md table.md
"""
from __future__ import annotations

import argparse
import json

SHAPES = [(4096, 4096), (11008, 4096), (4096, 11008)]
ROWS = [1, 8, 9, 16, 32, 48, 64, 96, 128, 192, 256]
COPIES = 8


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", required=True)
    ap.add_argument("--md", default=None, help="also write a markdown table here")
    ap.add_argument("--rows", type=int, nargs="*", default=ROWS)
    a = ap.parse_args()

    import torch

    import fp32_gemm_06_amd as fg

    torch.backends.cuda.matmul.allow_tf32 = False
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def timed(fn, it=100):
        for i in range(10):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(it):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / it * 1e3

    def check(rc):
        if rc:
            raise fg.Fp32GemmError(rc)

    # warm the clock
    big = torch.randn(4096, 4096, device=dev)
    for _ in range(60):
        torch.matmul(big, big)
    del big
    recs = []
    with open(a.out, "w") as out:
        for (N, K) in SHAPES:
            W = [torch.randn(K, N, device=dev) for _ in range(COPIES)]
            Wt = [torch.randn(N, K, device=dev) for _ in range(COPIES)]
            for M in a.rows:
                X = torch.randn(M, K, device=dev)
                Y = torch.empty(M, N, device=dev)
                rec = {"M": M, "N": N, "K": K}
                rec["nn_us"] = round(timed(lambda i: check(
                    fg.sgemm(M, N, K, 1.0, X, K, W[i % COPIES], N, 0.0, Y, N, sp))), 2)
                last = (100 - 1) % COPIES  # the weight copy of the last timed call
                ref = X.double() @ W[last].double()
                rec["nn_err"] = float(((Y.double() - ref).abs()
                                       / (X.abs().double() @ W[last].abs().double())).max())
                rec["nn_vendor_us"] = round(timed(lambda i: torch.matmul(X, W[i % COPIES])), 2)
                rec["nt_us"] = round(timed(lambda i: check(
                    fg.sgemm_ex(0, 1, M, N, K, 1.0, X, K, Wt[i % COPIES], K, 0.0, Y, N, sp))), 2)
                ref = X.double() @ Wt[last].double().t()
                rec["nt_err"] = float(((Y.double() - ref).abs()
                                       / (X.abs().double() @ Wt[last].abs().double().t())).max())
                rec["nt_vendor_us"] = round(timed(lambda i: torch.matmul(X, Wt[i % COPIES].t())), 2)
                print(json.dumps(rec), flush=True)
                out.write(json.dumps(rec) + "\n")
                recs.append(rec)
            del W, Wt
            torch.cuda.empty_cache()
    if a.md:
        lines = ["| M | N x K | nn us | vendor nn us | vendor / ours | nt us | vendor nt us "
                 "| vendor / ours | max_rel_err |", "|---" * 9 + "|"]
        for r in recs:
            lines.append(
                f"| {r['M']} | {r['N']} x {r['K']} | {r['nn_us']} | {r['nn_vendor_us']} "
                f"| {r['nn_vendor_us'] / r['nn_us']:.2f} | {r['nt_us']} | {r['nt_vendor_us']} "
                f"| {r['nt_vendor_us'] / r['nt_us']:.2f} | {max(r['nn_err'], r['nt_err']):.1e} |")
        with open(a.md, "w") as f:
            f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
