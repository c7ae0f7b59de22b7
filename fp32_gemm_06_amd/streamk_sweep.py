"""Stream-K sweep: sgemm, sgemm_splitk (the library's chunk count),
sgemm_streamk (the library's plan), every stream-K candidate (each tile at
256, 512, 768 and 1024 workgroups: one to four per CU) and the vendor
library, on shapes whose tiles fill the GPU badly (one to two rounds of
tiles, few tiles with a long K, decode batches of 48 to 288 rows) and on
larger ones.  Operands stay resident between calls (no rotation of B).

The worklog attributes part of the vendor BLAS's lead on such grids to
splitting K ("CUDA 矩阵乘法优化：从朴素 Kernel 到接近 cuBLAS", section
"10. cuBLAS 领先的性能差异与全尺寸 Benchmark").  Same device buffers, alpha =
1, beta = 0, fp32 with TF32 disabled; the vendor library is torch.matmul.
The table also gives how much slower the library's plan is than the best
candidate.  Its error column compares the plan's output with a float64 torch
product on the GPU, a sanity check of the timed runs; parity against the
oracle is tests/test_streamk.py.

    python -m fp32_gemm_06_amd.streamk_sweep --out sweep.jsonl --md table.md
"""
from __future__ import annotations

import argparse
import json

SHAPES = [(768, 768, 768), (1024, 1024, 1024), (1024, 1024, 4096), (1536, 1536, 1536),
          (2000, 2000, 2000), (384, 4096, 4096), (512, 4096, 4096), (768, 4096, 4096),
          (256, 256, 32768), (512, 512, 8192), (1024, 1024, 16384), (160, 4096, 4096),
          (48, 4096, 4096), (96, 11008, 4096), (128, 11008, 4096), (192, 11008, 4096),
          (256, 11008, 4096), (288, 4096, 4096), (96, 4096, 11008),
          (2048, 11008, 4096), (3072, 3072, 3072), (4096, 4096, 4096)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", required=True)
    ap.add_argument("--md", default=None, help="also write a markdown table here")
    ap.add_argument("--shapes", nargs="*", default=None, help="MxNxK ...")
    ap.add_argument("--configs", nargs="*", default=None,
                    help="stream-K candidates as tile:groups (default: every tile at 256, "
                         "512, 768 and 1024 workgroups)")
    a = ap.parse_args()

    import torch

    import fp32_gemm_06_amd as fg

    torch.backends.cuda.matmul.allow_tf32 = False
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    shapes = SHAPES if not a.shapes else [tuple(int(v) for v in s.split("x")) for s in a.shapes]

    def timed(fn, target_ms=30.0):
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

    def check(rc):
        if rc:
            raise fg.Fp32GemmError(rc)

    ntiles = 0
    while fg.fp32gemm_streamk_tile_name(ntiles) is not None:
        ntiles += 1
    if a.configs:
        cands = [tuple(int(v) for v in c.split(":")) for c in a.configs]
    else:
        cands = [(t, g) for t in range(ntiles) for g in (256, 512, 768, 1024)]
    big = torch.randn(4096, 4096, device=dev)   # warm the clock
    for _ in range(60):
        torch.matmul(big, big)
    del big
    recs = []
    with open(a.out, "w") as out:
        for (M, N, K) in shapes:
            A = torch.randn(M, K, device=dev)
            B = torch.randn(K, N, device=dev)
            C = torch.empty(M, N, device=dev)
            fl = 2.0 * M * N * K
            rec = {"M": M, "N": N, "K": K}
            rec["plain_us"] = timed(lambda: check(fg.sgemm(M, N, K, 1.0, A, K, B, N, 0.0, C, N,
                                                           sp)))
            wsb = fg.sgemm_splitk_workspace_size(M, N, K, 0)
            W = torch.empty(max(wsb // 4, 1), device=dev)
            rec["splitk_us"] = timed(lambda: check(fg.sgemm_splitk(
                0, 0, M, N, K, 1.0, A, K, B, N, 0.0, C, N, 0, W, wsb, sp)))
            rec["splitk_chunks"] = wsb // (4 * M * N) if wsb else 1
            del W
            wsb, t, g, ipw = fg.fp32gemm_streamk_plan(M, N, K)
            W = torch.empty(max(wsb // 4, 1), device=dev)
            rec["streamk_us"] = timed(lambda: check(fg.sgemm_streamk(
                0, 0, M, N, K, 1.0, A, K, B, N, 0.0, C, N, W, wsb, sp)))
            rec["streamk_plan"] = f"{fg.fp32gemm_streamk_tile_name(t)} g{g} ipw{ipw}"
            ref = torch.matmul(A.double(), B.double())
            rec["streamk_max_rel_err"] = float(((C.double() - ref).abs() /
                                                (A.abs().double() @ B.abs().double())).max())
            del W
            for tile, groups in cands:
                wsb, _, g, ipw = fg.fp32gemm_streamk_plan(M, N, K, tile, groups)
                W = torch.empty(max(wsb // 4, 1), device=dev)
                rec[f"sk{tile}_g{groups}_us"] = timed(lambda: check(
                    fg.fp32gemm_streamk_with_config(tile, groups, 0, 0, M, N, K, 1.0, A, K, B, N,
                                                    0.0, C, N, W, wsb, sp)))
                rec[f"sk{tile}_g{groups}_plan"] = f"g{g} ipw{ipw}"
                del W
            rec["vendor_us"] = timed(lambda: torch.matmul(A, B, out=C))
            for k in list(rec):
                if k.endswith("_us"):
                    rec[k] = round(rec[k], 3)
                    rec[k.replace("_us", "_tflops")] = round(fl / rec[k] / 1e6, 2)
            print(json.dumps(rec), flush=True)
            out.write(json.dumps(rec) + "\n")
            recs.append(rec)
            del A, B, C, ref
            torch.cuda.empty_cache()
    if a.md:
        names = [fg.fp32gemm_streamk_tile_name(t) for t in range(ntiles)]
        lines = ["| M x N x K | sgemm | split-K [chunks] | stream-K plan | best stream-K candidate "
                 "| plan vs best | vendor | stream-K max rel err |",
                 "|---" * 8 + "|"]
        for r in recs:
            def cell(k):
                return f"{r[k + '_us']:.1f} us ({r[k + '_tflops']:.1f})"
            cands = [k[:-3] for k in r if k.startswith("sk") and k.endswith("_us")]
            best = min(cands, key=lambda k: r[k + "_us"])
            t = int(best[2:best.index("_")])
            lines.append(
                f"| {r['M']} x {r['N']} x {r['K']} | {cell('plain')} | {cell('splitk')} "
                f"[{r['splitk_chunks']}] | {cell('streamk')} [{r['streamk_plan']}] | "
                f"{cell(best)} [{names[t]} {r[best + '_plan']}] | "
                f"{(r['streamk_us'] / r[best + '_us'] - 1) * 100:+.1f}% | {cell('vendor')} | "
                f"{r['streamk_max_rel_err']:.1e} |")
        with open(a.md, "w") as f:
            f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
