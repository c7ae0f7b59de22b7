"""Tile-configuration sweep and per-shape table generator.

The pages pick block and thread-tile sizes by timing every legal setting on
the target GPU and keeping the fastest ("CUDA 矩阵乘法优化：从朴素 Kernel 到接
近 cuBLAS", section "8. Kernel 9: 参数自动调优"); the best settings differ
from GPU to GPU.  This sweep does the same on MI355X over the library's
configurations (tile shape x tile-ordering group for SGEMM; unroll x
workgroup target for GEMV), through the C ABI with a forced configuration.

    python -m fp32_gemm_06_amd.tune --out results.jsonl     # on the GPU
    python -m fp32_gemm_06_amd.tune --table results.jsonl   # writes csrc/tune_table.inc

Results are appended one JSON line per (shape, configuration), so an
interrupted sweep resumes by skipping the keys already present.  Legality
(LDS <= 160 KB per workgroup, <= 512 registers per lane) is enforced at
compile time for every configuration in the library.
"""
from __future__ import annotations

import argparse
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
TABLE = os.path.join(HERE, "csrc", "tune_table.inc")

# (family, M, N, K, alpha, beta): the benchmark workloads, the square sizes of
# the pages' size comparison, and transformer projection shapes (prefill
# M = tokens; N, K = 4096 / 11008 hidden and FFN widths).
SHAPES = [
    ("gemm", 128, 128, 128, 1.0, 0.5),
    ("gemm", 4092, 4092, 4092, 1.0, 0.0),
    ("gemm", 4096, 4096, 4096, 0.5, 1.0),
    ("gemm", 2048, 11008, 4096, 1.0, 0.0),
    ("gemm", 256, 256, 256, 1.0, 0.0),
    ("gemm", 512, 512, 512, 1.0, 0.0),
    ("gemm", 768, 768, 768, 1.0, 0.0),
    ("gemm", 1024, 1024, 1024, 1.0, 0.0),
    ("gemm", 1536, 1536, 1536, 1.0, 0.0),
    ("gemm", 2048, 2048, 2048, 1.0, 0.0),
    ("gemm", 3072, 3072, 3072, 1.0, 0.0),
    ("gemm", 8192, 8192, 8192, 1.0, 0.0),
    ("gemm", 2048, 4096, 4096, 1.0, 0.0),
    ("gemm", 2048, 4096, 11008, 1.0, 0.0),
    ("gemm", 512, 11008, 4096, 1.0, 0.0),
    ("gemm", 512, 4096, 4096, 1.0, 0.0),
    ("gemv", 1, 4096, 4096, 1.0, 0.0),
    ("gemv", 4, 4096, 4096, 1.0, 0.0),
    ("gemv", 8, 4096, 4096, 1.0, 0.0),
    ("gemv", 1, 1024, 1024, 1.0, 0.0),
    ("gemv", 1, 2048, 2048, 1.0, 0.0),
    ("gemv", 1, 8192, 8192, 1.0, 0.0),
    ("gemv", 1, 11008, 4096, 1.0, 0.0),
    ("gemv", 8, 11008, 4096, 1.0, 0.0),
    ("gemv", 1, 4096, 11008, 1.0, 0.0),
    ("gemv", 8, 4096, 11008, 1.0, 0.0),
    ("gemv", 1, 16384, 4096, 1.0, 0.0),
    ("gemv", 1, 32000, 4096, 1.0, 0.0),
    ("gemv", 1, 65536, 1024, 1.0, 0.0),
    ("gemv", 2, 4096, 4096, 1.0, 0.0),
    ("gemv", 1, 3072, 4096, 1.0, 0.0),
    ("gemv", 1, 6144, 4096, 1.0, 0.0),
    ("gemv", 4, 11008, 4096, 1.0, 0.0),
    ("gemv", 4, 4096, 11008, 1.0, 0.0),
    ("gemv", 1, 4096, 8192, 1.0, 0.0),
    ("gemv", 1, 2048, 8192, 1.0, 0.0),
    ("gemv", 1, 14336, 4096, 1.0, 0.0),
    ("gemv", 1, 4096, 14336, 1.0, 0.0),
    ("gemv", 8, 8192, 8192, 1.0, 0.0),
    ("gemv", 4, 16384, 4096, 1.0, 0.0),
    ("gemv", 8, 14336, 4096, 1.0, 0.0),
]


def _key(fam, M, N, K, name):
    return f"{fam}:{M}x{N}x{K}:{name}"


def sweep(out_path: str, reps: int, warm: int, only: str | None):
    import torch

    import fp32_gemm_06_amd as fg

    done = set()
    if os.path.exists(out_path):
        with open(out_path) as f:
            for ln in f:
                if ln.strip():
                    done.add(json.loads(ln)["key"])
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    with open(out_path, "a") as out:
        for (fam, M, N, K, alpha, beta) in SHAPES:
            if only and only != fam:
                continue
            kind = fg.KIND_SGEMM if fam == "gemm" else fg.KIND_SGEMV
            A = torch.randn(M, K, device=dev)
            nbuf = 8 if fam == "gemv" else 1  # gemv: exceed the Infinity Cache
            Bs = [torch.randn(K, N, device=dev) for _ in range(nbuf)]
            C = torch.randn(M, N, device=dev)
            fn = fg.fp32gemm_sgemm_with_config if fam == "gemm" else fg.fp32gemm_sgemv_with_config
            auto = fg.fp32gemm_select_config(kind, M, N, K)
            for cfg in range(fg.fp32gemm_num_configs(kind)):
                name = fg.fp32gemm_config_name(kind, cfg)
                key = _key(fam, M, N, K, name)
                if key in done:
                    continue
                n = reps * (4 if fam == "gemv" else 1)

                def call(i):
                    rc = fn(cfg, M, N, K, alpha, A, K, Bs[i % nbuf], N, beta, C, N, sp)
                    if rc:
                        raise fg.Fp32GemmError(rc)

                for i in range(warm):
                    call(i)
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for i in range(n):
                    call(i)
                e1.record(stream)
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) / n * 1e3
                rec = {"key": key, "family": fam, "M": M, "N": N, "K": K, "config": name,
                       "us": round(us, 3), "auto": cfg == auto}
                if fam == "gemm":
                    rec["tflops"] = round(2.0 * M * N * K / (us * 1e-6) / 1e12, 3)
                else:
                    b = 4 * (M * K + K * N + M * N)
                    rec["gbps"] = round(b / (us * 1e-6) / 1e9, 1)
                out.write(json.dumps(rec) + "\n")
                out.flush()
                print(json.dumps(rec), flush=True)
            del A, Bs, C
            torch.cuda.empty_cache()


# SGEMM near-ties.  Tiles: the 4-wave 64x64 tile, four workgroups to a CU,
# varies most from GPU to GPU (at 2048^3 it timed 0.3% ahead of 128x128 on
# the sweep's GPU and 8% behind on another), so within TIE_TILE of the fastest
# time the largest tile wins.  Groups: tile-ordering groups of one tile shape
# often time within the sweep's noise of each other, but a larger group
# shares more A and B panels in each XCD's L2 (at 4092^3, group 8 fetched
# 407 MB per launch from the fabric against 603 MB for group 2), so within
# TIE of that tile's fastest time the largest group wins.
TIE_TILE = 0.01
TIE = 0.005


def _tile_area(config: str) -> int:
    bm, bn = config.split("x")[:2]
    return int(bm) * int(bn)


def best_by_shape(path: str):
    rows = {}
    with open(path) as f:
        for ln in f:
            if not ln.strip():
                continue
            r = json.loads(ln)
            rows.setdefault((r["family"], r["M"], r["N"], r["K"]), []).append(r)
    best = {}
    for k, rs in rows.items():
        b = min(rs, key=lambda r: r["us"])
        if k[0] == "gemm":
            near = [r for r in rs if r["us"] <= b["us"] * (1 + TIE_TILE)]
            area = max(_tile_area(r["config"]) for r in near)
            b = min((r for r in near if _tile_area(r["config"]) == area), key=lambda r: r["us"])
            tile = b["config"].rsplit("_g", 1)[0]
            same = [r for r in rs if r["config"].rsplit("_g", 1)[0] == tile
                    and r["us"] <= b["us"] * (1 + TIE)]
            b = max(same, key=lambda r: int(r["config"].rsplit("_g", 1)[1]))
        best[k] = b
    return best


def write_table(path: str, table: str = TABLE):
    best = best_by_shape(path)
    lines = [
        "// Per-shape configuration table.  Written by fp32_gemm_06_amd/tune.py from a",
        "// timing sweep on MI355X; entries name a configuration (tile shape and tile",
        "// ordering group for SGEMM, unroll and workgroup target for GEMV).",
        "// {M, N, K, \"configuration name\"}",
        "static const ShapeEntry kGemmTable[] = {",
    ]
    for (fam, M, N, K), r in sorted(best.items()):
        if fam == "gemm":
            lines.append(f"    {{{M}, {N}, {K}, \"{r['config']}\"}},  // {r['us']} us")
    lines.append("};")
    lines.append("static const ShapeEntry kGemvTable[] = {")
    for (fam, M, N, K), r in sorted(best.items()):
        if fam == "gemv":
            lines.append(f"    {{{M}, {N}, {K}, \"{r['config']}\"}},  // {r['us']} us")
    lines.append("};")
    with open(table, "w") as f:
        f.write("\n".join(lines) + "\n")
    return table


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None, help="append sweep results (JSON lines) here")
    ap.add_argument("--table", default=None, help="write tune_table.inc from these results")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--warm", type=int, default=5)
    ap.add_argument("--only", choices=["gemm", "gemv"], default=None)
    a = ap.parse_args()
    if a.out:
        sweep(a.out, a.reps, a.warm, a.only)
    if a.table:
        print(write_table(a.table))
    if not a.out and not a.table:
        ap.print_help()
        sys.exit(1)


if __name__ == "__main__":
    main()
