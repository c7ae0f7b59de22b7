#!/usr/bin/env python3
"""Benchmark: fp32 SGEMM at 4092^3 and the M=1 decode GEMV on one MI355X.

One step is one full sgemm() call on the 4092 x 4092 x 4092 workload
(alpha = 1, beta = 0, A, B ~ U[-1, 1)), the square fp32 product the worklog
benchmarks ("CUDA 矩阵乘法优化：从朴素 Kernel 到接近 cuBLAS", table at the top
of the page).  Inputs are resident in HBM before timing starts; W steps are
warm-up, then K steps are timed with HIP events on the stream the kernels run
on, bracketed by device synchronisations.  The default warm-up (60 steps,
about 60 ms) covers the clock ramp: the first ~30 dispatches after the GPU
wakes run slower while the clock rises.  The decode GEMV (M = 1, K = N =
4096) is timed in the same run, cycling over enough weight copies that each
call streams its weights from HBM rather than from the 256 MB Infinity Cache.

Prints one JSON line.  Extra keys: "roofline" (dominant kernel against the
fp32 matrix peak), "gemv" (decode GEMV bandwidth against HBM peak),
"cpu_baseline" (the CPU oracle timed on a bounded sample of the workload),
"parity" (sampled rows of this run's output against the oracle).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [os.path.join(ROOT, "fp32_gemm_06_amd", "csrc", f)
                  for f in ("sgemm_kernel.h", "sgemm_nn.hip", "common.h", "tune_table.inc")]
GEMV_SOURCES = [os.path.join(ROOT, "fp32_gemm_06_amd", "csrc", f)
                for f in ("sgemv.hip", "common.h", "tune_table.inc")]


def source_hash(paths) -> str:
    """Hash of the kernel code (comments excluded), as the profile summaries record it."""
    from fp32_gemm_06_amd.profiling import source_hash as code_hash
    return code_hash(paths)


def stored_traffic(name: str, paths):
    """HBM bytes per launch measured with rocprofv3 counters, if they were taken
    on the current kernel source; otherwise None."""
    path = os.path.join(PROFILES, f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(paths):
        return None
    return rec.get("bytes_per_launch")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=60)
    p.add_argument("--gemv-steps", type=int, default=400)
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample (0 disables)")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="also run a plain device copy of this size (counter calibration)")
    p.add_argument("--skip-gemv", action="store_true")
    return p.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); this library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp32_gemm_06_amd as fg
    from fp32_gemm_06_amd import accounting as acc
    from fp32_gemm_06_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fg.lib()  # fail loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def check(rc):
        if rc != 0:
            raise fg.Fp32GemmError(rc)

    # ---------------- SGEMM 4092^3 ----------------
    w = inputs.WORKLOADS["sgemm_4092_uniform"]
    A, B, C0 = inputs.make(w)
    dA = torch.from_numpy(A).to(dev)
    dB = torch.from_numpy(B).to(dev)
    dC = torch.from_numpy(C0).to(dev)
    M, N, K = w.M, w.N, w.K
    cfg = fg.fp32gemm_select_config(fg.KIND_SGEMM, M, N, K)
    cfg_name = fg.fp32gemm_config_name(fg.KIND_SGEMM, cfg)

    def step():
        check(fg.sgemm(M, N, K, w.alpha, dA, K, dB, N, w.beta, dC, N, sp))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    flop = acc.flops(M, N, K)
    tflops = flop / (ms * 1e-3) / 1e12

    # parity of this run's output on sampled rows (cheap, host oracle)
    parity = None
    try:
        import oracle
        rows = np.array([0, 1, 2047, M - 2, M - 1], dtype=np.int32)
        rr = np.repeat(rows, N).astype(np.int32)
        cc = np.tile(np.arange(N, dtype=np.int32), len(rows))
        got = dC.cpu().numpy()[rr, cc].astype(np.float64)
        ref = oracle.sgemm_entries(rr, cc, A, B, C0, w.alpha, w.beta)
        bnd = oracle.bound_entries(rr, cc, A, B, C0, w.alpha, w.beta)
        ok, worst = oracle.within_tolerance(got, ref, bnd)
        parity = {"rows": [int(r) for r in rows], "ok": bool(ok), "worst_err_over_tol": worst}
    except Exception as e:  # the number is still reported; the failure is visible
        parity = {"error": repr(e)}

    # optional calibration kernel for the HBM byte counters: an elementwise
    # negation reads and writes exactly n * 4 bytes each way
    calib = None
    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.empty(n, dtype=torch.float32, device=dev).uniform_()
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        calib = {"kernel": "torch.neg", "bytes_each_way": n * 4, "launches": 3}
        del src, dst

    # ---------------- GEMV M=1, K=N=4096 ----------------
    gemv = None
    if not args.skip_gemv:
        gw = inputs.WORKLOADS["decode_m1_4096"]
        X, W, Y0 = inputs.make(gw)
        # enough distinct weight copies to exceed the 256 MB Infinity Cache
        nbuf = 8
        dX = torch.from_numpy(X).to(dev)
        dWs = [torch.from_numpy(W).to(dev)]
        for _ in range(nbuf - 1):
            dWs.append(dWs[0].clone())
        dY = torch.zeros((gw.M, gw.N), dtype=torch.float32, device=dev)
        gcfg = fg.fp32gemm_select_config(fg.KIND_SGEMV, gw.M, gw.N, gw.K)

        def gstep(i):
            check(fg.sgemv(gw.M, gw.N, gw.K, gw.alpha, dX, gw.K, dWs[i % nbuf], gw.N, gw.beta,
                           dY, gw.N, sp))

        for i in range(32):
            gstep(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.gemv_steps):
            gstep(i)
        e1.record(stream)
        torch.cuda.synchronize()
        gus = e0.elapsed_time(e1) / args.gemv_steps * 1e3
        gbytes = acc.algorithmic_bytes(gw.M, gw.N, gw.K, gw.beta)
        gbps = gbytes / (gus * 1e-6) / 1e9
        # warm: one weight buffer, served largely from the Infinity Cache
        e0.record(stream)
        for i in range(args.gemv_steps):
            check(fg.sgemv(gw.M, gw.N, gw.K, gw.alpha, dX, gw.K, dWs[0], gw.N, gw.beta, dY, gw.N,
                           sp))
        e1.record(stream)
        torch.cuda.synchronize()
        warm_us = e0.elapsed_time(e1) / args.gemv_steps * 1e3
        gemv = {
            "metric": "GEMV HBM GB/s at M=1, K=N=4096",
            "value": round(gbps, 1), "unit": "GB/s", "us_per_call": round(gus, 3),
            "calls": args.gemv_steps, "weight_buffers": nbuf,
            "config": fg.fp32gemm_config_name(fg.KIND_SGEMV, gcfg),
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": acc.PEAK_HBM_GBPS,
                         "unit": "GB/s", "frac": round(gbps / acc.PEAK_HBM_GBPS, 4),
                         "traffic": stored_traffic("gemv_m1_4096", GEMV_SOURCES)},
            "warm_single_buffer": {"us_per_call": round(warm_us, 3),
                                   "GB/s": round(gbytes / (warm_us * 1e-6) / 1e9, 1)},
        }
        # the same decode with the weight stored N x K (a linear layer's
        # layout, y = x W^T): sgemm_ex(N, T) runs the row-dot kernel
        dWt = [dWs[0].t().contiguous()]
        del dWs
        for _ in range(nbuf - 1):
            dWt.append(dWt[0].clone())

        def tstep(i):
            check(fg.sgemm_ex(0, 1, gw.M, gw.N, gw.K, gw.alpha, dX, gw.K, dWt[i % nbuf], gw.K,
                              gw.beta, dY, gw.N, sp))

        for i in range(32):
            tstep(i)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.gemv_steps):
            tstep(i)
        e1.record(stream)
        torch.cuda.synchronize()
        tus = e0.elapsed_time(e1) / args.gemv_steps * 1e3
        tbps = gbytes / (tus * 1e-6) / 1e9
        gemv["weight_stored_transposed"] = {
            "call": "sgemm_ex(transA=0, transB=1)", "us_per_call": round(tus, 3),
            "GB/s": round(tbps, 1), "frac": round(tbps / acc.PEAK_HBM_GBPS, 4),
            "traffic": stored_traffic("gemv_nt_m1_4096", GEMV_SOURCES)}

        # the other decode batch sizes of the workload, both weight layouts,
        # the same rotating weight copies
        def timed_calls(fn):
            for i in range(32):
                fn(i)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(args.gemv_steps):
                fn(i)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / args.gemv_steps * 1e3

        dWk = [dWt[0].t().contiguous()]
        for _ in range(nbuf - 1):
            dWk.append(dWk[0].clone())
        batch_rows = []
        for name in ("decode_m4_4096", "decode_m8_4096"):
            bw = inputs.WORKLOADS[name]
            bX = torch.from_numpy(inputs.make(bw)[0]).to(dev)
            bY = torch.zeros((bw.M, bw.N), dtype=torch.float32, device=dev)
            nn_us = timed_calls(lambda i: check(fg.sgemv(
                bw.M, bw.N, bw.K, bw.alpha, bX, bw.K, dWk[i % nbuf], bw.N, bw.beta, bY, bw.N, sp)))
            nt_us = timed_calls(lambda i: check(fg.sgemm_ex(
                0, 1, bw.M, bw.N, bw.K, bw.alpha, bX, bw.K, dWt[i % nbuf], bw.K, bw.beta, bY, bw.N,
                sp)))
            bbytes = acc.algorithmic_bytes(bw.M, bw.N, bw.K, bw.beta)
            batch_rows.append({
                "workload": name, "M": bw.M,
                "weight_stored_KxN": {"us_per_call": round(nn_us, 3),
                                      "GB/s": round(bbytes / (nn_us * 1e-6) / 1e9, 1)},
                "weight_stored_NxK": {"us_per_call": round(nt_us, 3),
                                      "GB/s": round(bbytes / (nt_us * 1e-6) / 1e9, 1)}})
        gemv["decode_batch"] = batch_rows
        del dWt, dWk

    # ---------------- CPU oracle on a bounded sample ----------------
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        cores = oracle.threads()
        r0 = 16
        t0 = time.perf_counter()
        oracle.sgemm(A[:r0], B, None, 1.0, 0.0)
        t_cal = time.perf_counter() - t0
        rows = int(min(M, max(r0, r0 * args.cpu_seconds / max(t_cal, 1e-6))))
        # whole passes until the target CPU time is reached (the full product
        # can take less than the target)
        passes, t = 0, 0.0
        while passes == 0 or (t < args.cpu_seconds and passes < 20):
            t0 = time.perf_counter()
            oracle.sgemm(A[:rows], B, None, 1.0, 0.0)
            t += time.perf_counter() - t0
            passes += 1
        cpu = {"value": round(passes * acc.flops(rows, N, K) / t / 1e12, 6), "unit": "TFLOP/s",
               "cores": cores, "kind": "oracle",
               "sample": f"first {rows} of {M} rows of the 4092^3 product (fp64 triple loop), "
                         f"{passes} pass(es), {t:.2f} s"}

    traffic = stored_traffic("sgemm_4092", KERNEL_SOURCES)
    out = {
        "metric": "SGEMM TFLOPS (% FP32 peak) at 4092³; GEMV HBM GB/s at M=1, K=N=4096",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "sgemm_4092_uniform", "M": M, "N": N, "K": K,
                   "alpha": w.alpha, "beta": w.beta, "inputs": "U[-1,1) fp32, seed 102",
                   "kernel_config": cfg_name},
        "pct_fp32_peak": round(100.0 * tflops / acc.PEAK_FP32_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": acc.PEAK_FP32_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / acc.PEAK_FP32_TFLOPS, 4),
                     "traffic": traffic},
        "gemv": gemv,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    if calib:
        out["calibration_copy"] = calib
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
