#!/usr/bin/env python3
"""Benchmark: fp32 SGEMM at 4092^3 and the decode GEMV on one MI355X.

One step is one full sgemm() call on the 4092 x 4092 x 4092 workload
(alpha = 1, beta = 0, A, B ~ U[-1, 1)), the square fp32 product the worklog
benchmarks ("CUDA 矩阵乘法优化：从朴素 Kernel 到接近 cuBLAS", table at the top
of the page).  Inputs are resident in HBM before timing starts; W steps are
warm-up, then K steps are timed with HIP events on the stream the kernels run
on, bracketed by device synchronisations.

The same run measures the other workloads, each with a parity check of its
own output against the CPU oracle, under the key "configs":
  * 128^3 (alpha 1, beta 0.5): microseconds per call, launch-bound;
  * 4096^3 (alpha 0.5, beta 1) and the prefill product 2048 x 11008 x 4096
    (two launches, timed as one step): TFLOP/s and fraction of the fp32
    matrix peak;
  * the decode products M = 1, 4, 8 against a 4096 x 4096 weight, stored
    K x N (sgemv) and N x K (sgemm_ex with op(B) = B^T): GB/s and fraction of
    the HBM peak, each call cycling over enough weight copies that the
    weights stream from HBM rather than from the 256 MB Infinity Cache.
They run before the 4092^3 steps, so the graphics clock has left its idle
level (the first ~30 large dispatches after the GPU wakes run slower) by the
time the headline steps are timed.  The graphics clock is sampled during
every timed loop ("clocks").

Prints one JSON line.  Extra keys: "roofline" (headline kernel against the
fp32 matrix peak), "gemv" (the M = 1 decode GEMV against the HBM peak),
"configs" (every workload), "clocks", "cpu_baseline" (the CPU oracle timed on
the same host: a bounded sample of the headline workload, plus one pass of
each other workload), "parity" (sampled rows and columns of the headline
output against the oracle).
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
                for f in ("sgemv.hip", "gemv_split.hip", "common.h", "tune_table.inc")]
# the prefill product's two launches are planned in dispatch.hip
PREFILL_SOURCES = KERNEL_SOURCES + [os.path.join(ROOT, "fp32_gemm_06_amd", "csrc",
                                                 "dispatch.hip")]

# weight copies the decode calls cycle over: 8 x 67 MB exceeds the 256 MB
# Infinity Cache, so every call reads its weight from HBM
GEMV_WEIGHT_COPIES = 8


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
    p.add_argument("--small-steps", type=int, default=2000, help="timed calls of the 128^3 product")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample of the headline workload "
                        "(0 disables the CPU baseline)")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="also run a plain device copy of this size (counter calibration)")
    p.add_argument("--skip-gemv", action="store_true")
    p.add_argument("--only", default="",
                   help="comma-separated workloads to run (profiling runs); default all")
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
    from fp32_gemm_06_amd.clocks import ClockSampler

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fg.lib()  # fail loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    only = set(filter(None, args.only.split(",")))

    def wanted(name):
        return not only or name in only

    props = torch.cuda.get_device_properties(0)
    clocks = ClockSampler(props.pci_domain_id, props.pci_bus_id, props.pci_device_id).start()

    def check(rc):
        if rc != 0:
            raise fg.Fp32GemmError(rc)

    def timed(fn, warmup, steps, phase):
        """Average milliseconds per call of fn(i) over `steps` calls after
        `warmup` untimed ones, from HIP events on the library's stream."""
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        clocks.phase(phase)
        e0.record(stream)
        for i in range(steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        clocks.phase(None)
        return e0.elapsed_time(e1) / steps

    def sampled_parity(name, got, A, B, C0, alpha, beta, rows=None, cols=None):
        """got (host, fp32 M x N) against the oracle on whole rows and columns:
        the first two, the middle one and the last two of each."""
        import oracle
        M, N = got.shape
        rows = sorted({0, 1, M // 2, M - 2, M - 1}) if rows is None else rows
        cols = sorted({0, 1, N // 2, N - 2, N - 1}) if cols is None else cols
        rr = np.concatenate([np.repeat(rows, N), np.tile(np.arange(M), len(cols))]).astype(np.int32)
        cc = np.concatenate([np.tile(np.arange(N), len(rows)), np.repeat(cols, M)]).astype(np.int32)
        ref = oracle.sgemm_entries(rr, cc, A, B, C0, alpha, beta)
        bnd = oracle.bound_entries(rr, cc, A, B, C0, alpha, beta)
        ok, worst = oracle.within_tolerance(got[rr, cc].astype(np.float64), ref, bnd)
        return {"rows": [int(r) for r in rows], "cols": [int(c) for c in cols],
                "elements": int(rr.size), "ok": bool(ok), "worst_err_over_tol": worst}

    def full_parity(got, A, B, C0, alpha, beta):
        import oracle
        ref = oracle.sgemm(A, B, C0, alpha, beta)
        bnd = oracle.bound(A, B, C0, alpha, beta)
        ok, worst = oracle.within_tolerance(got.astype(np.float64), ref, bnd)
        return {"elements": int(got.size), "ok": bool(ok), "worst_err_over_tol": worst}

    def guarded(fn):
        try:
            return fn()
        except Exception as e:  # the numbers are still reported; the failure is visible
            return {"error": repr(e)}

    def upload(w):
        A, B, C0 = inputs.make(w)
        return (A, B, C0, torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev),
                torch.from_numpy(C0).to(dev))

    def mfma_entry(w, ms, extra=None):
        flop = acc.flops(w.M, w.N, w.K)
        tf = flop / (ms * 1e-3) / 1e12
        e = {"M": w.M, "N": w.N, "K": w.K, "alpha": w.alpha, "beta": w.beta,
             "ms_per_call": round(ms, 5), "TFLOP/s": round(tf, 3),
             "roofline": {"bound": "mfma", "achieved": round(tf, 3),
                          "peak": acc.PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(tf / acc.PEAK_FP32_TFLOPS, 4),
                          "flop_per_call": flop,
                          "algorithmic_bytes": acc.algorithmic_bytes(w.M, w.N, w.K, w.beta)}}
        if extra:
            e.update(extra)
        return e

    configs = {}

    # ---------------- 128^3, alpha 1, beta 0.5: launch-bound ----------------
    if wanted("sgemm_128_uniform"):
        w = inputs.WORKLOADS["sgemm_128_uniform"]
        A, B, C0, dA, dB, dC = upload(w)
        check(fg.sgemm(w.M, w.N, w.K, w.alpha, dA, w.K, dB, w.N, w.beta, dC, w.N, sp))
        torch.cuda.synchronize()
        par = guarded(lambda: full_parity(dC.cpu().numpy(), A, B, C0, w.alpha, w.beta))
        ms = timed(lambda i: check(fg.sgemm(w.M, w.N, w.K, w.alpha, dA, w.K, dB, w.N, w.beta, dC,
                                            w.N, sp)), 200, args.small_steps, w.name)

        def graph_rate(calls=100, replays=20):
            """Microseconds per call with the host out of the loop: `calls`
            sgemm calls captured in one HIP graph, replayed `replays` times."""
            def burst(n):
                for _ in range(n):
                    check(fg.sgemm(w.M, w.N, w.K, w.alpha, dA, w.K, dB, w.N, w.beta, dC, w.N,
                                   None))
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                burst(3)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                burst(calls)
            for _ in range(3):
                graph.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(replays):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            return round(e0.elapsed_time(e1) / (replays * calls) * 1e3, 3)

        graph_us = guarded(graph_rate)
        configs[w.name] = {"M": w.M, "N": w.N, "K": w.K, "alpha": w.alpha, "beta": w.beta,
                           "us_per_call": round(ms * 1e3, 3), "bound": "overhead",
                           "note": "back-to-back calls on one stream: launch rate, not the "
                                   "kernel's own duration",
                           "us_per_call_graph": graph_us,
                           "graph_note": "100 calls captured in one HIP graph and replayed: the "
                                         "GPU's rate per call without the host's launch work",
                           "kernel_config": fg.fp32gemm_config_name(
                               fg.KIND_SGEMM, fg.fp32gemm_select_config(fg.KIND_SGEMM, w.M, w.N,
                                                                        w.K)),
                           "parity": par}
        del dA, dB, dC

    # ---------------- decode products, M = 1, 4, 8 ----------------
    gemv = None
    if not args.skip_gemv and any(wanted(f"decode_m{m}_4096") for m in (1, 4, 8)):
        nbuf = GEMV_WEIGHT_COPIES
        W = inputs.make("decode_m1_4096")[1]  # the weight (same draw order for every M)
        dWk = [torch.from_numpy(W).to(dev)]
        for _ in range(nbuf - 1):
            dWk.append(dWk[0].clone())
        dWt = [dWk[0].t().contiguous()]
        for _ in range(nbuf - 1):
            dWt.append(dWt[0].clone())
        for m in (1, 4, 8):
            name = f"decode_m{m}_4096"
            if not wanted(name):
                continue
            gw = inputs.WORKLOADS[name]
            X, Wm, Y0 = inputs.make(gw)
            dX = torch.from_numpy(X).to(dev)
            dY = torch.zeros((gw.M, gw.N), dtype=torch.float32, device=dev)
            # each M's weight is its own draw; time on the M = 1 weight copies
            # (same shape and distribution) and check parity on its own
            dWown = torch.from_numpy(Wm).to(dev)
            check(fg.sgemv(gw.M, gw.N, gw.K, gw.alpha, dX, gw.K, dWown, gw.N, gw.beta, dY, gw.N,
                           sp))
            torch.cuda.synchronize()
            par_kn = guarded(lambda: full_parity(dY.cpu().numpy(), X, Wm, Y0, gw.alpha, gw.beta))
            dWown_t = dWown.t().contiguous()
            dY.zero_()
            check(fg.sgemm_ex(0, 1, gw.M, gw.N, gw.K, gw.alpha, dX, gw.K, dWown_t, gw.K, gw.beta,
                              dY, gw.N, sp))
            torch.cuda.synchronize()
            par_nk = guarded(lambda: full_parity(dY.cpu().numpy(), X, Wm, Y0, gw.alpha, gw.beta))
            del dWown, dWown_t
            kn_ms = timed(lambda i: check(fg.sgemv(gw.M, gw.N, gw.K, gw.alpha, dX, gw.K,
                                                   dWk[i % nbuf], gw.N, gw.beta, dY, gw.N, sp)),
                          32, args.gemv_steps, f"{name}_KxN")
            nk_ms = timed(lambda i: check(fg.sgemm_ex(0, 1, gw.M, gw.N, gw.K, gw.alpha, dX, gw.K,
                                                      dWt[i % nbuf], gw.K, gw.beta, dY, gw.N,
                                                      sp)),
                          32, args.gemv_steps, f"{name}_NxK")
            warm_ms = timed(lambda i: check(fg.sgemv(gw.M, gw.N, gw.K, gw.alpha, dX, gw.K,
                                                     dWk[0], gw.N, gw.beta, dY, gw.N, sp)),
                            32, args.gemv_steps, f"{name}_KxN_warm")
            gbytes = acc.algorithmic_bytes(gw.M, gw.N, gw.K, gw.beta)

            def bw(ms):
                g = gbytes / (ms * 1e-3) / 1e9
                return {"us_per_call": round(ms * 1e3, 3), "GB/s": round(g, 1),
                        "frac": round(g / acc.PEAK_HBM_GBPS, 4)}

            gcfg = fg.fp32gemm_select_config(fg.KIND_SGEMV, gw.M, gw.N, gw.K)
            configs[name] = {
                "M": gw.M, "N": gw.N, "K": gw.K, "algorithmic_bytes": gbytes,
                "weight_copies": nbuf, "calls": args.gemv_steps,
                "weight_stored_KxN": dict(bw(kn_ms), call="sgemv",
                                          kernel_config=fg.fp32gemm_config_name(fg.KIND_SGEMV,
                                                                                gcfg),
                                          traffic=stored_traffic(f"gemv_m{m}_4096",
                                                                 GEMV_SOURCES),
                                          parity=par_kn),
                "weight_stored_NxK": dict(bw(nk_ms), call="sgemm_ex(transA=0, transB=1)",
                                          parity=par_nk),
                "warm_single_buffer_KxN": bw(warm_ms),
            }
            del dX, dY
            if m == 1:
                kn = configs[name]["weight_stored_KxN"]
                nk = configs[name]["weight_stored_NxK"]
                gemv = {
                    "metric": "GEMV HBM GB/s at M=1, K=N=4096",
                    "value": kn["GB/s"], "unit": "GB/s", "us_per_call": kn["us_per_call"],
                    "calls": args.gemv_steps, "weight_buffers": nbuf,
                    "config": kn["kernel_config"],
                    "roofline": {"bound": "hbm", "achieved": kn["GB/s"],
                                 "peak": acc.PEAK_HBM_GBPS, "unit": "GB/s", "frac": kn["frac"],
                                 "traffic": stored_traffic("gemv_m1_4096", GEMV_SOURCES)},
                    "warm_single_buffer": configs[name]["warm_single_buffer_KxN"],
                    "weight_stored_transposed": dict(
                        nk, traffic=stored_traffic("gemv_nt_m1_4096", GEMV_SOURCES)),
                }
        del dWk, dWt

    # ---------------- 4096^3 (alpha 0.5, beta 1) and the prefill product ----------------
    big_warmup = max(args.warmup, 30)
    for name, traffic_tag, srcs in (("sgemm_4096_normal", "sgemm_4096", KERNEL_SOURCES),
                                    ("prefill_2048x4096x11008", "prefill_2048x4096x11008",
                                     PREFILL_SOURCES)):
        if not wanted(name):
            continue
        w = inputs.WORKLOADS[name]
        A, B, C0, dA, dB, dC = upload(w)
        # parity of one call from the seeded C0, then the timed calls (with
        # beta = 1 they keep accumulating into C, which changes no timing)
        check(fg.sgemm(w.M, w.N, w.K, w.alpha, dA, w.K, dB, w.N, w.beta, dC, w.N, sp))
        torch.cuda.synchronize()
        par = guarded(lambda: sampled_parity(name, dC.cpu().numpy(), A, B, C0, w.alpha, w.beta))
        ms = timed(lambda i: check(fg.sgemm(w.M, w.N, w.K, w.alpha, dA, w.K, dB, w.N, w.beta, dC,
                                            w.N, sp)), big_warmup, args.steps, name)
        dim, first = fg.fp32gemm_round_split(w.M, w.N, w.K)
        extra = {"warmup": big_warmup, "steps": args.steps, "parity": par,
                 "launches_per_call": 2 if dim else 1,
                 "kernel_config": fg.fp32gemm_config_name(
                     fg.KIND_SGEMM, fg.fp32gemm_select_config(fg.KIND_SGEMM, w.M, w.N, w.K))}
        if dim:
            extra["round_split"] = {"dim": "columns" if dim == 1 else "rows", "first": first}
        configs[name] = mfma_entry(w, ms, extra)
        configs[name]["roofline"]["traffic"] = stored_traffic(traffic_tag, srcs)
        del dA, dB, dC

    # ---------------- headline: 4092^3, alpha 1, beta 0 ----------------
    w = inputs.WORKLOADS["sgemm_4092_uniform"]
    M, N, K = w.M, w.N, w.K
    cfg_name = fg.fp32gemm_config_name(fg.KIND_SGEMM, fg.fp32gemm_select_config(fg.KIND_SGEMM,
                                                                                M, N, K))
    A = B = None
    ms = tflops = parity = None
    if wanted(w.name):
        A, B, C0, dA, dB, dC = upload(w)
        ms = timed(lambda i: check(fg.sgemm(M, N, K, w.alpha, dA, K, dB, N, w.beta, dC, N, sp)),
                   args.warmup, args.steps, w.name)
        flop = acc.flops(M, N, K)
        tflops = flop / (ms * 1e-3) / 1e12
        parity = guarded(lambda: sampled_parity(w.name, dC.cpu().numpy(), A, B, C0, w.alpha,
                                                w.beta, rows=[0, 1, 2047, M - 2, M - 1],
                                                cols=[0, 1, 2047, N - 2, N - 1]))
        configs[w.name] = mfma_entry(w, ms, {"warmup": args.warmup, "steps": args.steps,
                                             "parity": parity, "kernel_config": cfg_name})
        del dA, dB, dC

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
    clocks.stop()
    clk = clocks.summary()

    # ---------------- CPU oracle on the same host ----------------
    cpu = None
    if args.cpu_seconds > 0 and A is not None:
        cpu = guarded(lambda: cpu_baseline(args, A, B, w))

    traffic = stored_traffic("sgemm_4092", KERNEL_SOURCES)
    out = {
        "metric": "SGEMM TFLOPS (% FP32 peak) at 4092³; GEMV HBM GB/s at M=1, K=N=4096",
        "value": None if tflops is None else round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": None if ms is None else round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "sgemm_4092_uniform", "M": M, "N": N, "K": K,
                   "alpha": w.alpha, "beta": w.beta, "inputs": "U[-1,1) fp32, seed 102",
                   "kernel_config": cfg_name},
        "pct_fp32_peak": None if tflops is None else round(100.0 * tflops / acc.PEAK_FP32_TFLOPS,
                                                            2),
        "roofline": None if tflops is None else {
            "bound": "mfma", "achieved": round(tflops, 3), "peak": acc.PEAK_FP32_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tflops / acc.PEAK_FP32_TFLOPS, 4),
            "traffic": traffic},
        "gemv": gemv,
        "configs": configs,
        "clocks": clk,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    hc = clk.get(w.name) if isinstance(clk, dict) else None
    if hc and tflops is not None:
        # the matrix peak at the clock the headline steps actually ran at
        peak_at = acc.CUS * 256 * hc["median_mhz"] * 1e6 / 1e12
        out["pct_fp32_peak_at_measured_sclk"] = round(100.0 * tflops / peak_at, 2)
    if calib:
        out["calibration_copy"] = calib
    print(json.dumps(out), flush=True)


def cpu_baseline(args, A, B, w):
    """The oracle as it stands, on this host's cores: whole passes of a row
    sample of the headline product up to about args.cpu_seconds, then one
    pass of every other workload, and the 128^3 product on one core too."""
    import oracle
    from fp32_gemm_06_amd import accounting as acc
    from fp32_gemm_06_amd import inputs
    from fp32_gemm_06_amd.clocks import cpu_model

    cores = oracle.threads()
    M, N, K = w.M, w.N, w.K
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

    def one_pass(name):
        x = inputs.WORKLOADS[name]
        Ax, Bx, Cx = inputs.make(x)
        t0 = time.perf_counter()
        oracle.sgemm(Ax, Bx, Cx, x.alpha, x.beta)
        dt = time.perf_counter() - t0
        return {"seconds": round(dt, 4), "GFLOP/s": round(acc.flops(x.M, x.N, x.K) / dt / 1e9, 3)}

    per = {}
    for name in ("sgemm_128_uniform", "sgemm_4096_normal", "prefill_2048x4096x11008",
                 "decode_m1_4096", "decode_m4_4096", "decode_m8_4096"):
        per[name] = dict(one_pass(name), cores=cores)
    oracle.set_threads(1)
    try:
        per["sgemm_128_uniform_one_core"] = dict(one_pass("sgemm_128_uniform"), cores=1)
    finally:
        oracle.set_threads(cores)
    return {"value": round(passes * acc.flops(rows, N, K) / t / 1e12, 6), "unit": "TFLOP/s",
            "cores": cores, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"first {rows} of {M} rows of the 4092^3 product (fp64 triple loop), "
                      f"{passes} pass(es), {t:.2f} s",
            "per_config_one_pass": per}


if __name__ == "__main__":
    main()
