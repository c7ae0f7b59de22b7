"""What the fp32 matrix cores deliver on this GPU, and the SGEMM against it.

    python -m fp32_gemm_06_amd.mfma_ceiling --md out.md

Times the matrix-core probe of libmfmaprobe.so (256 workgroups, one per CU,
each wave issuing independent MFMAs back to back with no memory access) for
both fp32 MFMA forms at one and two waves per SIMD, and reads the shader
clock under that load from the kernel itself (s_memtime cycles over
s_memrealtime ticks of each workgroup's loop), also per XCD (workgroup id
mod 8: the hardware deals workgroups to the 8 XCDs in turn).  Then times the
library's sgemm on the 4092^3 and 4096^3 workloads the same way (HIP events
over back-to-back calls after a warm-up).  Fractions are of the 157.3
TFLOP/s fp32 peak (256 CUs x 256 FLOP/clk x 2.4 GHz), of the best probe
rate, and of the peak at the slowest XCD's median clock (the probe's launch
ends with its slowest workgroups).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB = os.path.join(HERE, "libmfmaprobe.so")
FORMS = [(32, 4), (32, 8), (16, 4), (16, 8)]  # (MFMA form, waves per workgroup)
GROUPS = 256
FLOP_PER_ITER = 131072  # per wave, either form
PEAK = 157.3


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--md", default=None)
    ap.add_argument("--iters", type=int, default=2000, help="loop trips per wave (about 2 ms)")
    args = ap.parse_args()

    import torch

    import fp32_gemm_06_amd as fg
    from fp32_gemm_06_amd import inputs

    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is not built; run `python -m fp32_gemm_06_amd.build`")
    L = ctypes.CDLL(PROBE_LIB)
    L.mfma_issue_rate.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 3
    L.mfma_issue_rate.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream()
    sp = st.cuda_stream
    sink = torch.empty(GROUPS * 512, device=dev)
    clocks = torch.zeros(2 * GROUPS, dtype=torch.int64, device=dev)

    def timed(fn, warm, calls):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(calls):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / calls * 1e3

    big = torch.randn(4096, 4096, device=dev)  # bring the clock up
    for _ in range(60):
        torch.matmul(big, big)
    del big

    rows = []
    for mf, waves in FORMS:
        def call():
            rc = L.mfma_issue_rate(mf, GROUPS, waves, args.iters, sink.data_ptr(),
                                   clocks.data_ptr(), sp)
            if rc != 0:
                raise RuntimeError(f"mfma_issue_rate returned {rc}")
        us = timed(call, 3, 10)
        c = clocks.cpu().tolist()
        cyc, ticks = c[0::2], c[1::2]
        mhz = [cy / (t / 100.0) for cy, t in zip(cyc, ticks)]
        by_xcd = [statistics.median(mhz[x::8]) for x in range(8)]
        tflops = GROUPS * waves * FLOP_PER_ITER * args.iters / us / 1e6
        rows.append({"kind": "probe", "form": f"{mf}x{mf}x{2 if mf == 32 else 4}",
                     "waves_per_simd": waves // 4, "us": round(us, 1), "TFLOP/s": round(tflops, 2),
                     "clock_mhz": round(statistics.median(mhz), 1),
                     "clock_range": f"{min(mhz):.0f}-{max(mhz):.0f}",
                     "clock_by_xcd": [round(v) for v in by_xcd],
                     "of_peak_at_clock": round(tflops / (256 * 256 * min(by_xcd) / 1e6), 4)})
        print(json.dumps(rows[-1]), flush=True)

    for name in ("sgemm_4092_uniform", "sgemm_4096_normal"):
        w = inputs.WORKLOADS[name]
        A = torch.rand(w.M, w.K, device=dev) * 2 - 1
        B = torch.rand(w.K, w.N, device=dev) * 2 - 1
        C = torch.rand(w.M, w.N, device=dev) * 2 - 1

        def gemm():
            rc = fg.sgemm(w.M, w.N, w.K, w.alpha, A, w.K, B, w.N, w.beta, C, w.N, sp)
            if rc:
                raise fg.Fp32GemmError(rc)
        us = timed(gemm, 30, 50)
        rows.append({"kind": f"sgemm {w.M}x{w.N}x{w.K}", "form": "32x32x2",
                     "waves_per_simd": 2, "us": round(us, 1),
                     "TFLOP/s": round(2.0 * w.M * w.N * w.K / us / 1e6, 2)})
        print(json.dumps(rows[-1]), flush=True)
        del A, B, C

    if args.md:
        best = max(r["TFLOP/s"] for r in rows if r["kind"] == "probe")
        lines = ["# fp32 matrix-core ceiling (MI355X)", "",
                 "Command (repository root, on an MI355X):", "", "```",
                 f"python -m fp32_gemm_06_amd.mfma_ceiling --md {args.md}", "```", "",
                 __doc__.split("\n\n", 2)[2].strip(), "",
                 "| call | MFMA form | waves per SIMD | us per call | TFLOP/s | of 157.3 | "
                 "of best probe | shader clock MHz (median, range) | median clock per XCD 0-7 | "
                 "of peak at slowest XCD's clock |",
                 "|---|---|---|---|---|---|---|---|---|---|"]
        for r in rows:
            clk = f"{r['clock_mhz']} ({r['clock_range']})" if "clock_mhz" in r else ""
            xcd = " / ".join(str(v) for v in r["clock_by_xcd"]) if "clock_by_xcd" in r else ""
            lines.append(f"| {r['kind']} | {r['form']} | {r['waves_per_simd']} | {r['us']} | "
                         f"{r['TFLOP/s']} | {r['TFLOP/s'] / PEAK:.3f} | "
                         f"{r['TFLOP/s'] / best:.3f} | {clk} | {xcd} | "
                         f"{r.get('of_peak_at_clock', '')} |")
        with open(args.md, "w") as f:
            f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
