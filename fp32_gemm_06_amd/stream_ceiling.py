"""What one pass over a decode-sized weight can reach on this GPU.

    python -m fp32_gemm_06_amd.stream_ceiling --md out.md

Times the streaming probe of libhbmprobe.so (plain 128-bit reads of a
contiguous piece per workgroup, nothing else) on 4096 x 4096 fp32 =
67,108,864 bytes, cycling over 8 copies so that every call reads from HBM
rather than the 256 MB Infinity Cache, in the launch shapes the decode
kernels use; then the library's M = 1 decode calls on the same sizes and
buffers, the same way.  One more call of each probe shape records every
workgroup's start and end (s_memrealtime, 10 ns): the dispatch ramp (last
start - first start), the median workgroup duration and the end of the last
workgroup, all relative to the first start.  The event time per call also
includes the launch and completion of the kernel.  Fractions are of the
8 TB/s HBM peak.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB = os.path.join(HERE, "libhbmprobe.so")
SHAPES = [(256, 4), (256, 8), (512, 8), (1024, 4), (1024, 8)]  # (workgroups, waves)
COPIES = 8
PEAK = 8000.0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--md", default=None)
    ap.add_argument("--calls", type=int, default=400)
    args = ap.parse_args()

    import torch

    import fp32_gemm_06_amd as fg

    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is not built; run `python -m fp32_gemm_06_amd.build`")
    L = ctypes.CDLL(PROBE_LIB)
    L.hbm_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.hbm_stream_read.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream()
    sp = st.cuda_stream
    N = K = 4096
    n = N * K
    bufs = [torch.randn(K, N, device=dev) for _ in range(COPIES)]
    sink = torch.empty(1024 * 512, device=dev)
    stamps = torch.zeros(2 * 1024, dtype=torch.int64, device=dev)

    def timed(fn):
        for i in range(32):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for i in range(args.calls):
            fn(i)
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.calls * 1e3

    rows = []
    for groups, waves in SHAPES:
        def call(i, tsp=None):
            rc = L.hbm_stream_read(bufs[i % COPIES].data_ptr(), n, groups, waves, sink.data_ptr(),
                                   tsp, sp)
            if rc != 0:
                raise RuntimeError(f"hbm_stream_read returned {rc}")
        us = timed(call)
        call(3, stamps.data_ptr())
        torch.cuda.synchronize()
        t = stamps[:2 * groups].cpu().tolist()
        starts, ends = t[0::2], t[1::2]
        t0 = min(starts)
        rows.append({"kind": "probe", "workgroups": groups, "threads": waves * 64,
                     "us_per_call": round(us, 3), "GB/s": round(n * 4 / us / 1e3, 1),
                     "ramp_us": round((max(starts) - t0) / 100.0, 2),
                     "median_wg_us": round(statistics.median(e - s for s, e in zip(starts, ends))
                                           / 100.0, 2),
                     "last_end_us": round((max(ends) - t0) / 100.0, 2)})
        print(json.dumps(rows[-1]), flush=True)

    # the library's M = 1 decode on the same sizes, the same way
    x = torch.randn(1, K, device=dev)
    y = torch.zeros(1, N, device=dev)

    def kn(i):
        rc = fg.sgemv(1, N, K, 1.0, x, K, bufs[i % COPIES], N, 0.0, y, N, sp)
        if rc:
            raise fg.Fp32GemmError(rc)

    def nk(i):  # the same buffers read as W stored N x K
        rc = fg.sgemm_ex(0, 1, 1, N, K, 1.0, x, K, bufs[i % COPIES], K, 0.0, y, N, sp)
        if rc:
            raise fg.Fp32GemmError(rc)

    nbytes = 4 * (K * N + K + N)
    for name, fn, cfg in (("sgemv (W stored K x N)", kn,
                           fg.fp32gemm_config_name(1, fg.fp32gemm_select_config(1, 1, N, K))),
                          ("sgemm_ex(N, T) (W stored N x K)", nk, "row-dot")):
        us = timed(fn)
        rows.append({"kind": name, "config": cfg, "us_per_call": round(us, 3),
                     "GB/s": round(nbytes / us / 1e3, 1)})
        print(json.dumps(rows[-1]), flush=True)

    if args.md:
        best = max(r["GB/s"] for r in rows if r["kind"] == "probe")
        lines = ["# HBM streaming ceiling for one decode-sized pass (MI355X)", "",
                 "Command (repository root, on an MI355X):", "", "```",
                 f"python -m fp32_gemm_06_amd.stream_ceiling --md {args.md}", "```", "",
                 __doc__.split("\n\n", 2)[2].strip(), "",
                 "| call | workgroups x threads | us per call | GB/s | of 8 TB/s | of best probe | "
                 "ramp us | median workgroup us | last end us |",
                 "|---|---|---|---|---|---|---|---|---|"]
        for r in rows:
            shape = (f"{r['workgroups']} x {r['threads']}" if r["kind"] == "probe"
                     else r["config"])
            lines.append(f"| {r['kind']} | {shape} | {r['us_per_call']} | {r['GB/s']} | "
                         f"{r['GB/s'] / PEAK:.3f} | {r['GB/s'] / best:.3f} | "
                         f"{r.get('ramp_us', '')} | {r.get('median_wg_us', '')} | "
                         f"{r.get('last_end_us', '')} |")
        with open(args.md, "w") as f:
            f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
