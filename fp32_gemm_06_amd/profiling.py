"""Summaries of rocprofv3 output for the profiles/ folder.

    python -m fp32_gemm_06_amd.profiling <run dir> <out prefix> "<command that made it>"

<run dir> holds the CSV output of one kernel-trace run (trace/) and of
counter runs (pmc*/), each made with ``--output-format csv``.  Writes
<out prefix>_<kernel>.md summaries and, for the SGEMM and the two GEMV kernels,
<out prefix>_<kernel>_traffic.json with HBM bytes per launch.

    python -m fp32_gemm_06_amd.profiling --trace-table <run dir> <out.md> "<command>"

writes one table of this library's launches in a kernel-trace run, by kernel
and launch shape (calls, mean and min duration).

    python -m fp32_gemm_06_amd.profiling --pmc-table <run dir> <out.md> "<command>"

writes the same table for counter runs (pmc*/ under <run dir>): the mean of
each counter per dispatch by kernel and launch shape, and the L2 hit rate
when TCC_HIT_sum and TCC_MISS_sum were collected.

    python -m fp32_gemm_06_amd.profiling --workload <run dir> <tag> <kernel needle>
        <skip> <count> <per step> <source files> <out dir> "<command>"

summarizes one workload's timed calls from a run that launched only that
workload (``bench.py --only <workload>``): see ``summarize_workload``.

HBM bytes come from FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each
scaled by what the same counter reads for a calibration kernel of known
size in the same run (an elementwise negation that reads and writes
``bytes_each_way``): scale = known bytes / counted bytes.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp32_gemm_06_amd", "csrc")
KERNELS = {
    "sgemm_4092": ("sgemm_kernel", ["sgemm_kernel.h", "sgemm_nn.hip", "common.h", "tune_table.inc"]),
    "gemv_m1_4096": ("sgemv_kernel<1,", ["sgemv.hip", "common.h", "tune_table.inc"]),
    "gemv_nt_m1_4096": ("sgemv_rows_kernel<1,", ["sgemv.hip", "common.h", "tune_table.inc"]),
}
CALIB = "neg_kernel"
CALIB_BYTES = 256 << 20


def code_text(path):
    """A source file without its comments and blank lines: what the compiler
    sees, so that editing a comment does not invalidate recorded counters."""
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())


def source_hash(files):
    """Hash of the code (comments excluded) of the named csrc files, or of
    the given paths when they are absolute."""
    h = hashlib.sha256()
    for f in files:
        h.update(code_text(f if os.path.isabs(f) else os.path.join(CSRC, f)).encode())
    return h.hexdigest()[:16]


def kernel_stats(run_dir):
    out = {}
    for path in glob.glob(os.path.join(run_dir, "trace", "*kernel_stats.csv")):
        for r in csv.DictReader(open(path)):
            out[r["Name"]] = {"calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                              "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3}
    return out


def dispatch_durations(run_dir):
    """{kernel name: [duration us, in dispatch order]} from the kernel trace."""
    out = defaultdict(list)
    for path in glob.glob(os.path.join(run_dir, "trace", "*kernel_trace.csv")):
        rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
        for r in rows:
            out[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return out


def counters(run_dir):
    """{kernel name: {counter: [values per dispatch]}} over all pmc*/ runs."""
    agg = defaultdict(lambda: defaultdict(list))
    for path in glob.glob(os.path.join(run_dir, "pmc*", "*counter_collection.csv")):
        for r in csv.DictReader(open(path)):
            agg[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return agg


def _find(d, key):
    hits = [k for k in d if key in k.replace(" ", "")]
    return hits[0] if hits else None


def _avg(v):
    return sum(v) / len(v) if v else float("nan")


def summarize(run_dir, prefix, command, timed=(100, 400)):
    """timed: dispatches of the timed window per kernel (the last ones of the
    SGEMM / GEMV sequence of the run; earlier ones are warm-up)."""
    stats = kernel_stats(run_dir)
    durs = dispatch_durations(run_dir)
    ctr = counters(run_dir)
    calib = _find(ctr, CALIB)
    fetch_scale = write_scale = None
    if calib:
        c = ctr[calib]
        # the largest dispatches of the calibration kernel are the 256 MiB ones
        if c.get("FETCH_SIZE"):
            fetch_scale = CALIB_BYTES / (max(c["FETCH_SIZE"]) * 1024.0)
        if c.get("WRITE_SIZE"):
            write_scale = CALIB_BYTES / (max(c["WRITE_SIZE"]) * 1024.0)
    written = []
    for tag, (needle, files) in KERNELS.items():
        sk = _find(stats, needle.replace(" ", ""))
        ck = _find(ctr, needle.replace(" ", ""))
        if not sk:
            continue
        s = stats[sk]
        lines = [f"# {tag}: rocprofv3 summary", "", f"Kernel: `{sk}`", "",
                 "Command (from the repository root, on an MI355X):", "", "```", command, "```", "",
                 f"Kernel source hash: `{source_hash(files)}`", "",
                 "| quantity | value |", "|---|---|",
                 f"| dispatches traced | {s['calls']} |",
                 f"| average duration | {s['avg_us']:.3f} us |",
                 f"| min / max duration | {s['min_us']:.3f} / {s['max_us']:.3f} us |"]
        rec = {"kernel": sk, "source_hash": source_hash(files), "avg_us": s["avg_us"]}
        d = durs.get(sk, [])
        want = timed[0] if tag.startswith("sgemm") else timed[1]
        if d:
            # the SGEMM's timed steps follow its warm-up; the GEMV's cycled calls
            # follow 32 warm-up calls and precede the single-buffer calls
            if tag.startswith("sgemm"):
                win = d[-want:]
            else:
                win = d[32:32 + want]
            rec["timed_avg_us"] = sum(win) / len(win)
            lines.append(f"| average over the timed window ({len(win)} dispatches) | "
                         f"{rec['timed_avg_us']:.3f} us |")
        if ck:
            c = ctr[ck]
            for name in sorted(c):
                lines.append(f"| {name} (mean per dispatch) | {_avg(c[name]):.6g} |")
            if c.get("SQ_VALU_MFMA_BUSY_CYCLES") and c.get("GRBM_GUI_ACTIVE"):
                # busy cycles are summed over the 1024 SIMDs, GUI_ACTIVE over the 8 XCDs
                util = _avg(c["SQ_VALU_MFMA_BUSY_CYCLES"]) / 1024.0 / (_avg(c["GRBM_GUI_ACTIVE"]) / 8.0)
                lines.append(f"| MFMA busy fraction (busy per SIMD / active cycles per XCD) | {util:.4f} |")
                rec["mfma_busy_fraction"] = util
            if c.get("FETCH_SIZE") and fetch_scale:
                fb = _avg(c["FETCH_SIZE"]) * 1024.0 * fetch_scale
                lines.append(f"| HBM read bytes per launch (FETCH_SIZE x {fetch_scale:.4f}) | {fb:.6g} |")
                rec["fetch_bytes"] = fb
                rec["fetch_scale"] = fetch_scale
            if c.get("WRITE_SIZE") and write_scale:
                wb = _avg(c["WRITE_SIZE"]) * 1024.0 * write_scale
                lines.append(f"| HBM write bytes per launch (WRITE_SIZE x {write_scale:.4f}) | {wb:.6g} |")
                rec["write_bytes"] = wb
                rec["write_scale"] = write_scale
            if "fetch_bytes" in rec and "write_bytes" in rec:
                rec["bytes_per_launch"] = rec["fetch_bytes"] + rec["write_bytes"]
        if calib:
            lines += ["", f"Calibration kernel `{calib[:60]}...` moves {CALIB_BYTES} bytes each way; "
                          "counter scale = known bytes / counted bytes."]
        md = f"{prefix}_{tag}.md"
        with open(md, "w") as f:
            f.write("\n".join(lines) + "\n")
        written.append(md)
        if "bytes_per_launch" in rec:
            js = os.path.join(os.path.dirname(prefix), f"{tag}_traffic.json")
            with open(js, "w") as f:
                json.dump(rec, f, indent=1)
            written.append(js)
    return written


def summarize_workload(run_dir, tag, needle, skip, count, per_step, sources, out_dir, command):
    """Summary of one workload's timed calls in a run that launched only that
    workload's products (``bench.py --only``).

    The dispatches whose kernel name contains ``needle`` are taken in launch
    order; the timed window is ``count`` of them after the first ``skip``
    (parity call and warm-up).  A call of the workload is ``per_step``
    consecutive dispatches (two for a product that runs as two launches), and
    its duration is their sum.  Counters from the pmc*/ runs are averaged per
    kernel over all its dispatches and summed over the kernels of one call.
    Writes ``rocprof_<tag>.md`` and, when both byte counters and the
    calibration kernel are present, ``<tag>_traffic.json``.
    """
    hits = sorted(glob.glob(os.path.join(run_dir, "trace", "*kernel_trace.csv")))
    if not hits:
        raise FileNotFoundError(f"no kernel_trace.csv under {run_dir}/trace")
    rows = []
    for path in hits:
        rows += [r for r in csv.DictReader(open(path)) if needle in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    win = rows[skip: skip + count]
    if len(win) < count or count % per_step:
        raise ValueError(f"{tag}: {len(rows)} dispatches of {needle!r}, window {skip}+{count} "
                         f"in calls of {per_step}")
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in win]
    calls = [sum(durs[i:i + per_step]) for i in range(0, len(durs), per_step)]
    names = []
    for r in win[:per_step]:
        if r["Kernel_Name"] not in names:
            names.append(r["Kernel_Name"])
    per_kernel = {}
    for k in names:
        d = [x for x, r in zip(durs, win) if r["Kernel_Name"] == k]
        grid = (int(win[[r["Kernel_Name"] for r in win].index(k)]["Grid_Size_X"]))
        per_kernel[k] = (sum(d) / len(d), grid)
    ctr = counters(run_dir)
    calib = _find(ctr, CALIB)
    scales = {}
    if calib:
        for cn in ("FETCH_SIZE", "WRITE_SIZE"):
            if ctr[calib].get(cn):
                scales[cn] = CALIB_BYTES / (max(ctr[calib][cn]) * 1024.0)
    summed = defaultdict(float)
    for k in names:
        for cn, vals in ctr.get(k, {}).items():
            summed[cn] += _avg(vals)
    h = source_hash(sources)
    avg_call = sum(calls) / len(calls)
    lines = [f"# {tag}: rocprofv3 summary", "",
             "Command (from the repository root, on an MI355X):", "", "```", command, "```", "",
             f"Kernel source hash: `{h}`", "",
             f"One call = {per_step} dispatch(es); timed window: {len(calls)} calls after "
             f"{skip} earlier dispatches (parity call and warm-up).", "",
             "| kernel | grid threads (x) | mean duration in the window |", "|---|---|---|"]
    for k in names:
        lines.append(f"| `{_short_kernel(k)}` | {per_kernel[k][1]} | {per_kernel[k][0]:.3f} us |")
    lines += ["", "| quantity | value |", "|---|---|",
              f"| calls in the window | {len(calls)} |",
              f"| mean duration per call (sum of its dispatches) | {avg_call:.3f} us |",
              f"| min / max per call | {min(calls):.3f} / {max(calls):.3f} us |"]
    rec = {"workload": tag, "kernels": names, "source_hash": h, "per_step": per_step,
           "timed_avg_us": avg_call}
    for cn in sorted(summed):
        lines.append(f"| {cn} (mean per call, summed over its kernels) | {summed[cn]:.6g} |")
    if summed.get("SQ_VALU_MFMA_BUSY_CYCLES") and summed.get("GRBM_GUI_ACTIVE"):
        util = summed["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024.0 / (summed["GRBM_GUI_ACTIVE"] / 8.0)
        lines.append(f"| MFMA busy fraction (busy per SIMD / active cycles per XCD) | {util:.4f} |")
        rec["mfma_busy_fraction"] = util
    for cn, key in (("FETCH_SIZE", "fetch_bytes"), ("WRITE_SIZE", "write_bytes")):
        if summed.get(cn) and cn in scales:
            b = summed[cn] * 1024.0 * scales[cn]
            lines.append(f"| HBM {'read' if cn == 'FETCH_SIZE' else 'write'} bytes per call "
                         f"({cn} x {scales[cn]:.4f}) | {b:.6g} |")
            rec[key] = b
            rec[key.replace("bytes", "scale")] = scales[cn]
    if "fetch_bytes" in rec and "write_bytes" in rec:
        rec["bytes_per_launch"] = rec["fetch_bytes"] + rec["write_bytes"]
    if calib:
        lines += ["", f"Calibration kernel `{_short_kernel(calib)[:60]}` moves {CALIB_BYTES} bytes "
                      "each way; counter scale = known bytes / counted bytes."]
    out = [os.path.join(out_dir, f"rocprof_{tag}.md")]
    with open(out[0], "w") as f:
        f.write("\n".join(lines) + "\n")
    if "bytes_per_launch" in rec:
        out.append(os.path.join(out_dir, f"{tag}_traffic.json"))
        with open(out[1], "w") as f:
            json.dump(rec, f, indent=1)
    return out


def _short_kernel(name):
    """This library's kernel name without namespaces and parameter list."""
    name = name.replace("void ", "", 1).replace("fp32gemm::(anonymous namespace)::", "")
    name = name.replace("fp32gemm::", "")
    depth = 0
    for i, ch in enumerate(name):
        depth += ch == "<"
        depth -= ch == ">"
        if ch == "(" and depth == 0:
            return name[:i]
    return name


def trace_table(run_dir, out_md, command):
    """Per-launch-shape durations of this library's kernels from a
    `rocprofv3 --kernel-trace` run: one row per (kernel, workgroups,
    workgroup size) with calls, mean and min duration."""
    hits = sorted(glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no kernel_trace.csv under {run_dir}")
    groups, other = {}, 0
    with open(hits[0], newline="") as f:
        for r in csv.DictReader(f):
            if "fp32gemm::" not in r["Kernel_Name"]:
                other += 1
                continue
            wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
            grid = (int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])),
                    int(r["Grid_Size_Y"]) // max(1, int(r["Workgroup_Size_Y"])))
            key = (_short_kernel(r["Kernel_Name"]), grid, wg)
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            groups.setdefault(key, []).append(d)
    lines = [f"# Kernel trace: {os.path.basename(out_md)[:-3]}", "",
             "Command (from the repository root, on an MI355X):", "", "```", command, "```", "",
             "One row per kernel and launch shape (workgroups x batch entries, threads per "
             "workgroup); durations in microseconds from the kernel trace. "
             f"{other} dispatches of other kernels (input generation, the vendor library) "
             "are not listed.", "",
             "| kernel | workgroups | threads | calls | mean us | min us |",
             "|---|---|---|---|---|---|"]
    for (k, grid, wg), v in sorted(groups.items()):
        lines.append(f"| `{k}` | {grid[0]} x {grid[1]} | {wg} | {len(v)} | "
                     f"{sum(v) / len(v):.1f} | {min(v):.1f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out_md


def pmc_table(run_dir, out_md, command):
    """Mean counter values per dispatch of this library's kernels, by kernel
    and workgroup count, from `rocprofv3 --pmc ... --output-format csv`
    runs under run_dir (every *counter_collection.csv below it)."""
    hits = sorted(glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    vals, names = {}, set()
    for path in hits:
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if "fp32gemm::" not in r["Kernel_Name"]:
                    continue
                groups = int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))
                key = (_short_kernel(r["Kernel_Name"]), groups, int(r["Workgroup_Size"]))
                d = vals.setdefault(key, {})
                d.setdefault(r["Counter_Name"], {})[r["Dispatch_Id"]] = float(r["Counter_Value"])
                names.add(r["Counter_Name"])
    names = sorted(names)
    hit = "TCC_HIT_sum" in names and "TCC_MISS_sum" in names
    lines = [f"# Counters: {os.path.basename(out_md)[:-3]}", "",
             "Command (from the repository root, on an MI355X):", "", "```", command, "```", "",
             "Mean per dispatch over every dispatch of the kernel with that workgroup count "
             "(threads per workgroup in brackets)." +
             (" L2 hit = TCC_HIT / (TCC_HIT + TCC_MISS)." if hit else ""), "",
             "| kernel | workgroups | dispatches | " + " | ".join(names) +
             (" | L2 hit |" if hit else " |"),
             "|---" * (3 + len(names) + hit) + "|"]
    for (k, groups, wg), d in sorted(vals.items()):
        n = max(len(v) for v in d.values())
        means = {c: _avg(list(d[c].values())) if c in d else float("nan") for c in names}
        row = f"| `{k}` | {groups} ({wg}) | {n} | " + " | ".join(f"{means[c]:.0f}" for c in names)
        if hit:
            h, m = means["TCC_HIT_sum"], means["TCC_MISS_sum"]
            row += f" | {h / (h + m):.3f}"
        lines.append(row + " |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out_md


if __name__ == "__main__":
    if sys.argv[1] == "--workload":
        # --workload <run dir> <tag> <kernel needle> <skip> <count> <per step>
        #            <source files, comma-separated> <out dir> "<command>"
        a = sys.argv[2:]
        for w in summarize_workload(a[0], a[1], a[2], int(a[3]), int(a[4]), int(a[5]),
                                    a[6].split(","), a[7], a[8]):
            print(w)
    elif sys.argv[1] == "--trace-table":
        print(trace_table(sys.argv[2], sys.argv[3], sys.argv[4]))
    elif sys.argv[1] == "--pmc-table":
        print(pmc_table(sys.argv[2], sys.argv[3], sys.argv[4]))
    else:
        for w in summarize(sys.argv[1], sys.argv[2], sys.argv[3]):
            print(w)
