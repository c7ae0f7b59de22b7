"""Build libfp32gemm.so (HIP, gfx950) in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 instructions
disabled, then linked into one shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libfp32gemm.so")
# the measurement probes (HBM streaming, matrix-core issue), one library each
PROBES = {"hbm_probe.hip": os.path.join(HERE, "libhbmprobe.so"),
          "mfma_probe.hip": os.path.join(HERE, "libmfmaprobe.so")}
SOURCES = ["api.hip", "dispatch.hip", "sgemm_configs.hip", "sgemm_nn.hip", "sgemm_nt.hip",
           "sgemm_tn.hip", "sgemm_tt.hip", "sgemv.hip", "gemv_split.hip", "skinny.hip",
           "splitk.hip", "streamk.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is harmless
    noise = [ln for ln in (r.stderr or "").splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(noise))
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def build(jobs: int = 8) -> str:
    os.makedirs(OBJ, exist_ok=True)
    probes = list(PROBES)
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(SOURCES) + len(probes))) as ex:
        objs = list(ex.map(_compile, SOURCES + probes))
    for src, obj in zip(probes, objs[len(SOURCES):]):
        _link([obj], PROBES[src])
    return _link(objs[:len(SOURCES)], LIB)


if __name__ == "__main__":
    print(build())
