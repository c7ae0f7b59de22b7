"""CPU oracle for C = alpha * A.B + beta * C0 (fp32 inputs, fp64 result).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  It shares no code
with the HIP library ``fp32_gemm_06_amd`` and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, OpenMP over rows); this module
only marshals numpy arrays into it.  The definition it follows is the one on
the page "GPU GEMM 优化完全拆解（一）：从朴素 Kernel 到共享内存分块",
section "什么是 GEMM", and the naive kernel of "CUDA 矩阵乘法优化：从朴素
Kernel 到接近 cuBLAS", section "1. Kernel 1: 朴素实现": element (i, j) is
alpha times the inner product of row i of A with column j of B, plus beta
times the old C.  See ``oracle.c`` for the readings taken where the pages are
silent (leading dimensions, beta == 0 / alpha == 0, rounding).

The fused variants (``sgemm_fused`` and friends) add a per-column bias and
an optional ReLU after the update: the operator-fusion example of "GPU 基础
原理", section "4.1 算子融合" (y = relu(x + 1)), applied to a GEMM output.

Every function here is pinned by ``tests/test_oracle.py`` against exact
rational arithmetic on tiny inputs, closed forms (identity and all-ones
operands), exact integer products, linearity in alpha/beta and the
transpose identity.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_F32P = ctypes.POINTER(ctypes.c_float)
_F64P = ctypes.POINTER(ctypes.c_double)
_I32P = ctypes.POINTER(ctypes.c_int)


def build(path: str = _LIB_PATH, mutant: int = 0) -> str:
    """Compile oracle.c into a shared library (host only, gcc + OpenMP)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall",
           f"-DORACLE_MUTANT={int(mutant)}", _SRC, "-o", path]
    subprocess.check_call(cmd)
    return path


def _bind(lib):
    i64 = ctypes.c_int64
    lib.oracle_sgemm.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                 _F32P, i64, _F32P, i64, ctypes.c_float, _F32P, i64, _F64P, i64]
    lib.oracle_bound.argtypes = lib.oracle_sgemm.argtypes
    lib.oracle_sgemm_entries.argtypes = [ctypes.c_int, _I32P, _I32P, ctypes.c_int, ctypes.c_float,
                                         _F32P, i64, _F32P, i64, ctypes.c_float, _F32P, i64, _F64P]
    lib.oracle_bound_entries.argtypes = lib.oracle_sgemm_entries.argtypes
    for f in (lib.oracle_sgemm, lib.oracle_bound, lib.oracle_sgemm_entries, lib.oracle_bound_entries):
        f.restype = None
    lib.oracle_epilogue.argtypes = [ctypes.c_int, _I32P, _I32P, _F32P, ctypes.c_int, _F64P,
                                    _F64P]
    lib.oracle_epilogue.restype = None
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = ctypes.c_int
    return lib


def load(path: str | None = None):
    """Load liboracle.so (building it first if it is absent)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _mat(x, rows: int, cols: int, name: str):
    """Check a row-major fp32 matrix view; return (base array, ld)."""
    if x is None:
        return None, max(1, cols)
    x = np.asarray(x)
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float32 array")
    if x.shape[0] < rows or x.shape[1] < cols:
        raise ValueError(f"{name} has shape {x.shape}, need at least {(rows, cols)}")
    if x.size == 0:
        return x, max(1, cols)
    if (x.shape[1] > 1 and x.strides[1] != 4) or x.strides[0] % 4 or x.strides[0] < 4 * cols:
        raise ValueError(f"{name} must be row-major with unit column stride")
    return x, max(1, x.strides[0] // 4)


def _ptr(x):
    if x is None:
        return ctypes.cast(None, _F32P)
    return x.ctypes.data_as(_F32P)


def sgemm(A, B, C0=None, alpha: float = 1.0, beta: float = 0.0, M=None, N=None, K=None,
          lib=None) -> np.ndarray:
    """Reference C = alpha * A[:M,:K] @ B[:K,:N] + beta * C0[:M,:N], returned as float64.

    A, B, C0 are 2-D row-major float32 arrays (row strides act as leading
    dimensions).  A/B may be None when alpha == 0 or K == 0; C0 may be None
    when beta == 0.
    """
    lib = lib or load()
    M = A.shape[0] if M is None else M
    K = A.shape[1] if K is None else K
    N = B.shape[1] if N is None else N
    A, lda = _mat(A, M, K, "A")
    B, ldb = _mat(B, K, N, "B")
    C0, ldc = _mat(C0, M, N, "C0")
    out = np.empty((M, N), dtype=np.float64)
    lib.oracle_sgemm(M, N, K, float(alpha), _ptr(A), lda, _ptr(B), ldb, float(beta),
                     _ptr(C0), ldc, out.ctypes.data_as(_F64P), max(1, N))
    return out


def bound(A, B, C0=None, alpha: float = 1.0, beta: float = 0.0, M=None, N=None, K=None,
          lib=None) -> np.ndarray:
    """Tolerance scale |alpha| * (|A| @ |B|) + |beta| * |C0| in float64."""
    lib = lib or load()
    M = A.shape[0] if M is None else M
    K = A.shape[1] if K is None else K
    N = B.shape[1] if N is None else N
    A, lda = _mat(A, M, K, "A")
    B, ldb = _mat(B, K, N, "B")
    C0, ldc = _mat(C0, M, N, "C0")
    out = np.empty((M, N), dtype=np.float64)
    lib.oracle_bound(M, N, K, float(alpha), _ptr(A), lda, _ptr(B), ldb, float(beta),
                     _ptr(C0), ldc, out.ctypes.data_as(_F64P), max(1, N))
    return out


def _entries(fn, rows, cols, A, B, C0, alpha, beta, K):
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    cols = np.ascontiguousarray(cols, dtype=np.int32)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be 1-D and of equal length")
    M = int(rows.max()) + 1 if rows.size else 0
    N = int(cols.max()) + 1 if cols.size else 0
    A, lda = _mat(A, M, K, "A")
    B, ldb = _mat(B, K, N, "B")
    C0, ldc = _mat(C0, M, N, "C0")
    out = np.empty(rows.shape, dtype=np.float64)
    fn(rows.size, rows.ctypes.data_as(_I32P), cols.ctypes.data_as(_I32P), K, float(alpha),
       _ptr(A), lda, _ptr(B), ldb, float(beta), _ptr(C0), ldc, out.ctypes.data_as(_F64P))
    return out


def sgemm_entries(rows, cols, A, B, C0=None, alpha: float = 1.0, beta: float = 0.0, K=None,
                  lib=None) -> np.ndarray:
    """Reference values of the selected elements (rows[t], cols[t]) only."""
    lib = lib or load()
    K = A.shape[1] if K is None else K
    return _entries(lib.oracle_sgemm_entries, rows, cols, A, B, C0, alpha, beta, K)


def bound_entries(rows, cols, A, B, C0=None, alpha: float = 1.0, beta: float = 0.0, K=None,
                  lib=None) -> np.ndarray:
    """Tolerance scale of the selected elements only."""
    lib = lib or load()
    K = A.shape[1] if K is None else K
    return _entries(lib.oracle_bound_entries, rows, cols, A, B, C0, alpha, beta, K)


ACT_NONE = 0
ACT_RELU = 1


def _epilogue(lib, vals, rows, cols, bias, act, bnd=None):
    """Apply the fused epilogue (oracle_epilogue) in place to float64 arrays."""
    rows = np.ascontiguousarray(rows, dtype=np.int32).ravel()
    cols = np.ascontiguousarray(cols, dtype=np.int32).ravel()
    if not vals.flags.c_contiguous:
        raise ValueError("epilogue values must be C-contiguous")
    flat = vals.reshape(-1)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    bp = None if b is None else b.ctypes.data_as(_F32P)
    lib.oracle_epilogue(flat.size, rows.ctypes.data_as(_I32P), cols.ctypes.data_as(_I32P), bp,
                        int(act), flat.ctypes.data_as(_F64P),
                        None if bnd is None else bnd.reshape(-1).ctypes.data_as(_F64P))


def sgemm_fused(A, B, C0=None, alpha: float = 1.0, beta: float = 0.0, bias=None,
                act: int = ACT_NONE, M=None, N=None, K=None, lib=None) -> np.ndarray:
    """Reference act(alpha A B + beta C0 + bias[None, :]) in float64 (bias: one
    float32 per column of C, or None; act: ACT_NONE or ACT_RELU)."""
    lib = lib or load()
    out = sgemm(A, B, C0, alpha, beta, M=M, N=N, K=K, lib=lib)
    rr, cc = np.indices(out.shape, dtype=np.int32)
    _epilogue(lib, out, rr, cc, bias, act)
    return out


def bound_fused(A, B, C0=None, alpha: float = 1.0, beta: float = 0.0, bias=None, M=None,
                N=None, K=None, lib=None) -> np.ndarray:
    """Tolerance scale of sgemm_fused: bound(...) + |bias[j]|."""
    lib = lib or load()
    bnd = bound(A, B, C0, alpha, beta, M=M, N=N, K=K, lib=lib)
    vals = np.zeros_like(bnd)
    rr, cc = np.indices(bnd.shape, dtype=np.int32)
    _epilogue(lib, vals, rr, cc, bias, ACT_NONE, bnd)
    return bnd


def sgemm_fused_entries(rows, cols, A, B, C0=None, alpha: float = 1.0, beta: float = 0.0,
                        bias=None, act: int = ACT_NONE, K=None, lib=None) -> np.ndarray:
    """sgemm_fused at the selected elements only."""
    lib = lib or load()
    out = sgemm_entries(rows, cols, A, B, C0, alpha, beta, K=K, lib=lib)
    _epilogue(lib, out, rows, cols, bias, act)
    return out


def bound_fused_entries(rows, cols, A, B, C0=None, alpha: float = 1.0, beta: float = 0.0,
                        bias=None, K=None, lib=None) -> np.ndarray:
    """bound_fused at the selected elements only."""
    lib = lib or load()
    bnd = bound_entries(rows, cols, A, B, C0, alpha, beta, K=K, lib=lib)
    vals = np.zeros_like(bnd)
    _epilogue(lib, vals, rows, cols, bias, ACT_NONE, bnd)
    return bnd


def threads(lib=None) -> int:
    """OpenMP threads the oracle's loops use."""
    return int((lib or load()).oracle_threads())


def set_threads(n: int, lib=None) -> int:
    """Use n OpenMP threads from now on; returns the number in effect."""
    return int((lib or load()).oracle_set_threads(int(n)))


def within_tolerance(got, ref, bnd, rel: float = 1e-4):
    """Acceptance rule: |got - ref| <= rel * bnd on every element where the
    reference is finite (and got must be finite there too); where the
    reference is NaN, got must be NaN, and where it is +-Inf, got must be the
    same infinity.  Returns (ok, worst ratio over the finite elements)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bnd = np.asarray(bnd, dtype=np.float64)
    finite_ref = np.isfinite(ref)
    bad_nonfinite = ~np.isfinite(got) & finite_ref
    # non-finite reference values are matched exactly: NaN by NaN, an
    # infinity by the same-signed infinity
    nan_ref = np.isnan(ref)
    inf_ref = np.isinf(ref)
    bad_nan = nan_ref & ~np.isnan(got)
    bad_inf = inf_ref & (got != ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        err = np.abs(got - ref)
        ratio = np.where(bnd > 0, err / (rel * bnd), np.where(err == 0, 0.0, np.inf))
    ratio = np.where(finite_ref, ratio, 0.0)
    worst = float(ratio.max()) if ratio.size else 0.0
    ok = not (bad_nonfinite.any() or bad_nan.any() or bad_inf.any()) and worst <= 1.0
    return ok, worst
