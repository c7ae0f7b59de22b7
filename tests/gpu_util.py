"""Helpers for the GPU tests: device copies and the HIP path through the C ABI."""
from __future__ import annotations

import numpy as np
import pytest

import fp32_gemm_06_amd as fg


def require_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def to_dev(x: np.ndarray, pad_value: float = np.nan):
    """Copy a (possibly strided) host view to the GPU, keeping its row stride.

    Returns (tensor view of shape x.shape, ld).  The padding columns of the
    device buffer hold ``pad_value``.
    """
    import torch
    r, c = x.shape
    ld = x.strides[0] // 4 if r > 1 else max(1, c)
    ld = max(ld, c, 1)
    buf = torch.full((max(r, 1), ld), float(pad_value), dtype=torch.float32, device="cuda")
    if r and c:
        buf[:r, :c] = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return buf[:r, :c], ld


def run_hip(A, B, C0, alpha, beta, config=None, family="auto", guard=0, offset=0):
    """Run the HIP path on host arrays; return (C as float64 host array, ok canaries).

    ``guard`` adds that many canary floats before and after C's buffer and
    checks them afterwards.  ``offset`` shifts A/B/C by that many floats
    from a 16-byte boundary (misaligned operands).
    """
    import torch
    M, K = A.shape
    N = B.shape[1]

    def dev(x):
        r, c = x.shape
        ld = max(x.strides[0] // 4 if r > 1 else c, c, 1)
        n = r * ld + guard * 2 + offset + 4
        flat = torch.full((n,), 12345.0, dtype=torch.float32, device="cuda")
        if r and c:
            v = flat[guard + offset: guard + offset + r * ld].view(r, ld)
            pad = np.full((r, ld), np.nan, dtype=np.float32)
            pad[:, :c] = x
            v.copy_(torch.from_numpy(pad))
        return flat, guard + offset, ld

    fa, oa, lda = dev(A)
    fb, ob, ldb = dev(B)
    fc, oc, ldc = dev(C0)
    pa = fa.data_ptr() + 4 * oa
    pb = fb.data_ptr() + 4 * ob
    pc = fc.data_ptr() + 4 * oc
    args = (M, N, K, float(alpha), pa, lda, pb, ldb, float(beta), pc, ldc)
    if config is None:
        rc = fg.sgemm(*args) if family == "auto" else fg.sgemv(*args)
    elif family == "gemv":
        rc = fg.fp32gemm_sgemv_with_config(config, *args)
    else:
        rc = fg.fp32gemm_sgemm_with_config(config, *args)
    if rc != 0:
        raise fg.Fp32GemmError(rc)
    torch.cuda.synchronize()
    host = fc.cpu().numpy()
    out = host[oc: oc + M * ldc].reshape(M, ldc)[:, :N].astype(np.float64) if M else \
        np.zeros((0, N))
    canary_ok = True
    if guard:
        canary_ok = bool(np.all(host[:oc] == 12345.0)) and bool(
            np.all(host[oc + M * ldc:] == 12345.0))
        if M and ldc > N:
            pads = host[oc: oc + M * ldc].reshape(M, ldc)[:, N:]
            canary_ok = canary_ok and bool(np.all(np.isnan(pads)))
    return out, canary_ok


def assert_parity(got, ref, bnd, what=""):
    import oracle
    ok, worst = oracle.within_tolerance(got, ref, bnd)
    assert ok, f"{what}: worst |err| / (1e-4 * bound) = {worst:.3g}"
    return worst


def assert_bitexact(got, ref_f64, what=""):
    """Compare with the oracle's double result rounded once to fp32."""
    want = ref_f64.astype(np.float32).astype(np.float64)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (f"{what}: {len(bad)} elements differ, first at {tuple(bad[0])}: "
                           f"got {got[tuple(bad[0])]!r} want {want[tuple(bad[0])]!r}")
