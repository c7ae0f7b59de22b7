"""Seeded random cases over every entry point, element by element against the oracle.

Each case draws an entry point (sgemm, sgemv, sgemm_ex, sgemm_strided_batched,
sgemm_fused, sgemm_splitk, sgemm_streamk with the library's plan or a forced
tile and workgroup count, or sgemm / sgemv with a tile or GEMV configuration
forced, drawn from all of them), a shape with M from the decode range (1..8, or
9..128 for the GEMV entry points) or up to a few tiles with ragged tails, operand transposes, padded leading
dimensions, operands shifted off 16-byte alignment, alpha and beta (zero
included), and for the fused and split-K entry points a bias, an activation and
a chunk count.  The operands live in one device buffer each, padding columns
hold NaN and a sentinel follows the last entry, so a read of padding or a stray
write shows up too.

Tolerance (every element): |C - C_ref| <= 1e-4 * (|alpha| |op(A)||op(B)| + |beta| |C0|
+ |bias|), the same rule as the other parity tests.
"""
import numpy as np
import pytest

import fp32_gemm_06_amd as fg
import oracle
from fp32_gemm_06_amd import inputs
from gpu_util import assert_parity, require_gpu

pytestmark = pytest.mark.gpu

ENTRIES = ("sgemm", "sgemv", "sgemm_ex", "batched", "fused", "splitk", "sgemm_cfg", "sgemv_cfg",
           "streamk")
N_CASES = 486
SENTINEL = 12345.0


def draw_case(i):
    g = np.random.default_rng(9000 + i)
    entry = ENTRIES[i % len(ENTRIES)]
    if entry in ("sgemv", "sgemv_cfg"):
        M = int(g.integers(1, 9)) if g.random() < 0.5 else int(g.integers(9, 129))
    elif g.random() < 0.3:
        M = int(g.integers(1, 9))
    else:
        M = int(g.integers(9, 331))
    N = int(g.integers(1, 331))
    K = int(g.integers(1, 401))
    trans = entry in ("sgemm_ex", "batched", "fused", "splitk", "streamk")
    ta = int(g.integers(0, 2)) if trans else 0
    tb = int(g.integers(0, 2)) if trans else 0
    pads = tuple(int(p) for p in g.integers(0, 6, size=3)) if g.random() < 0.5 else (0, 0, 0)
    offset = int(g.integers(1, 4)) if g.random() < 0.25 else 0
    alpha = float(g.choice([1.0, 0.5, -1.25, 2.0, 0.0], p=[0.3, 0.2, 0.2, 0.2, 0.1]))
    beta = float(g.choice([0.0, 1.0, 0.5, -2.0]))
    kind = "int" if g.random() < 0.3 else "uniform"
    batch = int(g.integers(1, 4)) if entry == "batched" else 1
    has_bias = entry == "fused" and g.random() < 0.8
    act = int(g.integers(0, 2)) if entry == "fused" else oracle.ACT_NONE
    splits = int(g.choice([0, 1, 2, 3, 7])) if entry == "splitk" else 0
    cfg = -1
    if entry == "sgemm_cfg":
        cfg = int(g.integers(0, fg.fp32gemm_num_configs(fg.KIND_SGEMM)))
    elif entry == "sgemv_cfg":
        # a configuration whose row limit takes this M
        ok = [c for c in range(fg.fp32gemm_num_configs(fg.KIND_SGEMV))
              if fg.fp32gemm_config_max_rows(fg.KIND_SGEMV, c) >= M]
        cfg = ok[int(g.integers(0, len(ok)))]
    # stream-K: the library's plan, or a forced tile with few workgroups (a
    # workgroup then spans several tiles and tiles are cut into many segments)
    sk_tile, sk_groups = -1, 0
    if entry == "streamk" and g.random() < 0.5:
        ntiles = 0
        while fg.fp32gemm_streamk_tile_name(ntiles) is not None:
            ntiles += 1
        sk_tile = int(g.integers(0, ntiles))
        sk_groups = int(g.choice([1, 3, 7, 40, 0]))
    return dict(entry=entry, M=M, N=N, K=K, ta=ta, tb=tb, pads=pads, offset=offset,
                alpha=alpha, beta=beta, kind=kind, batch=batch, has_bias=has_bias, act=act,
                splits=splits, cfg=cfg, sk_tile=sk_tile, sk_groups=sk_groups, seed=9000 + i)


def _draw(g, kind, r, c):
    if kind == "int":
        return g.integers(-4, 5, size=(r, c)).astype(np.float32)
    return inputs.uniform(g, (r, c))


def _store(torch, mats, ld, stride, offset, guard):
    """One device buffer holding `mats` (r x c each) at row stride ld and entry
    stride `stride`, `offset` floats past a 16-byte boundary; NaN in the row
    padding, SENTINEL everywhere else outside the entries."""
    r, c = mats[0].shape
    span = (r - 1) * ld + c
    n = offset + (len(mats) - 1) * stride + span + guard + 4
    host = np.full((n,), SENTINEL, dtype=np.float32)
    for b, m in enumerate(mats):
        base = offset + b * stride
        rows = np.full((r, ld), np.nan, dtype=np.float32)
        rows[:, :c] = m
        flat = rows.reshape(-1)[:span]
        host[base: base + span] = flat
    return torch.from_numpy(host).cuda(), offset


def run_case(c):
    torch = require_gpu()
    g = inputs.rng(c["seed"])
    M, N, K, batch = c["M"], c["N"], c["K"], c["batch"]
    As = [_draw(g, c["kind"], M, K) for _ in range(batch)]
    Bs = [_draw(g, c["kind"], K, N) for _ in range(batch)]
    Cs = [_draw(g, c["kind"], M, N) for _ in range(batch)]
    bias = inputs.uniform(g, (N,)) if c["has_bias"] else None

    a_store = [np.ascontiguousarray(a.T) if c["ta"] else a for a in As]
    b_store = [np.ascontiguousarray(b.T) if c["tb"] else b for b in Bs]
    lda = a_store[0].shape[1] + c["pads"][0]
    ldb = b_store[0].shape[1] + c["pads"][1]
    ldc = N + c["pads"][2]
    sA = a_store[0].shape[0] * lda + 3
    sB = b_store[0].shape[0] * ldb + 5
    sC = M * ldc + 7
    off = c["offset"]
    dA, oa = _store(torch, a_store, lda, sA, off, 8)
    dB, ob = _store(torch, b_store, ldb, sB, off, 8)
    dC, oc = _store(torch, Cs, ldc, sC, off, 64)
    pa, pb, pc = (t.data_ptr() + 4 * o for t, o in ((dA, oa), (dB, ob), (dC, oc)))
    ta, tb, al, be = c["ta"], c["tb"], c["alpha"], c["beta"]
    e = c["entry"]
    keep = []
    if e == "sgemm":
        rc = fg.sgemm(M, N, K, al, pa, lda, pb, ldb, be, pc, ldc)
    elif e == "sgemv":
        rc = fg.sgemv(M, N, K, al, pa, lda, pb, ldb, be, pc, ldc)
    elif e == "sgemm_cfg":
        rc = fg.fp32gemm_sgemm_with_config(c["cfg"], M, N, K, al, pa, lda, pb, ldb, be, pc, ldc)
    elif e == "sgemv_cfg":
        rc = fg.fp32gemm_sgemv_with_config(c["cfg"], M, N, K, al, pa, lda, pb, ldb, be, pc, ldc)
    elif e == "sgemm_ex":
        rc = fg.sgemm_ex(ta, tb, M, N, K, al, pa, lda, pb, ldb, be, pc, ldc)
    elif e == "batched":
        rc = fg.sgemm_strided_batched(ta, tb, M, N, K, al, pa, lda, sA, pb, ldb, sB, be, pc,
                                      ldc, sC, batch)
    elif e == "fused":
        db = None if bias is None else torch.from_numpy(bias).cuda()
        keep.append(db)
        rc = fg.sgemm_fused(ta, tb, M, N, K, al, pa, lda, pb, ldb, be, pc, ldc, db, c["act"])
    elif e == "streamk":
        if c["sk_tile"] < 0:
            nbytes = fg.sgemm_streamk_workspace_size(M, N, K)
        else:
            nbytes = fg.fp32gemm_streamk_plan(M, N, K, c["sk_tile"], c["sk_groups"])[0]
        ws = torch.empty(max(1, nbytes // 4), dtype=torch.float32, device="cuda")
        keep.append(ws)
        if c["sk_tile"] < 0:
            rc = fg.sgemm_streamk(ta, tb, M, N, K, al, pa, lda, pb, ldb, be, pc, ldc, ws, nbytes)
        else:
            rc = fg.fp32gemm_streamk_with_config(c["sk_tile"], c["sk_groups"], ta, tb, M, N, K, al,
                                                 pa, lda, pb, ldb, be, pc, ldc, ws, nbytes)
    else:
        nbytes = fg.sgemm_splitk_workspace_size(M, N, K, c["splits"])
        ws = torch.empty(max(1, nbytes // 4), dtype=torch.float32, device="cuda")
        keep.append(ws)
        rc = fg.sgemm_splitk(ta, tb, M, N, K, al, pa, lda, pb, ldb, be, pc, ldc, c["splits"],
                             ws, nbytes)
    if rc:
        raise fg.Fp32GemmError(rc)
    torch.cuda.synchronize()
    host = dC.cpu().numpy()
    outs, touched = [], np.zeros(host.shape, dtype=bool)
    for b in range(batch):
        base = oc + b * sC
        span = (M - 1) * ldc + N
        rows = np.full((M, ldc), np.nan, dtype=np.float32)
        rows.reshape(-1)[:span] = host[base: base + span]
        outs.append(rows[:, :N].astype(np.float64))
        for i in range(M):
            touched[base + i * ldc: base + i * ldc + N] = True
    # outside the entries: padding still NaN, everything else still the sentinel
    rest = host[~touched]
    guard_ok = bool(np.all(np.isnan(rest) | (rest == SENTINEL)))
    return As, Bs, Cs, bias, outs, guard_ok


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    c = draw_case(i)
    print("case", i, c, flush=True)
    As, Bs, Cs, bias, outs, guard_ok = run_case(c)
    assert guard_ok, f"case {i}: write outside C's entries"
    for b in range(c["batch"]):
        if c["entry"] == "fused":
            ref = oracle.sgemm_fused(As[b], Bs[b], Cs[b], c["alpha"], c["beta"], bias, c["act"])
            bnd = oracle.bound_fused(As[b], Bs[b], Cs[b], c["alpha"], c["beta"], bias)
        else:
            ref = oracle.sgemm(As[b], Bs[b], Cs[b], c["alpha"], c["beta"])
            bnd = oracle.bound(As[b], Bs[b], Cs[b], c["alpha"], c["beta"])
        assert_parity(outs[b], ref, bnd, f"case {i} entry {b}")
