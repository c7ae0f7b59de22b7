"""Transposed operands (sgemm_ex) and strided batches (sgemm_strided_batched)
against the CPU oracle.

The oracle computes the plain definition on op(A) and op(B) as row-major host
arrays; the GPU receives the storage (A stored K x M when op(A) = A^T, B stored
N x K when op(B) = B^T).  Integer inputs make the expected values exact, so
these cases are bit-exact; uniform inputs use the standard tolerance.
"""
import itertools

import numpy as np
import pytest

import fp32_gemm_06_amd as fg
import oracle
from fp32_gemm_06_amd import inputs
from gpu_util import assert_bitexact, assert_parity, require_gpu

pytestmark = pytest.mark.gpu

COMBOS = list(itertools.product((0, 1), (0, 1)))
SENTINEL = 12345.0


def _draw(g, kind, r, c):
    if kind == "int":
        return g.integers(-4, 5, size=(r, c)).astype(np.float32)
    return inputs.uniform(g, (r, c))


def _store(torch, mats, ld, stride, offset, guard):
    """Device buffer holding matrices `mats` (each r x c) with row stride ld,
    entry stride `stride` (elements), `offset` floats from a 16-byte boundary
    and `guard` sentinel floats after the last entry.  Row padding is NaN."""
    r, c = mats[0].shape
    span = (r - 1) * ld + c if r and c else 0
    n = offset + (len(mats) - 1) * stride + span + guard + 4
    flat = torch.full((n,), SENTINEL, dtype=torch.float32)
    for b, m in enumerate(mats):
        base = offset + b * stride
        for i in range(r):
            flat[base + i * ld: base + i * ld + c] = torch.from_numpy(m[i])
            if i + 1 < r:
                flat[base + i * ld + c: base + (i + 1) * ld] = float("nan")
    return flat.cuda(), offset


def run_batched(ta, tb, As, Bs, C0s, alpha, beta, pads=(0, 0, 0), gaps=(0, 0, 0), offset=0,
                config=None, share_a=False):
    """Run C_b <- alpha op(A_b) op(B_b) + beta C0_b for every entry on the GPU.

    As/Bs/C0s are the op() operands (row-major host arrays); returns the C
    entries (float64) and whether every sentinel outside them is intact."""
    torch = require_gpu()
    batch = len(C0s)
    M, K = As[0].shape
    N = Bs[0].shape[1]
    a_store = [np.ascontiguousarray(a.T) if ta else a for a in As]
    b_store = [np.ascontiguousarray(b.T) if tb else b for b in Bs]
    lda = a_store[0].shape[1] + pads[0]
    ldb = b_store[0].shape[1] + pads[1]
    ldc = N + pads[2]
    sA = 0 if share_a else a_store[0].shape[0] * lda + gaps[0]
    sB = b_store[0].shape[0] * ldb + gaps[1]
    sC = M * ldc + gaps[2]
    dA, oa = _store(torch, a_store[:1] if share_a else a_store, lda, sA, offset, 8)
    dB, ob = _store(torch, b_store, ldb, sB, offset, 8)
    dC, oc = _store(torch, C0s, ldc, sC, offset, 64)
    pa, pb, pc = (t.data_ptr() + 4 * o for t, o in ((dA, oa), (dB, ob), (dC, oc)))
    if batch == 1 and config is None:
        rc = fg.sgemm_ex(ta, tb, M, N, K, alpha, pa, lda, pb, ldb, beta, pc, ldc)
    elif config is not None:
        assert ta == 0 and tb == 0 and batch == 1
        rc = fg.fp32gemm_sgemm_with_config(config, M, N, K, alpha, pa, lda, pb, ldb, beta, pc, ldc)
    else:
        rc = fg.sgemm_strided_batched(ta, tb, M, N, K, alpha, pa, lda, sA, pb, ldb, sB, beta, pc,
                                      ldc, sC, batch)
    if rc:
        raise fg.Fp32GemmError(rc)
    torch.cuda.synchronize()
    host = dC.cpu().numpy()
    outs, ok = [], True
    touched = np.zeros(host.shape, dtype=bool)
    for b in range(batch):
        base = oc + b * sC
        rows = host[base: base + M * ldc].reshape(M, ldc) if M else np.zeros((0, ldc))
        outs.append(rows[:, :N].astype(np.float64))
        for i in range(M):
            touched[base + i * ldc: base + i * ldc + N] = True
            if ldc > N:
                ok = ok and bool(np.all(np.isnan(host[base + i * ldc + N: base + (i + 1) * ldc]))
                                 or i == M - 1)
    ok = ok and bool(np.all(host[~touched & ~np.isnan(host)] == SENTINEL))
    return outs, ok


def _case(seed, M, N, K, kind="int", batch=1):
    g = inputs.rng(seed)
    As = [_draw(g, kind, M, K) for _ in range(batch)]
    Bs = [_draw(g, kind, K, N) for _ in range(batch)]
    Cs = [_draw(g, kind, M, N) for _ in range(batch)]
    return As, Bs, Cs


@pytest.mark.parametrize("ta,tb", COMBOS)
@pytest.mark.parametrize("shape", [(70, 90, 110), (257, 129, 65), (300, 520, 260), (33, 31, 517),
                                   (12, 700, 300)], ids=str)
def test_transposes_bitexact(ta, tb, shape):
    M, N, K = shape
    As, Bs, Cs = _case(M * 7 + N * 3 + K, M, N, K)
    (got,), ok = run_batched(ta, tb, As, Bs, Cs, 1.0, 0.5, pads=(3, 5, 2))
    assert ok, "write outside C"
    assert_bitexact(got, oracle.sgemm(As[0], Bs[0], Cs[0], 1.0, 0.5), f"op {ta}{tb} {shape}")


@pytest.mark.parametrize("ta,tb", COMBOS)
def test_transposes_aligned_fast_path(ta, tb):
    """Shapes and strides that qualify for the 128-bit DMA path."""
    M, N, K = 260, 516, 132
    As, Bs, Cs = _case(5 + ta + 2 * tb, M, N, K)
    (got,), ok = run_batched(ta, tb, As, Bs, Cs, 1.0, 0.5, pads=(4, 8, 0))
    assert ok
    assert_bitexact(got, oracle.sgemm(As[0], Bs[0], Cs[0], 1.0, 0.5), f"op {ta}{tb} aligned")


@pytest.mark.parametrize("ta,tb", COMBOS)
@pytest.mark.parametrize("offset", [1, 3])
def test_transposes_misaligned(ta, tb, offset):
    """Operands off a 16-byte boundary take the 32-bit staged path."""
    M, N, K = 200, 132, 100
    As, Bs, Cs = _case(offset * 11 + ta + 2 * tb, M, N, K)
    (got,), ok = run_batched(ta, tb, As, Bs, Cs, 1.0, 0.5, offset=offset)
    assert ok
    assert_bitexact(got, oracle.sgemm(As[0], Bs[0], Cs[0], 1.0, 0.5), f"op {ta}{tb} off {offset}")


@pytest.mark.parametrize("ta,tb", COMBOS)
def test_transposes_uniform_tolerance(ta, tb):
    M, N, K = 1024, 768, 1000
    As, Bs, Cs = _case(77 + ta + 2 * tb, M, N, K, kind="uniform")
    (got,), _ = run_batched(ta, tb, As, Bs, Cs, 0.75, -1.25)
    assert_parity(got, oracle.sgemm(As[0], Bs[0], Cs[0], 0.75, -1.25),
                  oracle.bound(As[0], Bs[0], Cs[0], 0.75, -1.25), f"op {ta}{tb} uniform")


def test_every_config_every_combo():
    """Each tile configuration with each operand layout (through the batched
    entry point with one entry and the configuration the table picks is not
    enough: force every tile via a shape-independent check on NN, and cover
    the transposed layouts at the shapes that select each tile family)."""
    require_gpu()
    M, N, K = 300, 260, 130
    As, Bs, Cs = _case(99, M, N, K)
    ref = oracle.sgemm(As[0], Bs[0], Cs[0], 1.0, 0.5)
    for cfg in range(fg.fp32gemm_num_configs(0)):
        (got,), ok = run_batched(0, 0, As, Bs, Cs, 1.0, 0.5, pads=(4, 4, 4), config=cfg)
        assert ok
        assert_bitexact(got, ref, fg.fp32gemm_config_name(0, cfg))
    # transposed layouts at sizes whose table/fallback pick 64x64, 128x128 and 256x256 tiles
    for (M, N, K) in [(300, 260, 130), (2000, 2000, 64), (4092, 4092, 40)]:
        As, Bs, Cs = _case(M + K, M, N, K)
        ref = oracle.sgemm(As[0], Bs[0], Cs[0], 1.0, 0.5) if M < 1000 else None
        for ta, tb in COMBOS:
            (got,), ok = run_batched(ta, tb, As, Bs, Cs, 1.0, 0.5)
            assert ok
            if ref is not None:
                assert_bitexact(got, ref, f"op {ta}{tb} {(M, N, K)}")
            else:
                rows = np.array([0, 1, M // 2, M - 1], dtype=np.int32)
                rr = np.repeat(rows, N).astype(np.int32)
                cc = np.tile(np.arange(N, dtype=np.int32), len(rows))
                want = oracle.sgemm_entries(rr, cc, As[0], Bs[0], Cs[0], 1.0, 0.5)
                assert_bitexact(got[rr, cc], want, f"op {ta}{tb} {(M, N, K)} sampled")


@pytest.mark.parametrize("ta,tb", COMBOS)
def test_tile96_every_layout(ta, tb):
    """The 96x96 tile (four waves of 48x48 on 16x16x4 blocks; its k-rows of
    96 floats are 24 float4 chunks, so one DMA instruction spans parts of
    three rows) in every operand layout: shapes that fill one round of 256
    tiles route to it.  Aligned (128-bit DMA path), ragged M, N and K, and
    operands off a 16-byte boundary (32-bit staged path); bit-exact on
    integers."""
    for (M, N, K, pads, offset) in [(1536, 1536, 256, (4, 8, 4), 0), (1530, 1530, 257, (3, 5, 2), 0),
                                    (1534, 1535, 260, (0, 0, 0), 1)]:
        assert fg.fp32gemm_config_name(0, fg.fp32gemm_select_config(0, M, N, K)) == \
            "96x96x32_w48x48_m16_g8", (M, N, K)
        As, Bs, Cs = _case(M + N + K + offset + ta + 2 * tb, M, N, K)
        (got,), ok = run_batched(ta, tb, As, Bs, Cs, 1.0, 0.5, pads=pads, offset=offset)
        assert ok, "write outside C"
        assert_bitexact(got, oracle.sgemm(As[0], Bs[0], Cs[0], 1.0, 0.5),
                        f"96x96 op {ta}{tb} {(M, N, K)} offset {offset}")


@pytest.mark.parametrize("ta,tb", COMBOS)
def test_tile16x16_every_layout(ta, tb):
    """The 64x64 tile on 16x16x4 blocks in every operand layout (its lane
    quarters read k-rows from both k-halves of an mn-contiguous tile), through
    shapes the library runs on it.  Aligned, ragged M, N and K, and operands
    off a 16-byte boundary (32-bit staged path); bit-exact on integers."""
    for (M, N, K, pads, offset) in [(1024, 2048, 128, (4, 8, 4), 0), (1500, 1400, 130, (3, 5, 2), 0),
                                    (1401, 1503, 97, (0, 0, 0), 1)]:
        assert fg.fp32gemm_config_name(0, fg.fp32gemm_select_config(0, M, N, K)) == \
            "64x64x32_w32x32_m16_g8", (M, N, K)
        As, Bs, Cs = _case(M + N + K + offset + 3 * ta + 5 * tb, M, N, K)
        (got,), ok = run_batched(ta, tb, As, Bs, Cs, 1.0, 0.5, pads=pads, offset=offset)
        assert ok, "write outside C"
        assert_bitexact(got, oracle.sgemm(As[0], Bs[0], Cs[0], 1.0, 0.5),
                        f"16x16 blocks op {ta}{tb} {(M, N, K)} offset {offset}")


@pytest.mark.parametrize("ta,tb", COMBOS)
def test_tile32x32_every_layout(ta, tb):
    """The 32x32 tiles (four waves of one 16x16x4 block each) in every operand
    layout, through shapes the library runs on them: four K slices per stage
    (aligned, and ragged K past a stage), two (ragged M, N, K), and operands
    off a 16-byte boundary (32-bit staged path); bit-exact on integers."""
    for (M, N, K, pads, offset, cfg) in [(256, 512, 1024, (4, 8, 4), 0, "32x32x32_w16x16_p4_m16_g8"),
                                         (200, 300, 1100, (0, 4, 0), 0, "32x32x32_w16x16_p4_m16_g8"),
                                         (333, 517, 261, (3, 5, 2), 0, "32x32x32_w16x16_p2_m16_g8"),
                                         (301, 203, 157, (0, 0, 0), 1, "32x32x32_w16x16_p2_m16_g8")]:
        assert fg.fp32gemm_config_name(0, fg.fp32gemm_select_config(0, M, N, K)) == cfg, (M, N, K)
        As, Bs, Cs = _case(M + N + K + offset + 3 * ta + 5 * tb, M, N, K)
        (got,), ok = run_batched(ta, tb, As, Bs, Cs, 1.0, 0.5, pads=pads, offset=offset)
        assert ok, "write outside C"
        assert_bitexact(got, oracle.sgemm(As[0], Bs[0], Cs[0], 1.0, 0.5),
                        f"32x32 tile op {ta}{tb} {(M, N, K)} offset {offset}")


@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 1)])
def test_batched_32x32_tiles(ta, tb):
    """Eight entries of 192 x 160 x 300: 48 tiles of 64x64 over the batch, so
    the batch runs on 240 tiles of 32x32; the entries come from blockIdx.y and
    their tiles must not overlap."""
    M, N, K, batch = 192, 160, 300, 8
    As, Bs, Cs = _case(43 + ta, M, N, K, batch=batch)
    outs, ok = run_batched(ta, tb, As, Bs, Cs, 1.0, 0.5, pads=(4, 4, 4), gaps=(4, 8, 4))
    assert ok, "write outside the C entries"
    for b in range(batch):
        assert_bitexact(outs[b], oracle.sgemm(As[b], Bs[b], Cs[b], 1.0, 0.5), f"entry {b}")


@pytest.mark.parametrize("ta,tb", COMBOS)
def test_batched(ta, tb):
    M, N, K, batch = 100, 132, 70, 5
    As, Bs, Cs = _case(31 + ta + 2 * tb, M, N, K, batch=batch)
    outs, ok = run_batched(ta, tb, As, Bs, Cs, 1.0, 0.5, pads=(4, 0, 4), gaps=(8, 4, 12))
    assert ok, "write outside the C entries"
    for b in range(batch):
        assert_bitexact(outs[b], oracle.sgemm(As[b], Bs[b], Cs[b], 1.0, 0.5), f"entry {b}")


@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 1)])
def test_batched_rounds_of_96x96_tiles(ta, tb):
    """Two entries of 768 x 1536 x 260: 256 tiles of 96x96 over the batch, one
    round, a shape the library runs on that tile; the entries come from
    blockIdx.y and their tiles must not overlap."""
    M, N, K, batch = 768, 1536, 260, 2
    As, Bs, Cs = _case(41 + ta, M, N, K, batch=batch)
    outs, ok = run_batched(ta, tb, As, Bs, Cs, 1.0, 0.5, pads=(4, 4, 4), gaps=(4, 8, 4))
    assert ok, "write outside the C entries"
    for b in range(batch):
        assert_bitexact(outs[b], oracle.sgemm(As[b], Bs[b], Cs[b], 1.0, 0.5), f"entry {b}")


def test_batched_shared_a_misaligned_strides():
    """strideA = 0 (one A for every entry); odd strides force the 32-bit path."""
    M, N, K, batch = 64, 96, 33, 4
    As, Bs, Cs = _case(8, M, N, K, batch=batch)
    As = [As[0]] * batch
    outs, ok = run_batched(0, 1, As, Bs, Cs, 2.0, -1.0, gaps=(0, 1, 3), share_a=True)
    assert ok
    for b in range(batch):
        assert_bitexact(outs[b], oracle.sgemm(As[b], Bs[b], Cs[b], 2.0, -1.0), f"entry {b}")


def test_batched_large_uniform():
    """Per-head attention scores: batch of Q K^T with K stored row-major (op(B) = B^T)."""
    heads, seq, dim = 16, 512, 128
    g = inputs.rng(3)
    Q = [inputs.uniform(g, (seq, dim)) for _ in range(heads)]
    Kt = [inputs.uniform(g, (dim, seq)) for _ in range(heads)]   # op(B) = K^T
    Z = [np.zeros((seq, seq), np.float32) for _ in range(heads)]
    outs, ok = run_batched(0, 1, Q, Kt, Z, 0.125, 0.0)
    assert ok
    for b in (0, 7, 15):
        assert_parity(outs[b], oracle.sgemm(Q[b], Kt[b], None, 0.125, 0.0),
                      oracle.bound(Q[b], Kt[b], None, 0.125, 0.0), f"head {b}")


def test_batched_scale_only():
    """alpha = 0: every entry becomes beta * C (A and B never read)."""
    torch = require_gpu()
    M, N, batch = 30, 40, 3
    C = torch.arange(batch * M * N, dtype=torch.float32, device="cuda").reshape(batch, M, N)
    want = 0.5 * C.clone()
    rc = fg.sgemm_strided_batched(1, 1, M, N, 10, 0.0, None, M, 0, None, 10, 0, 0.5, C, N,
                                  M * N, batch)
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.equal(C, want)


@pytest.mark.parametrize("ta,tb", COMBOS)
@pytest.mark.parametrize("M", [1, 3, 8])
def test_batched_small_m_gemv(ta, tb, M):
    """M <= 8 entries run on the GEMV kernels (column stripes for op(B) = B,
    row dots for op(B) = B^T), one grid over the batch: the decode-time
    attention products (q K^T and p V per head)."""
    N, K, batch = 300, 500, 5
    As, Bs, Cs = _case(40 + M + 10 * ta + 20 * tb, M, N, K, batch=batch)
    outs, ok = run_batched(ta, tb, As, Bs, Cs, 1.0, 0.5, pads=(4, 4, 4), gaps=(8, 4, 12))
    assert ok, "write outside the C entries"
    for b in range(batch):
        assert_bitexact(outs[b], oracle.sgemm(As[b], Bs[b], Cs[b], 1.0, 0.5), f"M={M} entry {b}")


def test_batched_decode_attention_shapes():
    """32 heads, head dimension 128, 2048 cached positions, one query row:
    scores q K^T (K cache stored positions x dim) and the weighted sum p V."""
    heads, seq, dim = 32, 2048, 128
    g = inputs.rng(9)
    q = [inputs.uniform(g, (1, dim)) for _ in range(heads)]
    kt = [inputs.uniform(g, (dim, seq)) for _ in range(heads)]       # op(B) = K^T
    z = [np.zeros((1, seq), np.float32) for _ in range(heads)]
    outs, ok = run_batched(0, 1, q, kt, z, 0.088, 0.0)
    assert ok
    for b in (0, 17, 31):
        assert_parity(outs[b], oracle.sgemm(q[b], kt[b], None, 0.088, 0.0),
                      oracle.bound(q[b], kt[b], None, 0.088, 0.0), f"scores head {b}")
    p = [inputs.uniform(g, (1, seq)) for _ in range(heads)]
    v = [inputs.uniform(g, (seq, dim)) for _ in range(heads)]
    z = [np.zeros((1, dim), np.float32) for _ in range(heads)]
    outs, ok = run_batched(0, 0, p, v, z, 1.0, 0.0)
    assert ok
    for b in (0, 17, 31):
        assert_parity(outs[b], oracle.sgemm(p[b], v[b], None, 1.0, 0.0),
                      oracle.bound(p[b], v[b], None, 1.0, 0.0), f"p V head {b}")


def test_batched_small_m_shared_and_misaligned():
    """strideA = 0 with M = 2, and odd strides (32-bit loads in the GEMV kernels)."""
    M, N, K, batch = 2, 77, 301, 4
    As, Bs, Cs = _case(12, M, N, K, batch=batch)
    As = [As[0]] * batch
    for tb in (0, 1):
        outs, ok = run_batched(0, tb, As, Bs, Cs, 2.0, -1.0, gaps=(0, 1, 3), share_a=True, offset=1)
        assert ok
        for b in range(batch):
            assert_bitexact(outs[b], oracle.sgemm(As[b], Bs[b], Cs[b], 2.0, -1.0), f"tb={tb} {b}")
