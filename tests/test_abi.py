"""The C-ABI library on the CPU: it builds/loads, exports every symbol the
header declares, and its host-side logic (argument checks, quick returns,
configuration names and selection) works without a GPU."""
import os
import re
import subprocess

import pytest

import fp32_gemm_06_amd as fg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp32gemm.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fg.LIB_PATH):
        from fp32_gemm_06_amd import build
        build.build()
    return fg.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b([A-Za-z_]\w*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_declares_the_documented_entry_points():
    names = declared_functions()
    assert set(names) == set(fg.EXPORTS), names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", fg.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(ln.split()[-1] for ln in out.splitlines() if " T " in ln)
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    # nothing else leaks out of the library as a global function
    assert exported == set(declared_functions()), exported - set(declared_functions())


def test_header_compiles_as_c():
    src = f'#include "{HEADER}"\nint main(void) {{ return sgemm(0,0,0,1.0f,0,1,0,1,0.0f,0,1,0); }}\n'
    r = subprocess.run(["gcc", "-x", "c", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-"],
                       input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


ARGS = dict(M=4, N=4, K=4, alpha=1.0, A=16, lda=4, B=16, ldb=4, beta=0.0, C=16, ldc=4)


def call(fn, **kw):
    a = dict(ARGS, **kw)
    return fn(a["M"], a["N"], a["K"], a["alpha"], a["A"], a["lda"], a["B"], a["ldb"], a["beta"],
              a["C"], a["ldc"], 0)


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), -1), (dict(N=-1), -2), (dict(K=-1), -3),
    (dict(A=None), -5), (dict(K=8, lda=4), -6), (dict(B=None), -7),
    (dict(N=8, ldb=4, ldc=8), -8), (dict(C=None), -10), (dict(N=8, ldb=8, ldc=4), -11),
    (dict(lda=(1 << 20) + 1), -6), (dict(ldb=(1 << 20) + 1), -8), (dict(ldc=(1 << 20) + 1), -11),
])
def test_argument_checks_need_no_gpu(lib, kw, code):
    assert call(fg.sgemm, **kw) == code
    assert call(fg.sgemv, **kw) == code
    assert "invalid argument" in fg.strerror(code)


def test_quick_returns_need_no_gpu(lib):
    # M == 0 or N == 0: nothing happens, NULL pointers are fine
    assert call(fg.sgemm, M=0, A=None, B=None, C=None) == 0
    assert call(fg.sgemm, N=0, A=None, B=None, C=None, ldb=1, ldc=1) == 0
    # alpha == 0 and beta == 1: C is left alone, A and B may be NULL
    assert call(fg.sgemm, alpha=0.0, beta=1.0, A=None, B=None) == 0
    # K == 0 and beta == 1
    assert call(fg.sgemm, K=0, lda=1, beta=1.0, A=None, B=None) == 0


EX = dict(ta=0, tb=0, M=4, N=4, K=4, alpha=1.0, A=16, lda=4, B=16, ldb=4, beta=0.0, C=16, ldc=4)


def call_ex(**kw):
    a = dict(EX, **kw)
    return fg.sgemm_ex(a["ta"], a["tb"], a["M"], a["N"], a["K"], a["alpha"], a["A"], a["lda"],
                       a["B"], a["ldb"], a["beta"], a["C"], a["ldc"], 0)


@pytest.mark.parametrize("kw,code", [
    (dict(ta=2), -1), (dict(tb=-1), -2), (dict(M=-1), -3), (dict(N=-1), -4), (dict(K=-1), -5),
    (dict(A=None), -7), (dict(K=8, lda=4), -8), (dict(ta=1, M=8, lda=4, ldc=4, N=4), -8),
    (dict(B=None), -9), (dict(tb=1, K=8, lda=8, ldb=4), -10), (dict(C=None), -12),
    (dict(N=8, ldb=8, ldc=4), -13),
])
def test_sgemm_ex_argument_checks(lib, kw, code):
    assert call_ex(**kw) == code


def test_batched_argument_checks(lib):
    def b(**kw):
        a = dict(ta=0, tb=0, M=4, N=4, K=4, alpha=1.0, A=16, lda=4, sA=16, B=16, ldb=4, sB=16,
                 beta=0.0, C=16, ldc=4, sC=16, batch=2)
        a.update(kw)
        return fg.sgemm_strided_batched(a["ta"], a["tb"], a["M"], a["N"], a["K"], a["alpha"],
                                        a["A"], a["lda"], a["sA"], a["B"], a["ldb"], a["sB"],
                                        a["beta"], a["C"], a["ldc"], a["sC"], a["batch"], 0)
    assert b(sA=-1) == -9
    assert b(sB=-4) == -12
    assert b(sC=8) == -16          # C entries would overlap
    assert b(batch=-1) == -17
    assert b(batch=70000) == -17
    assert b(batch=0, A=None, B=None, C=None) == 0   # nothing to do
    assert b(M=0, C=None) == 0
    assert b(alpha=0.0, beta=1.0, A=None, B=None) == 0
    assert fg.strerror(-17) == "invalid argument 17"


def test_gemv_batch_range(lib):
    """M from 1 to 128; each configuration runs up to its own row limit."""
    assert call(fg.sgemv, M=129) == -1
    assert call(fg.sgemv, M=0) == -1
    assert fg.fp32gemm_sgemv_with_config(0, 129, 4, 4, 1.0, 16, 4, 16, 4, 0.0, 16, 4, 0) == -1
    names = fg.config_names(fg.KIND_SGEMV)
    rows = [fg.fp32gemm_config_max_rows(fg.KIND_SGEMV, c) for c in range(len(names))]
    assert set(rows) == {8, 32, 64, 128}
    for cfg, name in enumerate(names):
        # the 4-rows-per-lane, <= 8-wave GEMV configurations take 32 rows,
        # the MFMA ones 128 (16- and 32-column stripes) or 64 (64 columns),
        # the others 8
        if name.startswith("mfma"):
            assert rows[cfg] == {"16": 128, "32": 128, "64": 64}[name[4:6]], name
        elif name.startswith("split"):
            assert rows[cfg] == 8, name
        else:
            waves, unroll = (int(v[1:]) for v in name.split("_")[1:3])
            assert rows[cfg] == (32 if unroll == 4 and waves <= 8 else 8), name
        # M = 9 with a NULL C: a runnable configuration reaches the argument
        # check (-10), the others stop at the configuration check
        for M in (9, 33, 65):
            rc = fg.fp32gemm_sgemv_with_config(cfg, M, 4, 4, 1.0, 16, 4, 16, 4, 0.0, None, 4, 0)
            assert rc == (-10 if M <= rows[cfg] else fg.ERR_CONFIG), (name, M, rc)
    assert fg.fp32gemm_config_max_rows(fg.KIND_SGEMV, len(names)) == -1
    assert fg.fp32gemm_config_max_rows(fg.KIND_SGEMM, 0) > 128


def test_configs(lib):
    for kind in (fg.KIND_SGEMM, fg.KIND_SGEMV):
        n = fg.fp32gemm_num_configs(kind)
        assert n > 0
        names = fg.config_names(kind)
        assert len(set(names)) == n and all(names)
        assert fg.fp32gemm_config_name(kind, n) is None
        assert fg.fp32gemm_config_name(kind, -1) is None
    assert fg.fp32gemm_num_configs(7) == 0
    assert fg.fp32gemm_select_config(7, 1, 1, 1) == fg.ERR_CONFIG
    assert fg.fp32gemm_sgemm_with_config(10 ** 6, 4, 4, 4, 1.0, 16, 4, 16, 4, 0.0, 16, 4, 0) == \
        fg.ERR_CONFIG
    assert fg.strerror(fg.ERR_CONFIG) == "unknown configuration id"


@pytest.mark.parametrize("shape", [(4092, 4092, 4092), (4096, 4096, 4096), (2048, 11008, 4096),
                                   (128, 128, 128), (1, 1, 1), (100000, 16, 16)])
def test_selection_is_a_valid_sgemm_config(lib, shape):
    cfg = fg.fp32gemm_select_config(fg.KIND_SGEMM, *shape)
    assert 0 <= cfg < fg.fp32gemm_num_configs(fg.KIND_SGEMM)


def test_tuned_shapes_resolve_to_their_table_entries(lib):
    table = open(os.path.join(ROOT, "fp32_gemm_06_amd", "csrc", "tune_table.inc")).read()
    gemm_part, gemv_part = table.split("kGemvTable")
    for fam, part in ((fg.KIND_SGEMM, gemm_part), (fg.KIND_SGEMV, gemv_part)):
        for M, N, K, name in re.findall(r'\{(\d+), (\d+), (\d+), "([^"]+)"\}', part):
            cfg = fg.fp32gemm_select_config(fam, int(M), int(N), int(K))
            assert fg.fp32gemm_config_name(fam, cfg) == name, (M, N, K, name)


SK = dict(ta=0, tb=0, M=64, N=64, K=4096, alpha=1.0, A=16, lda=4096, B=16, ldb=64, beta=0.0,
          C=16, ldc=64, splits=4, ws=None, wsb=0)


def call_sk(**kw):
    a = dict(SK, **kw)
    return fg.sgemm_splitk(a["ta"], a["tb"], a["M"], a["N"], a["K"], a["alpha"], a["A"],
                           a["lda"], a["B"], a["ldb"], a["beta"], a["C"], a["ldc"], a["splits"],
                           a["ws"], a["wsb"], 0)


def test_splitk_argument_checks_need_no_gpu(lib):
    assert call_sk(ta=3) == -1
    assert call_sk(K=-1) == -5
    assert call_sk(lda=100) == -8
    assert call_sk(splits=-1) == -14
    assert call_sk(splits=70000) == -14
    assert call_sk() == -15                       # four chunks need a workspace
    assert call_sk(ws=16, wsb=4 * 64 * 64 * 4 - 1) == -16
    assert call_sk(M=0, A=None, B=None, C=None) == 0
    assert call_sk(alpha=0.0, beta=1.0, A=None, B=None) == 0


def test_splitk_noalloc_checks_need_no_gpu(lib):
    """The no-allocation split-K: argument errors and the scratch limit are
    reported before anything is enqueued."""
    def f(**kw):
        a = dict(SK)
        a.update(kw)
        return fg.sgemm_splitk_noalloc(a["ta"], a["tb"], a["M"], a["N"], a["K"], a["alpha"],
                                       a["A"], a["lda"], a["B"], a["ldb"], a["beta"], a["C"],
                                       a["ldc"], a["splits"], 0)
    assert f(ta=3) == -1
    assert f(K=-1) == -5
    assert f(lda=100) == -8
    assert f(splits=-1) == -14
    assert f(splits=70000) == -14
    assert f(C=None) == -12
    # 4 chunks x 2048 x 2048 floats = 16 Mi > the 4 Mi scratch
    assert f(M=2048, N=2048, lda=4096, ldb=2048, ldc=2048) == fg.ERR_SCRATCH
    assert "16 MiB" in fg.strerror(fg.ERR_SCRATCH)
    assert f(M=0, A=None, B=None, C=None) == 0
    assert f(alpha=0.0, beta=1.0, A=None, B=None) == 0


def test_splitk_workspace_size(lib):
    ws = fg.sgemm_splitk_workspace_size
    assert ws(64, 64, 4096, 4) == 4 * 64 * 64 * 4
    # 100 / 4 = 25, rounded up to a 32-value chunk: ceil(100 / 32) = 4 chunks
    assert ws(64, 64, 100, 4) == 4 * 64 * 64 * 4
    assert ws(64, 64, 96, 4) == 3 * 64 * 64 * 4   # chunks of 32: three of them
    assert ws(64, 64, 32, 4) == 0                 # one chunk: no workspace
    assert ws(8, 64, 4096, 4) == 0                # M <= 8 runs the GEMV kernel
    assert ws(64, 64, 4096, 1) == 0
    assert ws(64, 64, 4096, -1) == 0
    # the automatic choice: none for a grid that fills the GPU, several for
    # a small C with a long K, and the size follows the chosen count
    assert fg.fp32gemm_splitk_splits(4096, 4096, 4096) == 1
    s = fg.fp32gemm_splitk_splits(256, 256, 32768)
    assert s >= 8
    assert ws(256, 256, 32768, 0) == s * 256 * 256 * 4


def call_stk(**kw):
    a = dict(SK, **kw)
    return fg.sgemm_streamk(a["ta"], a["tb"], a["M"], a["N"], a["K"], a["alpha"], a["A"],
                            a["lda"], a["B"], a["ldb"], a["beta"], a["C"], a["ldc"], a["ws"],
                            a["wsb"], 0)


def test_streamk_argument_checks_need_no_gpu(lib):
    """sgemm_streamk and its forced-plan hook report argument errors before
    anything is enqueued (the hook's positions are shifted by its two leading
    arguments)."""
    need = fg.sgemm_streamk_workspace_size(64, 64, 4096)
    assert need > 0
    assert call_stk(ta=3) == -1
    assert call_stk(K=-1) == -5
    assert call_stk(lda=100) == -8
    assert call_stk(C=None) == -12
    assert call_stk() == -14                      # no workspace
    assert call_stk(ws=16, wsb=need - 1) == -15  # too small
    assert call_stk(M=0, A=None, B=None, C=None) == 0
    assert call_stk(alpha=0.0, beta=1.0, A=None, B=None) == 0

    def hook(tile, groups, **kw):
        a = dict(SK, **kw)
        return fg.fp32gemm_streamk_with_config(tile, groups, a["ta"], a["tb"], a["M"], a["N"],
                                               a["K"], a["alpha"], a["A"], a["lda"], a["B"],
                                               a["ldb"], a["beta"], a["C"], a["ldc"], a["ws"],
                                               a["wsb"], 0)
    assert hook(99, 0) == fg.ERR_CONFIG
    assert hook(-2, 0) == fg.ERR_CONFIG
    assert hook(0, -1) == -2
    assert hook(0, 0, tb=5) == -4
    assert hook(0, 0) == -16
    assert hook(0, 0, ws=16, wsb=fg.fp32gemm_streamk_plan(64, 64, 4096, 0, 0)[0] - 1) == -17


def _sk_tile_edge(t):
    return int(fg.fp32gemm_streamk_tile_name(t).split("x")[0])


@pytest.mark.parametrize("shape", [(768, 768, 768), (1024, 1024, 1024), (1536, 1536, 1536),
                                   (384, 4096, 4096), (256, 256, 32768), (4160, 4160, 96),
                                   (16384, 16384, 1024), (9, 5000, 33), (4092, 4092, 4092)])
def test_streamk_plan_covers_every_unit(lib, shape):
    """Every plan deals each (tile, K slice) unit to exactly one workgroup:
    groups x ipw >= units > (groups - 1) x ipw, never more workgroups than
    asked for, and the workspace holds two partial tiles per workgroup plus
    one counter per tile."""
    M, N, K = shape
    for tile in (-1, 0, 1):
        for groups in (0, 1, 7, 300, 10 ** 9):
            wsb, t, g, ipw = fg.fp32gemm_streamk_plan(M, N, K, tile, groups)
            assert t >= 0 and (tile < 0 or t == tile), (shape, tile, groups)
            e = _sk_tile_edge(t)
            tiles = -(-M // e) * -(-N // e)
            units = tiles * -(-K // 32)
            assert g >= 1 and g * ipw >= units > (g - 1) * ipw, (shape, tile, groups, g, ipw)
            if groups:
                assert g <= groups
            assert wsb == (2 * g * e * e + tiles + 64) * 4
    assert fg.sgemm_streamk_workspace_size(M, N, K) == (
        fg.fp32gemm_streamk_plan(M, N, K)[0] if M > 8 else 0)
    assert fg.sgemm_streamk_workspace_size(8, N, K) == 0
    assert fg.fp32gemm_streamk_plan(0, N, K) == (0, -1, 0, 0)


def test_fused_argument_checks_need_no_gpu(lib):
    def f(**kw):
        a = dict(EX, bias=None, act=0)
        a.update(kw)
        return fg.sgemm_fused(a["ta"], a["tb"], a["M"], a["N"], a["K"], a["alpha"], a["A"],
                              a["lda"], a["B"], a["ldb"], a["beta"], a["C"], a["ldc"], a["bias"],
                              a["act"], 0)
    assert f(act=2) == -15
    assert f(act=-1) == -15
    assert f(ta=5) == -1
    assert f(C=None) == -12
    assert f(M=0, A=None, B=None, C=None, act=1) == 0
    # alpha == 0, beta == 1 and no epilogue: C is left alone without a launch
    assert f(alpha=0.0, beta=1.0, A=None, B=None) == 0


def test_round_split_plan():
    """The dispatcher's two-launch plan: one launch where the 256x256 tiles
    fill whole rounds (or the split would not pay), and where it splits, the
    first part is whole rounds of 256 tiles and the rest is non-empty."""
    assert fg.fp32gemm_round_split(4092, 4092, 4092) == (0, 0)
    assert fg.fp32gemm_round_split(4096, 4096, 4096) == (0, 0)
    assert fg.fp32gemm_round_split(8192, 8192, 8192) == (0, 0)
    assert fg.fp32gemm_round_split(128, 128, 128) == (0, 0)
    assert fg.fp32gemm_round_split(2048, 11008, 4096) == (1, 8192)
    assert fg.fp32gemm_round_split(3072, 8192, 4096) == (2, 2048)
    for (M, N, K, b) in [(2048, 11008, 4096, 1), (3072, 8192, 4096, 1), (4096, 13824, 4096, 1),
                         (8192, 32000, 4096, 1), (256, 300, 1024, 256), (1024, 28672, 4096, 1)]:
        dim, first = fg.fp32gemm_round_split(M, N, K, b)
        assert dim in (1, 2)
        across = -(-M // 256) if dim == 1 else -(-N // 256)
        along = N if dim == 1 else M
        assert first % 256 == 0 and 0 < first < along
        assert (across * (first // 256) * b) % 256 == 0


def test_model_choices():
    """The fallback tile model on shapes the table does not list: short K
    moves large products from 256x256 to 128x128 tiles (each tile's fixed
    cost is a larger share), fewer than 192 tiles of 64x64 go to 32x32 tiles,
    192..256 of them take the variant with two K slices per barrier (K >= 512
    only), more tiles keep the plain 64x64 tile, and a K too short to stage
    keeps it too."""
    name = lambda *s: fg.fp32gemm_config_name(0, fg.fp32gemm_select_config(0, *s))
    assert name(8192, 4096, 4096).startswith("256x256x32_")
    assert name(8192, 4096, 128).startswith("128x128x32_w64x32")
    assert name(4096, 4096, 64).startswith("128x128x32_w64x32")
    for shape in [(160, 4096, 4096), (192, 4096, 4096), (256, 4096, 11008), (1000, 1000, 1000)]:
        assert name(*shape) == "64x64x32_w32x32_p2_g8", shape
    for shape in [(384, 4096, 4096), (320, 4096, 4096), (1100, 1100, 1100)]:
        assert name(*shape).startswith("64x64x32_w32x32_g"), shape
    # 32x32 tiles below 192 tiles of 64x64 (K >= 128): four K slices per
    # stage with at most 512 of them and K >= 1024, two otherwise
    for shape in [(200, 2000, 8000), (100, 100, 4096), (512, 512, 8192), (256, 1024, 4096)]:
        assert name(*shape) == "32x32x32_w16x16_p4_m16_g8", shape
    for shape in [(300, 520, 260), (800, 800, 800), (64, 11008, 4096), (1000, 700, 300),
                  (700, 700, 700)]:
        assert name(*shape) == "32x32x32_w16x16_p2_m16_g8", shape
    for shape in [(896, 896, 896), (850, 850, 850), (512, 512, 100)]:
        assert not name(*shape).startswith("32x32"), shape
    # 32-row tiles where they save a round of 256 tiles (516 -> 430), not
    # where the rounds stay the same
    assert name(160, 11008, 4096) == "32x128x32_w32x32_g8"
    # 16x16x4 blocks from two rounds of 64x64 tiles on
    assert name(768, 4096, 4096) == "64x64x32_w32x32_m16_g8"
    assert name(1100, 1100, 1100).startswith("64x64x32_w32x32_g")
    for shape in [(96, 11008, 4096), (352, 4096, 4096)]:
        assert name(*shape).startswith("64x64x32_w32x32_g"), shape
    assert name(288, 11008, 4096) == "64x64x32_w32x32_m16_g8"
    # 96x96 tiles where they fill one or two whole rounds of 256 (89% of the
    # last round's slots, 95% of the tile area inside C), K >= 256
    for shape in [(1536, 1536, 4096), (384, 6144, 4096), (1536, 3072, 1536), (192, 11008, 4096),
                  (1530, 1530, 257), (768, 3072, 4096)]:
        assert name(*shape) == "96x96x32_w48x48_m16_g8", shape
    # not with half a round, four rounds, padding past C, or short K
    for shape in [(768, 1536, 4096), (1152, 1152, 1152), (3072, 3072, 3072), (160, 11008, 4096),
                  (1530, 1530, 100)]:
        assert not name(*shape).startswith("96x96"), shape


def test_split_gemv_choice():
    """K split across workgroups for large weights with few 256-column
    blocks: from about 12 M weights at M <= 4, from 16 M with at most 16
    column blocks at M = 5..8; not for small products or above 64 column
    blocks."""
    name = lambda *s: fg.fp32gemm_config_name(1, fg.fp32gemm_select_config(1, *s))
    for shape in [(1, 4000, 4096), (1, 4608, 4096), (4, 4096, 4096), (1, 4096, 11008),
                  (8, 4096, 11008), (6, 4000, 9000), (2, 16384, 4096), (1, 8192, 8192),
                  (6, 4096, 4096), (8, 4096, 4096)]:
        assert name(*shape) in ("split256_w4_u4", "split256_w8_u4"), shape
    for shape in [(1, 2048, 2048), (1, 1024, 1024), (8, 4000, 4096), (1, 32000, 4096),
                  (1, 16640, 4096), (8, 8192, 8192), (7, 14000, 4096)]:
        assert not name(*shape).startswith("split"), shape


def test_stripe_width_by_rounds():
    """Column-stripe and skinny widths: the narrowest stripe whose grid needs
    the fewest rounds of 256 workgroups (weighted by the wider stripes' cost
    per workgroup), within each configuration's row limit."""
    name = lambda *s: fg.fp32gemm_config_name(1, fg.fp32gemm_select_config(1, *s))
    # M <= 8 below the split kernel's size: 16 columns while one round
    # holds the grid (N <= 4096), then 32, then 64
    assert name(1, 4000, 2048) == "c16_w8_u4"
    assert name(4, 4000, 2048) == "c16_w4_u8"
    for N in (4608, 6144, 7168):
        assert name(1, N, 1024) == "c32_w8_u4", N
    assert name(1, 9216, 1024) == "c64_w8_u4"
    assert name(8, 16384, 1024) == "c64_w8_u4"
    # M = 5..8 on the skinny kernel while its stripes fit one round
    assert name(8, 4000, 2048) == "mfma16_w8"
    assert name(6, 8192, 2048) == "mfma32_w8"
    assert name(8, 9216, 1024) == "c64_w8_u4"
    # skinny kernel: 64-column stripes up to M = 64, 32-column up to 128
    assert name(16, 4096, 4096) == "mfma16_w8"
    assert name(48, 4608, 4096) == "mfma32_w8"
    assert name(48, 11008, 4096) == "mfma64_w8"
    assert name(80, 8192, 4096) == "mfma32_w8"
    assert name(80, 11008, 4096) == "mfma16_w8"   # 3 rounds of 16 against 2 of 32 at 1.5x
    assert name(128, 16384, 4096) == "mfma32_w8"
    for M in (65, 100, 128):
        cfg = fg.fp32gemm_select_config(1, M, 16384, 4096)
        assert fg.fp32gemm_config_max_rows(1, cfg) >= M


def test_measurement_probes_check_their_arguments():
    """The two measurement probes (their own libraries, outside the GEMM
    ABI) load, export one entry point each, and reject shapes their kernels
    do not take before touching the GPU."""
    import ctypes
    from fp32_gemm_06_amd import build
    for path in build.PROBES.values():
        if not os.path.exists(path):
            build.build()
            break
    hbm = ctypes.CDLL(build.PROBES["hbm_probe.hip"])
    hbm.hbm_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    n = 4096 * 4096
    assert hbm.hbm_stream_read(16, n, 256, 6, 16, None, None) == -1       # waves 4 or 8
    assert hbm.hbm_stream_read(16, n + 256, 256, 4, 16, None, None) == -1  # whole steps only
    assert hbm.hbm_stream_read(16, n, 0, 4, 16, None, None) == -1
    assert hbm.hbm_stream_read(16, 0, 256, 4, 16, None, None) == -1
    mfma = ctypes.CDLL(build.PROBES["mfma_probe.hip"])
    mfma.mfma_issue_rate.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 3
    assert mfma.mfma_issue_rate(8, 256, 4, 10, 16, 16, None) == -1   # 32x32x2 or 16x16x4
    assert mfma.mfma_issue_rate(32, 256, 2, 10, 16, 16, None) == -1  # waves 4 or 8
    assert mfma.mfma_issue_rate(32, 0, 4, 10, 16, 16, None) == -1
    assert mfma.mfma_issue_rate(32, 256, 4, 0, 16, 16, None) == -1
    assert mfma.mfma_issue_rate(32, 256, 4, 10, None, 16, None) == -1
    assert mfma.mfma_issue_rate(32, 256, 4, 10, 16, None, None) == -1
