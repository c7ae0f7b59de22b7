"""The benchmark's work/traffic accounting reproduces the numbers the pages print.

Fixture: tests/golden/pages_numbers.txt (each line cites its page and section).
"""
import os

import pytest

from fp32_gemm_06_amd import accounting as acc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.txt")


def _golden():
    out = {}
    with open(GOLDEN, encoding="utf-8") as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            key, val, tol, _cite = [x.strip() for x in line.split("|", 3)]
            out[key] = (float(val), float(tol))
    return out


G = _golden()
N4092 = 4092


def _computed():
    return {
        "flops_4092": acc.flops(N4092, N4092, N4092, with_update=True),
        "matrix_bytes_4092": acc.FP32 * N4092 * N4092,
        # beta != 0 counts the extra read of C, as the page does
        "min_traffic_4092": acc.algorithmic_bytes(N4092, N4092, N4092, beta=1.0),
        "min_reads_4092": 3 * acc.FP32 * N4092 * N4092,
        "naive_traffic_4092": acc.naive_bytes(N4092, N4092, N4092),
        "smem32_traffic_4092": acc.tile_operand_bytes(N4092, N4092, N4092, 32, 32),
        "tile_ai_32": acc.tile_intensity(32),
        "tile_ai_64": acc.tile_intensity(64),
        "grid_4092_by_32": acc.grid(N4092, N4092, 32, 32)[0],
        "last_block_rows_4092_by_32": acc.valid_in_last_block(N4092, 32),
        "grid_65_by_32": acc.grid(65, 65, 32, 32)[1],
        "compute_ms_a6000": acc.flops(N4092, N4092, N4092) / 30e12 * 1e3,
        "memory_ms_a6000": acc.algorithmic_bytes(N4092, N4092, N4092, beta=1.0) / 768e9 * 1e3,
    }


@pytest.mark.parametrize("key", sorted(G))
def test_printed_number(key):
    val, tol = G[key]
    got = _computed()[key]
    if tol == 0:
        assert got == val
    else:
        assert abs(got - val) <= tol * abs(val), (key, got, val)


def test_beta_zero_traffic_skips_c_read():
    # 201 MB when beta == 0: A, B read and C written once
    assert acc.algorithmic_bytes(N4092, N4092, N4092, beta=0.0) == 200_933_568
    assert acc.flops(N4092, N4092, N4092) == 137_036_693_376


def test_decode_bytes():
    assert acc.algorithmic_bytes(1, 4096, 4096, 0.0) == 67_141_632
    assert acc.algorithmic_bytes(8, 4096, 4096, 0.0) == 67_371_008


def test_l2_intensity_above_ridge():
    ridge = acc.PEAK_FP32_TFLOPS * 1e12 / (acc.PEAK_HBM_GBPS * 1e9)
    assert acc.l2_intensity(256, 256) == 64
    assert acc.l2_intensity(128, 128) == 32
    assert acc.l2_intensity(128, 128) > ridge
