"""The tuning table generator's choice rules, on synthetic sweep records (CPU)."""
import json

from fp32_gemm_06_amd import tune


def _write(tmp_path, recs):
    p = tmp_path / "sweep.jsonl"
    with open(p, "w") as f:
        for (M, cfg, us) in recs:
            f.write(json.dumps({"key": f"gemm:{M}:{cfg}", "family": "gemm", "M": M, "N": M, "K": M,
                                "config": cfg, "us": us}) + "\n")
    return str(p)


def test_clear_winner_kept(tmp_path):
    p = _write(tmp_path, [(64, "64x64x32_w32x32_g8", 100.0), (64, "128x128x32_w64x32_g8", 110.0),
                          (64, "256x256x32_w128x64_g8", 150.0)])
    assert tune.best_by_shape(p)[("gemm", 64, 64, 64)]["config"] == "64x64x32_w32x32_g8"


def test_near_tie_goes_to_larger_tile(tmp_path):
    # 128x128 within 1% of the fastest 64x64 time: the larger tile wins
    p = _write(tmp_path, [(64, "64x64x32_w32x32_g8", 100.0), (64, "128x128x32_w64x32_g4", 100.8),
                          (64, "128x128x32_w64x32_g8", 101.5)])
    assert tune.best_by_shape(p)[("gemm", 64, 64, 64)]["config"] == "128x128x32_w64x32_g4"


def test_near_tie_goes_to_larger_group(tmp_path):
    # within the chosen tile, the largest group within 0.5% of its best
    p = _write(tmp_path, [(64, "256x256x32_w128x64_g2", 100.0), (64, "256x256x32_w128x64_g8", 100.3),
                          (64, "256x256x32_w128x64_g4", 100.2), (64, "256x256x32_w128x64_g1", 99.9)])
    assert tune.best_by_shape(p)[("gemm", 64, 64, 64)]["config"] == "256x256x32_w128x64_g8"


def test_outside_tie_window_not_taken(tmp_path):
    p = _write(tmp_path, [(64, "64x64x32_w32x32_g8", 100.0), (64, "128x128x32_w64x32_g8", 101.2)])
    assert tune.best_by_shape(p)[("gemm", 64, 64, 64)]["config"] == "64x64x32_w32x32_g8"
