"""bench.py's command-line contract that can be checked without a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="4")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True,
                       text=True, timeout=120, env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_traffic_record_is_ignored_when_the_kernel_changed(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import json

    import bench
    rec = {"source_hash": "not-the-current-hash", "bytes_per_launch": 123.0}
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    (tmp_path / "sgemm_4092_traffic.json").write_text(json.dumps(rec))
    assert bench.stored_traffic("sgemm_4092", bench.KERNEL_SOURCES) is None
    rec["source_hash"] = bench.source_hash(bench.KERNEL_SOURCES)
    (tmp_path / "sgemm_4092_traffic.json").write_text(json.dumps(rec))
    assert bench.stored_traffic("sgemm_4092", bench.KERNEL_SOURCES) == 123.0
