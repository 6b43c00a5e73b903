"""bench.py's contract on the host: more than one GPU is refused with a
message, and a traffic summary taken on another kernel source is ignored."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_needs_matching_kernel_source(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    f.write_text("# test\ngemm_source_sha256: %s\nhbm_bytes_per_gemm_call: 123.0\n" % ("0" * 64))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_from_profile() is None
    f.write_text("gemm_source_sha256: %s\nhbm_bytes_per_gemm_call: 123.0\n" % bench.gemm_source_sha())
    assert bench.traffic_from_profile() == 123.0
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.txt"))
    assert bench.traffic_from_profile() is None
