"""Host-side logic of bench.py (no GPU): the traffic figure is taken from the
committed rocprofv3 summary only for the workload and kernel sources it was
measured on, and more than one GPU is refused."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _summary(tmp_path, workload, sha):
    p = tmp_path / "traffic.md"
    p.write_text("# summary\n\nhbm_bytes_per_launch: 1.250000e+10\n"
                 f"workload: {workload}\nkernel_source_sha256: {sha}\n")
    return p


def test_traffic_needs_matching_workload_and_sources(tmp_path, monkeypatch):
    sha = bench.kernel_source_hash()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # kernel_source_hash reads the sources under ROOT: keep the repository's hash
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: sha)
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", "traffic.md")
    _summary(tmp_path, "llama7b_stage4", sha)
    assert bench.measured_traffic("llama7b_stage4") == 1.25e10
    assert bench.measured_traffic("llama70b_slice2") is None
    _summary(tmp_path, "llama7b_stage4", "0" * 16)
    assert bench.measured_traffic("llama7b_stage4") is None
    (tmp_path / "traffic.md").unlink()
    assert bench.measured_traffic("llama7b_stage4") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout
