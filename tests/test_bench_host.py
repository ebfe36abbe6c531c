"""Host-side logic of bench.py (no GPU): the traffic figure is taken from the
committed rocprofv3 summary only for the workload and kernel sources it was
measured on, and more than one GPU is refused."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _summary(tmp_path, workload, sha, name="traffic.md"):
    p = tmp_path / name
    p.write_text("# summary\n\nhbm_bytes_per_launch: 1.250000e+10\n"
                 f"workload: {workload}\nkernel_source_sha256: {sha}\n")
    return p


def test_traffic_needs_matching_workload_and_sources(tmp_path, monkeypatch):
    sha = bench.kernel_source_hash()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # kernel_source_hash reads the sources under ROOT: keep the repository's hash
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: sha)
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARIES", {"llama7b_stage4": "traffic.md",
                                                      "llama7b_stage4_fp8": "traffic_fp8.md"})
    _summary(tmp_path, "llama7b_stage4", sha)
    assert bench.measured_traffic("llama7b_stage4") == 1.25e10
    assert bench.measured_traffic("llama70b_slice2") is None
    # the fp8 workload reads its own summary only
    assert bench.measured_traffic("llama7b_stage4_fp8") is None
    (tmp_path / "traffic.md").rename(tmp_path / "traffic_fp8.md")
    assert bench.measured_traffic("llama7b_stage4_fp8") is None  # summary names another workload
    _summary(tmp_path, "llama7b_stage4", sha)
    _summary(tmp_path, "llama7b_stage4_fp8", sha, name="traffic_fp8.md")
    assert bench.measured_traffic("llama7b_stage4_fp8") == 1.25e10
    _summary(tmp_path, "llama7b_stage4", "0" * 16)
    assert bench.measured_traffic("llama7b_stage4") is None
    (tmp_path / "traffic.md").unlink()
    assert bench.measured_traffic("llama7b_stage4") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout


def test_issue_plan_pairs_adjacent_w_only():
    """The bench issues the generator's order as is, except that W(j)
    directly followed by W(j+1) becomes one pair call; every microbatch's
    F, B and W appear exactly once and in the order's positions."""
    import split_backward_amd as zb
    order = zb.schedule_generate("zb", 8, 16, 16, (1, 1, 1), 3)["ops"]
    plan = bench.issue_plan(order)
    assert [("P", 8), ("P", 10), ("P", 12), ("P", 14)] == [op for op in plan if op[0] == "P"]
    expanded = []
    for t, j in plan:
        expanded += [("W", j), ("W", j + 1)] if t == "P" else [(t, j)]
    assert expanded == [tuple(op) for op in order]
    assert bench.issue_plan(order, pair_w=False) == [tuple(op) for op in order]
    # a W followed by a W of a non-adjacent microbatch is not paired
    assert bench.issue_plan([("W", 0), ("W", 2), ("W", 3)]) == [("W", 0), ("P", 2)]
