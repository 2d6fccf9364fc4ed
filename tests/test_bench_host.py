"""Host-side logic of bench.py (no GPU): the refusal of more than one GPU and
the per-launch HBM bytes read from a committed counter summary."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def _summary(tmp_path, monkeypatch, lines, digest="abc"):
    (tmp_path / "traffic_wl.txt").write_text("\n".join(["# header line = ignored"] + lines) + "\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda workload=None: digest)


def test_traffic_of_one_kernel_and_of_a_pair(tmp_path, monkeypatch):
    _summary(tmp_path, monkeypatch, [
        "source_hash = abc",
        "bytes_per_launch.norm_bwd_rows[rms+rope] = 2000",
        "bytes_per_launch.colreduce = 30",
        "bytes_per_launch.rope_apply_kernel = 77",
    ])
    assert bench.read_traffic("rope_apply_kernel", "wl") == 77.0
    # "+" inside the brackets is part of the name; outside it joins kernels
    assert bench.read_traffic("norm_bwd_rows[rms+rope]+colreduce", "wl") == 2030.0
    assert bench.read_traffic("norm_bwd_rows[rms+rope]", "wl") == 2000.0
    # any part missing: unknown
    assert bench.read_traffic("norm_bwd_rows[rms]+colreduce", "wl") is None


def test_traffic_taken_on_other_sources_is_not_used(tmp_path, monkeypatch):
    _summary(tmp_path, monkeypatch, ["source_hash = old", "bytes_per_launch.k = 5"], digest="new")
    assert bench.read_traffic("k", "wl") is None
    assert bench.read_traffic("k", "no_such_workload") is None


def test_operation_mix():
    import bench
    assert bench.op_mix("rmsnorm_bwd") == "2R1W"
    assert bench.op_mix("layernorm_gelu_bwd") == "2R1W"
    assert bench.op_mix("rmsnorm_fwd") == "1R1W"
    assert bench.op_mix("rope_inverse") == "1R1W"


def test_dominant_kernel_counts_launches_and_pairs():
    import bench
    ops = [("a", "k1", None, 10), ("b", "k2+k3", None, 30), ("c", "k1", None, 10)]
    per_op = {"a": dict(ms_mean=1.0), "b": dict(ms_mean=1.5), "c": dict(ms_mean=1.0)}
    name, k = bench.dominant_kernel(ops, per_op)
    assert name == "k1" and k["launches"] == 2 and k["bytes"] == 20 and k["ops"] == ["a", "c"]
    per_op["b"]["ms_mean"] = 2.5
    assert bench.dominant_kernel(ops, per_op)[0] == "k2+k3"
