"""Host-side checks of the benchmark's contract (no GPU): it measures one
GPU and refuses more with a message, and it reports HBM traffic only from a
counter record taken on the current kernel sources."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       env={**os.environ, **env}, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""                              # no JSON line for a refused run


def test_traffic_follows_the_record():
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic_vicuna7b.json")))
    fresh = rec["sources_sha256"] == bench.kernel_sources_sha256()
    for k in ("attn_prefix", "attn_combine", "topk"):
        b = bench.measured_traffic("vicuna7b", k)
        if fresh:
            assert isinstance(b, int) and b > 0
        else:                                          # kernels changed since the counters
            assert b is None
    # the scale factors come from the plain-copy calibration runs
    cal = rec["copy_calibration"]
    kib = cal["bytes_per_launch"] / 1024
    assert cal["fetch_scale"] == pytest.approx(kib / cal["fetch_kib"], rel=1e-3)
    assert cal["write_scale"] == pytest.approx(kib / cal["write_kib"], rel=1e-3)


def test_traffic_is_dropped_when_stale(monkeypatch):
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda: "0" * 64)
    assert bench.measured_traffic("vicuna7b", "attn_prefix") is None
    assert bench.measured_traffic("no_such_workload", "attn_prefix") is None


def test_kernel_trace_summary_names_its_command():
    text = open(os.path.join(ROOT, "profiles", "vicuna7b_step_kernel_trace.md")).read()
    assert "rocprofv3 --kernel-trace --stats" in text and "bench.py" in text
    # the three kernels of a step appear in it
    for name in ("attn_prefix_bf16", "topk_kernel", "attn_combine"):
        assert name in text
