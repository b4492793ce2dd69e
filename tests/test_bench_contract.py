"""Host-side checks of the benchmark's contract (no GPU): it measures one
GPU and refuses more with a message, it defaults to the large-vocabulary
batch, and it reports HBM traffic and matrix-core counters only from a
record taken on the current sources of the kernel concerned."""
import glob
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

PROFILES = os.path.join(ROOT, "profiles")


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       env={**os.environ, **env}, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""                              # no JSON line for a refused run


def test_default_workload_is_the_large_vocabulary_batch(monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert a.workload == "largevocab" and a.gpus == 1 and not a.no_cold


def _records(kind):
    return sorted(glob.glob(os.path.join(PROFILES, f"{kind}_*.json")))


def test_traffic_follows_the_record():
    recs = _records("traffic")
    assert any(p.endswith("traffic_largevocab.json") for p in recs)
    for path in recs:
        workload = os.path.basename(path)[len("traffic_"):-len(".json")]
        rec = json.load(open(path))
        for kernel, (prefix, _) in bench.KERNEL_SOURCES.items():
            fresh = rec["sources_sha256"].get(prefix) == bench.kernel_sources_sha256(kernel)
            b = bench.measured_traffic(workload, kernel)
            if fresh and prefix in rec["per_kernel"]:
                assert isinstance(b, int) and b > 0
            else:                                      # the kernel changed since the counters
                assert b is None
        # the scale factors come from the plain-copy calibration runs
        cal = rec["copy_calibration"]
        kib = cal["bytes_per_launch"] / 1024
        assert cal["fetch_scale"] == pytest.approx(kib / cal["fetch_kib"], rel=1e-3)
        assert cal["write_scale"] == pytest.approx(kib / cal["write_kib"], rel=1e-3)
        assert "rocprofv3 --pmc FETCH_SIZE" in rec["commands"]["fetch"]


def test_mfma_record_is_consistent():
    recs = _records("mfma")
    assert any(p.endswith("mfma_largevocab.json") for p in recs)
    for path in recs:
        rec = json.load(open(path))
        simds = rec["simds"]
        for prefix, k in rec["per_kernel"].items():
            # busy fraction = MFMA busy cycles / (active cycles x SIMDs)
            assert k["busy_frac"] == pytest.approx(
                k["SQ_VALU_MFMA_BUSY_CYCLES"] / (k["GRBM_GUI_ACTIVE"] * simds), rel=1e-3)
            assert k["mops_flops"] == pytest.approx(k["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512, rel=1e-6)
            assert 0 <= k["busy_frac"] <= 1
        assert "SQ_VALU_MFMA_BUSY_CYCLES" in rec["command"]


def test_records_are_dropped_when_stale(monkeypatch):
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda kernel: "0" * 64)
    assert bench.measured_traffic("largevocab", "attn_prefix") is None
    assert bench.measured_mfma("largevocab", "attn_prefix") is None
    assert bench.measured_traffic("no_such_workload", "attn_prefix") is None


def test_kernel_trace_summaries_name_their_command():
    paths = sorted(glob.glob(os.path.join(PROFILES, "*_kernel_trace.md")))
    assert any("largevocab" in os.path.basename(p) for p in paths)
    for path in paths:
        text = open(path).read()
        assert "rocprofv3 --kernel-trace --stats" in text and "bench.py" in text
        # the three kernels of a step appear in it (the top-k launch is the
        # few-row step kernel on the single-sequence workloads)
        for name in ("attn_prefix_bf16", "attn_merge_bf16"):
            assert name in text, (path, name)
        assert "topk_kernel" in text or "step_kernel" in text, path


def test_top_k_launch_maps_to_its_kernel_record():
    from synth import workloads as W
    assert bench.record_kernel(W.WORKLOADS["vicuna7b"], "topk") == "step"
    assert bench.record_kernel(W.WORKLOADS["codellama34b"], "topk") == "step"
    assert bench.record_kernel(W.WORKLOADS["largevocab"], "topk") == "topk"     # 2592 rows
    assert bench.record_kernel(W.WORKLOADS["vicuna7b"], "attn_prefix") == "attn_prefix"
