"""Host-side parts of bench.py, on the CPU: the one-GPU refusal, the CPU
baseline's sampling of the oracle, and the traffic records' validity check."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

from moe_workloads import Workload, make_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "--gpus 2 is not supported" in r.stderr + r.stdout
    assert not r.stdout.strip().startswith("{")  # no result line


@pytest.mark.parametrize("wl", [
    Workload("cpu_bl_f32", T=64, d=128, E=4, k=2, f=128, dtype="f32"),
    Workload("cpu_bl_e4m3", T=64, d=128, E=4, k=2, f=128, dtype="e4m3"),
], ids=lambda w: w.dtype)
def test_cpu_baseline_samples_the_oracle(bench, wl):
    inp = make_inputs(wl, seed=0, device="cpu")
    out = bench.cpu_baseline(wl, inp, budget_s=0.05)
    assert out["unit"] == "TFLOP/s" and out["kind"] == "oracle"
    assert out["value"] is not None and out["value"] > 0
    assert out["cores"] >= 1
    assert f"all {wl.T} tokens" in out["sample"]
    if wl.dtype == "e4m3":
        assert out["sample"].startswith("fp64") and "fp64" not in {k for k in out if k != "sample"}
    else:
        assert out["sample"].startswith("fp32") and out["fp64"]["value"] > 0


def test_traffic_records_follow_the_kernel_sources(bench, tmp_path, monkeypatch):
    wl = Workload("qwen3_bf16", T=8192, d=4096, E=128, k=8, f=1536)
    rec_path = os.path.join(ROOT, "profiles", "traffic_gemm_qwen3_bf16.txt")
    rec = json.loads("".join(ln for ln in open(rec_path) if not ln.startswith("#")))
    # a record taken on the current sources is used
    if rec["kernel_sources_sha256"] == bench.kernel_sources_sha256("bf16"):
        assert bench.gemm_traffic(wl) == rec["hbm_bytes_per_step"]
    # a record of other sources, or none at all, gives no traffic figure
    stale = dict(rec, kernel_sources_sha256="0" * 64)
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic_gemm_qwen3_bf16.txt").write_text(json.dumps(stale))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda dt: "1" * 64)
    assert bench.gemm_traffic(wl) is None
    assert bench.gemm_traffic(Workload("no_record", T=1, d=128, E=1, k=1, f=128)) is None
    # each dtype's record is keyed to its own kernel file
    monkeypatch.undo()
    assert bench.kernel_sources_sha256("bf16") != bench.kernel_sources_sha256("e4m3")
