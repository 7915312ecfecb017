"""bench.py's driver contract: one JSON line with the required keys, one GPU only."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.gpu
def test_bench_prints_one_contract_line():
    r = subprocess.run([sys.executable, BENCH, "--workload", "single_head_f32", "--steps", "3",
                        "--warmup", "1", "--cpu-budget", "0.5"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"] == "single_head_f32"
    rl = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in rl, key
    assert 0 < rl["frac"] < 1 and abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]


def test_traffic_is_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    """roofline.traffic comes from profiles/traffic.json only while the kernel
    source still has the digest recorded with the counters; otherwise null."""
    import hashlib

    sys.path.insert(0, ROOT)
    import bench
    from workloads import WORKLOADS

    w = WORKLOADS["causal_prefill_bf16"]
    src = os.path.join(ROOT, "io_aware_tiled_fa_amd", "csrc", "fa_fwd.hip")
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({w.name: {"bytes_per_launch": 123, "source_sha256_16": digest},
                             "other": {"bytes_per_launch": 7, "source_sha256_16": "0" * 16}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.load_traffic(w) == 123
    assert bench.load_traffic(w, key="other") is None          # stale digest
    assert bench.load_traffic(w, key="missing") is None
    assert bench.load_traffic(w, source="fa_bwd.hip") is None  # digest of another file
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.json"))
    assert bench.load_traffic(w) is None
