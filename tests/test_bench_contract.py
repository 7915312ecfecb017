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
    assert cb["cpu_model"] and cb["blas"]


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


def test_kernel_label_follows_the_dispatch_rules():
    """roofline.kernel names what fa_fwd / fa_fwd_splitkv launch: the pipelined
    kernel for 16-bit D in {64, 96, 128} and, zero-padded, the other multiples
    of 8 except 32 (split-KV too), else the general or fp32 kernels (the fp32
    key-split kernel only for small plain grids)."""
    sys.path.insert(0, ROOT)
    import bench
    from workloads import WORKLOADS

    pipe = "fa_fwd_lp_pipe_kernel"
    w = WORKLOADS["causal_prefill_bf16"]
    assert bench.fwd_kernel_name(w) == pipe
    assert bench.fwd_kernel_name(w, splits=4) == pipe + " + fa_merge_kernel (split-KV)"
    for D in (64, 96):
        assert bench.fwd_kernel_name(w.with_(D=D), splits=2).startswith(pipe)
    for D in (8, 40, 112):
        assert bench.fwd_kernel_name(w.with_(D=D)) == pipe
        assert bench.fwd_kernel_name(w.with_(D=D), splits=2).startswith(pipe)
    assert bench.fwd_kernel_name(w.with_(D=32)) == "fa_fwd_lp_kernel"
    assert bench.fwd_kernel_name(w.with_(D=100)) == "fa_fwd_lp_kernel"
    assert bench.fwd_kernel_name(w.with_(D=100), splits=3).startswith("fa_fwd_lp_kernel +")
    f32 = WORKLOADS["single_head_f32"]
    assert bench.fwd_kernel_name(f32, cus=256) == "fa_fwd_f32_ksplit_kernel"
    assert bench.fwd_kernel_name(f32.with_(B=64, H=16), cus=256) == "fa_fwd_f32_kernel"
    assert bench.fwd_kernel_name(f32, splits=8).startswith("fa_fwd_f32_kernel +")


def test_sclk_sampler_parses_the_current_level(tmp_path):
    sys.path.insert(0, ROOT)
    import bench

    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 1600Mhz\n2: 2100Mhz *\n3: 2400Mhz\n")
    s = bench.SclkSampler()
    s.paths = [str(f)]
    assert s._read() == 2100.0
    s.samples = [2100.0, 2000.0, 2200.0]
    assert s.summary()["median_mhz"] == 2100.0
    s.paths = [str(tmp_path / "absent")]
    assert s._read() is None
