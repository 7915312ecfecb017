#!/usr/bin/env python3
"""Throughput of the attention forward pass (fa_fwd) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--pass fwd|bwd]

A step is one fa_fwd call over the whole batch of the workload: the complete
hot path (Q tile load, K/V streaming through LDS, both MFMA products, online
softmax, epilogue) with Q, K and V already resident in HBM.  W untimed warmup
steps, then exactly K timed steps between two device synchronisations.  One JSON
line goes to stdout; progress goes to stderr.

FLOP accounting: the headline value uses 4*B*H*M*N*D, halved for causal.  The
roofline object uses the algorithmic count, 4*D FLOP per visible (query, key)
pair, over the average duration of one launch measured with HIP events on the
stream the kernel runs on.  Peak: MI355X dense bf16/fp16 MFMA 2516.6 TFLOP/s
(fp32 MFMA 157.3 TFLOP/s for fp32 inputs).

The cpu_baseline object times the fp64 CPU oracle (untuned) on a bounded sample
of the same workload (whole heads, all rows) on this host's cores.

``--sdpa`` times PyTorch's own fused scaled_dot_product_attention (its flash or
memory-efficient backend; never the math path) on the same inputs, as context
only: another party's implementation, not a target.  Causal calls need M = N
(PyTorch aligns its causal mask top-left).

``--pass bwd`` times fa_bwd instead (the forward runs once before the timed
region and its O and LSE are inputs, as in training).  Its algorithmic work is
the pages' count for a backward pass with recomputation, five products of
2*D FLOP per visible (query, key) pair (QK^T again, dP, dV, dQ, dK); the
kernels execute seven (S and dP are recomputed once more for dQ), which the
config records.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from workloads import (BENCH_WORKLOAD, WORKLOADS, compulsory_bytes, exact_flops,  # noqa: E402
                       make_inputs, metric_flops)

PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}
HBM_PEAK_GBS = 8000.0
METRIC = "attn fwd TFLOP/s + % of MI355X MFMA peak (N=4096 d=128 causal bf16)"
METRIC_BWD = "attn bwd TFLOP/s (5 products per pair) + % of MI355X MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_info():
    """CPU model and BLAS library the oracle's timing ran with."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info

        libs = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info()
                if i.get("user_api") == "blas"]
        if libs:
            blas = ", ".join(libs)
    except Exception:  # noqa: BLE001
        pass
    return {"cpu_model": model, "blas": blas}


def cpu_baseline(w, qc, kc, vc, budget_s: float = 15.0, max_heads: int = 1 << 30):
    """Time the fp64 oracle on whole heads of the workload until ~budget_s."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    qf = qc.reshape(-1, w.M, w.D)
    kf = kc.reshape(-1, w.N, w.D)
    vf = vc.reshape(-1, w.N, w.D)
    # widen one head at a time inside the timed loop (part of the oracle's work)
    t0 = time.perf_counter()
    done = 0
    for h in range(min(max_heads, qf.shape[0])):
        oracle.attention(qf[h], kf[h], vf[h], w.scale, w.causal)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    fl = metric_flops(1, done, w.M, w.N, w.D, w.causal)
    return {
        "value": fl / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} of {w.B * w.H} heads, all {w.M} rows, fp64 numpy, "
                  f"{dt:.1f} s wall ({os.cpu_count()} cpus visible)",
        **host_info(),
    }


def cpu_baseline_bwd(w, qc, kc, vc, gc, budget_s: float = 15.0):
    """Time the fp64 oracle's backward on whole heads until ~budget_s."""
    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    qf, kf = qc.reshape(-1, w.M, w.D), kc.reshape(-1, w.N, w.D)
    vf, gf = vc.reshape(-1, w.N, w.D), gc.reshape(-1, w.M, w.D)
    t0 = time.perf_counter()
    done = 0
    for h in range(qf.shape[0]):
        oracle.attention_bwd(qf[h], kf[h], vf[h], gf[h], w.scale, w.causal)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    fl = 2.5 * exact_flops(1, done, w.M, w.N, w.D, w.causal)
    return {
        "value": fl / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} of {w.B * w.H} heads, all {w.M} rows, fp64 numpy backward, "
                  f"{dt:.1f} s wall ({os.cpu_count()} cpus visible)",
        **host_info(),
    }


def fwd_kernel_name(w, splits=0, cus=None):
    """The forward kernel(s) one fa_fwd (splits = 0) or fa_fwd_splitkv call
    launches for workload w, by the dispatch rules of fa_fwd.hip: fp16/bf16
    with D in {64, 96, 128}, or a multiple of 8 other than 32 (zero-padded to
    the next of those), run the pipelined direct-to-LDS kernel (split-KV too),
    other 16-bit head dims the general kernel, fp32 the fp32 kernel (the
    key-split one for small plain grids)."""
    if w.dtype == "f32":
        if splits:
            name = "fa_fwd_f32_kernel"
        else:
            if cus is None:
                import torch

                cus = torch.cuda.get_device_properties(0).multi_processor_count
            grid = w.B * w.H * ((w.M + 127) // 128)
            name = ("fa_fwd_f32_ksplit_kernel" if w.D <= 64 and w.N > 0 and 2 * grid < cus
                    else "fa_fwd_f32_kernel")
    elif w.N > 0 and w.D % 8 == 0 and w.D != 32:
        name = "fa_fwd_lp_pipe_kernel"
    else:
        name = "fa_fwd_lp_kernel"
    return name + " + fa_merge_kernel (split-KV)" if splits and w.N > 0 else name


class SclkSampler:
    """Samples the GPU's current shader clock (MHz) from the driver's sysfs
    table (the level marked '*' in pp_dpm_sclk) on a background thread while
    the timed batches run; `summary()` gives the median and range, or None
    where the file is not readable."""

    def __init__(self, period_s: float = 0.01):
        import glob
        import threading

        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.samples = []
        self.period = period_s
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        vals = []
        for p in self.paths:
            try:
                for line in open(p):
                    if line.rstrip().endswith("*"):
                        vals.append(float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0]))
            except (OSError, ValueError, IndexError):
                continue
        return max(vals) if vals else None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.paths:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        xs = sorted(self.samples)
        return {"median_mhz": xs[len(xs) // 2], "min_mhz": xs[0], "max_mhz": xs[-1],
                "samples": len(xs), "source": "sysfs pp_dpm_sclk (current level)"}


def timed_batches(step, stream, est_ms: float, batches: int = 5, min_batch_ms: float = 100.0):
    """The timing procedure for the reported distribution: `batches` batches of
    R back-to-back launches each, R chosen so a batch lasts at least
    min_batch_ms, each timed with HIP events on the launch stream.  Returns the
    per-launch mean of every batch (ms), R, and the clock sampled meanwhile."""
    import torch

    R = max(1, int(math.ceil(min_batch_ms / max(est_ms, 1e-6))))
    per = []
    with SclkSampler() as clk:
        for _ in range(batches):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(R):
                step()
            b.record(stream)
            torch.cuda.synchronize()
            per.append(a.elapsed_time(b) / R)
    return per, R, clk.summary()


def load_traffic(w, key=None, source="fa_fwd.hip"):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match:
    the record under ``key`` (default: the workload's name) in profiles/traffic.json,
    taken while ``source`` had the digest stored with it."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        rec = json.load(open(TRAFFIC_FILE)).get(key or w.name)
    except Exception:  # noqa: BLE001
        return None
    if not rec:
        return None
    src = os.path.join(ROOT, "io_aware_tiled_fa_amd", "csrc", source)
    import hashlib

    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    if rec.get("source_sha256_16") != digest:
        return None  # the kernel changed since the counters were taken
    return rec.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=BENCH_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--batches", type=int, default=5,
                    help="timed batches after the K steps (median and minimum are reported)")
    ap.add_argument("--batch-ms", type=float, default=100.0,
                    help="minimum duration of one timed batch (launches per batch follow)")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd"), default="fwd",
                    help="time the forward (default, the headline metric) or the backward pass")
    ap.add_argument("--splits", type=int, default=0,
                    help="forward only: time fa_fwd_splitkv with this many key chunks "
                         "(0: plain fa_fwd, the headline path)")
    ap.add_argument("--seq", type=int, default=0, metavar="S",
                    help="measurement sweeps: run the workload with M = N = S (the driver's "
                         "line uses the workload's own sizes)")
    ap.add_argument("--batch", type=int, default=0, metavar="B",
                    help="measurement sweeps: run the workload with this batch size")
    ap.add_argument("--sdpa", action="store_true",
                    help="context only: time PyTorch's fused SDPA (flash / memory-efficient "
                         "backend) on the same workload instead of fa_fwd")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="instead of attention, run a plain device-to-device copy of BYTES "
                         "(3 times); used to scale the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: every (batch, head) of the attention forward "
              "pass is independent, so a multi-GPU run would shard heads with no communication, "
              "and this benchmark reports the one-GPU share. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import io_aware_tiled_fa_amd as fa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {4 * n} bytes 3 times")
        return
    fa.load()
    w = WORKLOADS[args.workload]
    if args.seq or args.batch:
        B = args.batch or w.B
        M = args.seq or w.M
        N = args.seq or w.N
        w = w.with_(name=f"{w.name}_B{B}_M{M}_N{N}", B=B, M=M, N=N)
    if args.which == "bwd":
        return bench_bwd(args, w)
    if args.sdpa:
        return bench_sdpa(args, w)
    dev = torch.device("cuda:0")
    log(f"workload {w}")
    qc, kc, vc = make_inputs(w)
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.M), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    code = {"f32": fa.DTYPE_F32, "f16": fa.DTYPE_F16, "bf16": fa.DTYPE_BF16}[w.dtype]
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr())
    if args.splits:
        wsb = fa.fa_splitkv_workspace_bytes(w.B, w.H, w.M, w.D, args.splits)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)

        def step():
            st = fa.fa_fwd_splitkv(*ptrs, w.B, w.H, w.M, w.N, w.D, w.scale, int(w.causal), code,
                                   args.splits, ws.data_ptr(), wsb, stream.cuda_stream)
            if st != 0:
                raise fa.FaError(st, "fa_fwd_splitkv")
    else:
        def step():
            st = fa.fa_fwd(*ptrs, w.B, w.H, w.M, w.N, w.D, w.scale, int(w.causal), code,
                           stream.cuda_stream)
            if st != 0:
                raise fa.FaError(st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(K):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    ms_per_step = total_ms / K
    avg_launch_ms = sum(launch_ms) / K
    med_launch_ms = sorted(launch_ms)[K // 2]

    fl_metric = metric_flops(w.B, w.H, w.M, w.N, w.D, w.causal)
    fl_exact = exact_flops(w.B, w.H, w.M, w.N, w.D, w.causal)
    tflops = fl_metric / (ms_per_step * 1e-3) / 1e12
    log(f"timed batches (>= 5 x >= {args.batch_ms:.0f} ms) ...")
    per_batch, R, sclk = timed_batches(step, stream, avg_launch_ms, args.batches, args.batch_ms)
    med_batch = sorted(per_batch)[len(per_batch) // 2]
    peak = PEAK_TFLOPS[w.dtype]
    achieved = fl_exact / (avg_launch_ms * 1e-3) / 1e12
    traffic = None if args.splits else load_traffic(w)
    log(f"ms/step {ms_per_step:.4f}  avg launch {avg_launch_ms:.4f} ms  median {med_launch_ms:.4f} ms  "
        f"{tflops:.1f} TFLOP/s ({100 * tflops / peak:.1f}% of {peak} peak)  wall {wall:.3f}s")
    log(f"batches of {R}: median {med_batch:.4f} ms/launch ({fl_metric / (med_batch * 1e-3) / 1e12:.1f} "
        f"TFLOP/s), min {min(per_batch):.4f} ms; sclk {sclk}")

    out = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1), see workloads)",
        "pct_of_mfma_peak": round(100.0 * tflops / peak, 2),
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "M": w.M, "N": w.N, "D": w.D,
            "causal": w.causal, "scale": w.scale, "splits": args.splits, "flop_metric": fl_metric,
            "flop_visible_pairs": fl_exact, "compulsory_bytes": compulsory_bytes(w),
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "kernel": fwd_kernel_name(w, args.splits),
            "avg_launch_ms": round(avg_launch_ms, 5),
            "median_launch_ms": round(med_launch_ms, 5),
            "min_launch_ms": round(min(launch_ms), 5),
            "hbm_gbs_compulsory": round(compulsory_bytes(w) / (avg_launch_ms * 1e-3) / 1e9, 1),
        },
        "timing": {
            "procedure": f"{len(per_batch)} batches of {R} back-to-back launches after the K "
                         "timed steps, HIP events on the launch stream, per-launch mean per batch",
            "batches": len(per_batch), "launches_per_batch": R,
            "batch_ms_per_launch": [round(x, 5) for x in per_batch],
            "median_ms": round(med_batch, 5), "min_ms": round(min(per_batch), 5),
            "median_tflops": round(fl_metric / (med_batch * 1e-3) / 1e12, 3),
            "sclk": sclk,
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(w, qc, kc, vc, budget_s=args.cpu_budget)
    print(json.dumps(out), flush=True)


def bench_sdpa(args, w):
    """Context: PyTorch's fused SDPA forward on the workload, timed like fa_fwd."""
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel

    import io_aware_tiled_fa_amd as fa

    if w.dtype == "f32" or (w.causal and w.M != w.N):
        print("--sdpa covers fp16/bf16 workloads, causal ones only with M = N (PyTorch aligns "
              "its causal mask top-left)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    log(f"workload {w} (PyTorch SDPA, context)")
    qc, kc, vc = make_inputs(w)
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    backend = None
    for b in (SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION):
        try:
            with sdpa_kernel(b):
                o_ref = F.scaled_dot_product_attention(q, k, v, is_causal=w.causal, scale=w.scale)
            torch.cuda.synchronize()
            backend = b
            break
        except RuntimeError as e:  # backend not built for this GPU or shape: try the next
            log(f"{b.name}: unavailable ({str(e).splitlines()[0][:120]})")
    if backend is None:
        print(json.dumps({"metric": "context: PyTorch SDPA forward", "value": None,
                          "note": "no fused SDPA backend available", "torch": torch.__version__}))
        return
    o_fa, _ = fa.fwd(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    diff = (o_fa.float() - o_ref.float()).abs().max().item()
    stream = torch.cuda.current_stream(dev)

    def step():
        with sdpa_kernel(backend):
            F.scaled_dot_product_attention(q, k, v, is_causal=w.causal, scale=w.scale)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for _ in range(K):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / K
    peak = PEAK_TFLOPS[w.dtype]
    tflops = metric_flops(w.B, w.H, w.M, w.N, w.D, w.causal) / (ms * 1e-3) / 1e12
    log(f"SDPA ({backend.name}) ms/step {ms:.4f}  {tflops:.1f} TFLOP/s  max|O_sdpa - O_fa_fwd| {diff:.3e}")
    print(json.dumps({
        "metric": "context: PyTorch SDPA forward TFLOP/s on the same workload (not a target)",
        "value": round(tflops, 3), "unit": "TFLOP/s", "ms_per_step": round(ms, 5),
        "pct_of_mfma_peak": round(100.0 * tflops / peak, 2), "steps": K, "warmup": args.warmup,
        "backend": backend.name, "torch": torch.__version__,
        "max_abs_diff_vs_fa_fwd": diff, "config": {"workload": w.name, "B": w.B, "H": w.H,
                                                   "M": w.M, "N": w.N, "D": w.D,
                                                   "causal": w.causal, "dtype": w.dtype},
    }), flush=True)


def bench_bwd(args, w):
    import torch

    import io_aware_tiled_fa_amd as fa
    from workloads import make_dout

    dev = torch.device("cuda:0")
    log(f"workload {w} (backward)")
    qc, kc, vc = make_inputs(w)
    gc = make_dout(w)
    q, k, v, g = qc.to(dev), kc.to(dev), vc.to(dev), gc.to(dev)
    o, lse = fa.fwd(q, k, v, causal=w.causal, scale=w.scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((2, w.B, w.H, w.M), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    code = {"f32": fa.DTYPE_F32, "f16": fa.DTYPE_F16, "bf16": fa.DTYPE_BF16}[w.dtype]
    ptrs = tuple(t.data_ptr() for t in (q, k, v, o, lse, g, dq, dk, dv, delta))

    def step():
        st = fa.fa_bwd(*ptrs, w.B, w.H, w.M, w.N, w.D, w.scale, int(w.causal), code,
                       stream.cuda_stream)
        if st != 0:
            raise fa.FaError(st, "fa_bwd")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(K):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / K
    avg_launch_ms = sum(a.elapsed_time(b) for a, b in ev) / K
    fl_alg = 2.5 * exact_flops(w.B, w.H, w.M, w.N, w.D, w.causal)   # 5 products
    fl_exec = 3.5 * exact_flops(w.B, w.H, w.M, w.N, w.D, w.causal)  # 7 products
    peak = PEAK_TFLOPS[w.dtype]
    tflops = fl_alg / (ms_per_step * 1e-3) / 1e12
    achieved = fl_alg / (avg_launch_ms * 1e-3) / 1e12
    log(f"bwd ms/step {ms_per_step:.4f}  avg call {avg_launch_ms:.4f} ms  {tflops:.1f} TFLOP/s "
        f"algorithmic ({100 * tflops / peak:.1f}% of peak), "
        f"{fl_exec / (avg_launch_ms * 1e-3) / 1e12:.1f} TFLOP/s executed")
    out = {
        "metric": METRIC_BWD, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs and incoming gradient, see workloads)",
        "pct_of_mfma_peak": round(100.0 * tflops / peak, 2),
        "config": {
            "workload": w.name, "pass": "bwd", "B": w.B, "H": w.H, "M": w.M, "N": w.N, "D": w.D,
            "causal": w.causal, "flop_algorithmic": fl_alg, "flop_executed": fl_exec,
        },
        "roofline": {
            "bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": load_traffic(w, key=w.name + "/bwd", source="fa_bwd.hip"),
            "kernel": ("fa_bwd (fp32: delta + dkdv + dq kernels on 32x32x2 fp32 MFMA, one call)"
                       if w.dtype == "f32" else "fa_bwd (delta + dkdv + dq kernels, one call)"),
            "avg_launch_ms": round(avg_launch_ms, 5),
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle backward on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline_bwd(w, qc, kc, vc, gc, budget_s=args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
