"""Run in a fresh process by tests/test_gpu_edges.py::test_launch_history_does_not_change_results.

Forward and backward at D = 128 first, then at D = 64 with more work items than
compute units, all into outputs prefilled with NaN.  Asserts that every output
element was written and that the last head of each problem (whose work items are
scheduled last) matches the oracle under the standard per-element bounds.  A
separate script so that the launch history of the process is exactly this one."""

import math
import os
import sys

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)
import io_aware_tiled_fa_amd as fa  # noqa: E402
import oracle  # noqa: E402
from oracle.definition import scale_as_kernel  # noqa: E402
from parity import check  # noqa: E402
from parity_bwd import bounds  # noqa: E402
from parity_bwd import check as check_bwd  # noqa: E402
from workloads import Workload, make_dout, make_inputs  # noqa: E402

dev = torch.device("cuda:0")
dtype = sys.argv[1] if len(sys.argv) > 1 else "bf16"


def run(D, B, H, M, N, causal, seed):
    w = Workload(f"order_{dtype}_d{D}", B, H, M, N, D, dtype, causal, 1 / math.sqrt(D), seed)
    print(f"CASE {w}", flush=True)
    qc, kc, vc = make_inputs(w)
    gc = make_dout(w)
    q, k, v, g = qc.to(dev), kc.to(dev), vc.to(dev), gc.to(dev)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, M), float("nan"), device=dev)
    fa.fwd(q, k, v, causal=causal, scale=w.scale, out=out, lse=lse)
    dq, dk, dv = (torch.full_like(x, float("nan")) for x in (q, k, v))
    fa.bwd(q, k, v, out, lse, g, causal=causal, scale=w.scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for name, t in (("o", out), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        n = int(torch.isnan(t).sum())
        assert n == 0, f"{w.name}: {n} elements of {name} never written"
    h = B * H - 1  # the last head: its items are the last ones scheduled
    q64, k64, v64, g64 = (x.reshape(B * H, -1, D)[h].double().numpy() for x in (qc, kc, vc, gc))
    O_ref, L_ref = oracle.attention(q64, k64, v64, w.scale, causal)
    o_h = out.reshape(B * H, M, D)[h].double().cpu().numpy()
    check(f"{w.name}[head {h}]", dtype, o_h, lse.reshape(B * H, M)[h].cpu().numpy(), O_ref, L_ref)
    s = scale_as_kernel(w.scale)
    rq, rk, rv, parts = oracle.head_bwd(q64, k64, v64, g64, s, causal, return_parts=True)
    bq, bk, bv = bounds(parts, q64, k64, g64, s, dtype)
    for name, got, ref, bnd in (("dq", dq, rq, bq), ("dk", dk, rk, bk), ("dv", dv, rv, bv)):
        check_bwd(f"{w.name}[head {h}] {name}", dtype,
                  got.reshape(B * H, -1, D)[h].double().cpu().numpy(), ref, bnd)


run(128, 1, 64, 1024, 1024, True, 1501)   # D = 128 first: 8-wave persistent kernels
run(64, 4, 16, 1024, 1024, False, 1502)   # then D = 64: 512 forward query tiles
print("ORDER_CASE_OK", flush=True)
