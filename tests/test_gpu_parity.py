"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle on the
seeded workloads, at their full sizes and in the launch configuration the
benchmark times.  Where the oracle cannot cover every row in seconds, it is
run on seeded samples of rows (each row against all N keys)."""

import json
import math

import numpy as np
import pytest

import io_aware_tiled_fa_amd as fa
import oracle
from gpu_calls import nan_fwd
from parity import check
from workloads import WORKLOADS, make_inputs, sample_rows

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"CASE {msg}", flush=True)


def _run(w, qc, kc, vc):
    import torch

    dev = torch.device("cuda:0")
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    o, lse = nan_fwd(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return o, lse


def _flat(x):
    return x.reshape(-1, *x.shape[2:])


def test_worked_example_three_keys():
    """The three-key example through fa_fwd (fp32, D = 1, scale 1): ~25.752 / 3.4076."""
    import torch

    g = json.load(open(__file__.replace("test_gpu_parity.py", "golden/worked_example_three_keys.json")))
    _say("worked example fp32 D=1 M=1 N=3")
    dev = torch.device("cuda:0")
    q = torch.tensor(g["Q"], dtype=torch.float32, device=dev)[None, None]
    k = torch.tensor(g["K"], dtype=torch.float32, device=dev)[None, None]
    v = torch.tensor(g["V"], dtype=torch.float32, device=dev)[None, None]
    o, lse = nan_fwd(q, k, v, scale=g["scale"])
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), g["scale"])
    check("worked_example", "f32", o.cpu().numpy(), lse.cpu().numpy(), O_ref, L_ref)
    assert abs(o.item() - g["final"]["O"]) <= g["tol"]
    assert abs(math.exp(lse.item() - 3.0) - g["final"]["l"]) <= g["tol"]


def test_single_head_f32_full():
    w = WORKLOADS["single_head_f32"]
    _say(f"{w}")
    qc, kc, vc = make_inputs(w)
    o, lse = _run(w, qc, kc, vc)
    O_ref, L_ref = oracle.attention(qc, kc, vc, w.scale, w.causal)
    check(w.name, "f32", o.cpu().numpy(), lse.cpu().numpy(), O_ref, L_ref)


@pytest.mark.parametrize("M,N,D", [(7, 13, 8), (35, 67, 32), (64, 129, 128)])
def test_f32_odd_shapes(M, N, D):
    """The odd single-head fp32 shapes the Triton walkthrough checks."""
    w = WORKLOADS["single_head_f32"].with_(M=M, N=N, D=D, scale=1 / math.sqrt(D), seed=77)
    _say(f"{w}")
    qc, kc, vc = make_inputs(w)
    o, lse = _run(w, qc, kc, vc)
    O_ref, L_ref = oracle.attention(qc, kc, vc, w.scale, False)
    check(f"f32_{M}x{N}x{D}", "f32", o.cpu().numpy(), lse.cpu().numpy(), O_ref, L_ref)


@pytest.mark.parametrize("M,N,D", [(300, 700, 64), (257, 257, 40), (700, 300, 32), (1, 65536, 64),
                                   (5, 1000, 1)])
def test_f32_small_grid_key_split(M, N, D):
    """fp32 grids too small to fill the GPU run with the keys of each workgroup
    split over its waves and merged at the end: causal (bottom-right), several
    128-key steps with a ragged tail, full and padded D, and (M > N) rows that
    see no key at all."""
    w = WORKLOADS["single_head_f32"].with_(B=1, H=2, M=M, N=N, D=D, scale=1 / math.sqrt(D),
                                           causal=True, seed=91)
    _say(f"{w}")
    qc, kc, vc = make_inputs(w)
    o, lse = _run(w, qc, kc, vc)
    O_ref, L_ref = oracle.attention(qc, kc, vc, w.scale, True)
    check(f"f32_split_{M}x{N}x{D}", "f32", o.cpu().numpy(), lse.cpu().numpy(), O_ref, L_ref)


def _sampled_check(w, o, lse, qc, kc, vc, rows_per_head, full_heads=()):
    import torch

    BH = w.B * w.H
    qf, kf, vf = _flat(qc), _flat(kc), _flat(vc)
    rows = np.stack([sample_rows(w.M, h, rows_per_head) for h in range(BH)])
    idx = torch.from_numpy(rows).to(o.device)
    of = o.reshape(BH, w.M, w.D)
    og = torch.gather(of, 1, idx[:, :, None].expand(-1, -1, w.D)).double().cpu().numpy()
    lg = torch.gather(lse.reshape(BH, w.M), 1, idx).cpu().numpy()
    O_ref, L_ref = oracle.attention_rows(qf, kf, vf, w.scale, w.causal, rows)
    check(f"{w.name}[{rows_per_head} rows x {BH} heads]", w.dtype, og, lg, O_ref, L_ref)
    for hh in full_heads:
        O_h, L_h = oracle.attention(qf[hh], kf[hh], vf[hh], w.scale, w.causal)
        check(f"{w.name}[head {hh} all rows]", w.dtype, of[hh].double().cpu().numpy(),
              lse.reshape(BH, w.M)[hh].cpu().numpy(), O_h, L_h)


def test_gpt2_medium_f16():
    w = WORKLOADS["gpt2_medium_f16"]
    _say(f"{w}")
    qc, kc, vc = make_inputs(w)
    o, lse = _run(w, qc, kc, vc)
    _sampled_check(w, o, lse, qc, kc, vc, 48, full_heads=(0, 517, 1023))


def test_causal_prefill_bf16():
    w = WORKLOADS["causal_prefill_bf16"]
    _say(f"{w}")
    qc, kc, vc = make_inputs(w)
    o, lse = _run(w, qc, kc, vc)
    _sampled_check(w, o, lse, qc, kc, vc, 48, full_heads=(255,))


@pytest.mark.parametrize("name", ["stress_f16", "stress_f16_causal", "stress_f16_causal_mgtn"])
def test_stress_f16_all_rows(name):
    w = WORKLOADS[name]
    _say(f"{w}")
    qc, kc, vc = make_inputs(w)
    o, lse = _run(w, qc, kc, vc)
    O_ref, L_ref = oracle.attention(qc, kc, vc, w.scale, w.causal)
    check(w.name, w.dtype, o.double().cpu().numpy(), lse.cpu().numpy(), O_ref, L_ref)


def test_persistent_launch_all_rows():
    """More (head, query tile) items than workgroups (persistent schedule),
    with an item count (333) that does not divide evenly over the XCDs."""
    from workloads import Workload

    w = Workload(name="persistent_bf16_d128", B=3, H=37, M=600, N=600, D=128, dtype="bf16",
                 causal=False, scale=1.0 / math.sqrt(128), seed=1101)
    _say(f"{w}")
    qc, kc, vc = make_inputs(w)
    o, lse = _run(w, qc, kc, vc)
    O_ref, L_ref = oracle.attention(_flat(qc), _flat(kc), _flat(vc), w.scale, w.causal)
    check(w.name, w.dtype, _flat(o.double()).cpu().numpy(), _flat(lse).cpu().numpy(), O_ref, L_ref)


def test_long_context_bf16_sampled():
    w = WORKLOADS["long_context_bf16"]
    _say(f"{w}")
    qc, kc, vc = make_inputs(w)
    o, lse = _run(w, qc, kc, vc)
    _sampled_check(w, o, lse, qc, kc, vc, 256)
