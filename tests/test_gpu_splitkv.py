"""Parity of the split-KV forward (fa_fwd_splitkv through the C ABI) with the
fp64 oracle, under the same per-element tolerance as fa_fwd (tests/parity.py),
on seeded inputs: few query tiles and long key runs (the case it exists for),
every dtype, both mask modes, empty rows, more splits than key tiles."""

import numpy as np
import pytest

import io_aware_tiled_fa_amd as fa
import oracle
from gpu_calls import nan_fwd
from parity import check
from workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"CASE {msg}", flush=True)


def _wl(name, B, H, M, N, D, dtype, causal, seed, q_mult=1.0):
    return Workload(name=name, B=B, H=H, M=M, N=N, D=D, dtype=dtype, causal=causal,
                    scale=1.0 / np.sqrt(D), seed=seed, q_mult=q_mult)


def _run_split(w, splits, ws=None):
    import torch

    dev = torch.device("cuda:0")
    qc, kc, vc = make_inputs(w)
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    if ws is None:
        o, lse = nan_fwd(q, k, v, causal=w.causal, scale=w.scale, splits=splits)
    else:
        o, lse = fa.fwd(q, k, v, causal=w.causal, scale=w.scale, splits=splits, workspace=ws)
    torch.cuda.synchronize()
    return qc, kc, vc, o.cpu(), lse.cpu()


def _flat(x):
    return x.reshape(-1, *x.shape[2:])


CASES = [
    (WORKLOADS["single_head_f32"], 1),
    (WORKLOADS["single_head_f32"], 2),
    (WORKLOADS["single_head_f32"], 16),
    (_wl("split_bf16_causal_long_keys", 1, 2, 300, 4000, 128, "bf16", True, 4101), 8),
    (_wl("split_f16_d65", 1, 2, 200, 1500, 65, "f16", False, 4102), 5),
    (_wl("split_f16_stress_causal", 1, 2, 1000, 3000, 96, "f16", True, 4103, q_mult=8.0), 12),
    (_wl("split_bf16_empty_rows", 1, 2, 700, 300, 64, "bf16", True, 4104), 3),
    (_wl("split_f32_more_splits_than_tiles", 1, 1, 50, 100, 32, "f32", False, 4105), 64),
    (_wl("split_f16_d1", 1, 1, 33, 777, 1, "f16", True, 4106), 7),
    # decode shape: one query row against 64K keys per head
    (_wl("split_bf16_decode_64k", 2, 8, 1, 65536, 128, "bf16", False, 4107), 32),
    # a short causal block at the end of a long context (bottom-right mask)
    (_wl("split_f16_causal_tail_32k", 1, 4, 16, 32768, 64, "f16", True, 4108), 16),
]


@pytest.mark.parametrize("w,splits", CASES, ids=[f"{w.name}-s{s}" for w, s in CASES])
def test_splitkv_matches_oracle(w, splits):
    _say(f"{w} splits={splits}")
    qc, kc, vc, o, lse = _run_split(w, splits)
    O_ref, L_ref = oracle.attention(_flat(qc), _flat(kc), _flat(vc), w.scale, w.causal)
    check(f"{w.name}-splits{splits}", w.dtype, _flat(o.double()).numpy(), _flat(lse).numpy(),
          O_ref, L_ref)


def test_splitkv_reuses_one_workspace_and_is_deterministic():
    import torch

    w = _wl("split_reuse_bf16", 1, 4, 128, 2048, 128, "bf16", True, 4110)
    _say(f"{w} splits 8 then 3 on one workspace, twice")
    need = fa.fa_splitkv_workspace_bytes(w.B, w.H, w.M, w.D, 8)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda:0")  # NaN bit patterns
    _, _, _, o8, l8 = _run_split(w, 8, ws)
    qc, kc, vc, o3, l3 = _run_split(w, 3, ws)
    _, _, _, o8b, l8b = _run_split(w, 8, ws)
    assert torch.equal(o8, o8b) and torch.equal(l8, l8b)
    O_ref, L_ref = oracle.attention(_flat(qc), _flat(kc), _flat(vc), w.scale, w.causal)
    for o, lse, s in ((o8, l8, 8), (o3, l3, 3)):
        check(f"{w.name}-s{s}", w.dtype, _flat(o.double()).numpy(), _flat(lse).numpy(), O_ref, L_ref)


def test_splitkv_rejects_small_workspace():
    import torch

    w = _wl("split_small_ws", 1, 1, 64, 512, 64, "f16", False, 4111)
    need = fa.fa_splitkv_workspace_bytes(w.B, w.H, w.M, w.D, 4)
    ws = torch.empty(need - 4, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(fa.FaError) as e:
        _run_split(w, 4, ws)
    assert e.value.status == 9
