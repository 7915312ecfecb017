"""fa_fwd_splitkv_noalloc (static device scratch, no allocation) through the C
ABI against fa_fwd_splitkv with a caller workspace (the same kernels: the
results must be bit-identical) and against the fp64 oracle under the standard
per-element bounds, on two calls in a row, the second one smaller, both into
NaN-filled outputs."""

import math

import numpy as np
import pytest

import io_aware_tiled_fa_amd as fa
import oracle
from parity import check
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

CODE = {"f32": fa.DTYPE_F32, "f16": fa.DTYPE_F16, "bf16": fa.DTYPE_BF16}


def _flat(x):
    return x.reshape(-1, *x.shape[2:])


def _run_both(w, splits):
    import torch

    dev = torch.device("cuda:0")
    qc, kc, vc = make_inputs(w)
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    o1 = torch.full_like(q, math.nan)
    l1 = torch.full((w.B, w.H, w.M), math.nan, device=dev)
    o2 = torch.full_like(q, math.nan)
    l2 = torch.full((w.B, w.H, w.M), math.nan, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (w.B, w.H, w.M, w.N, w.D, w.scale, int(w.causal), CODE[w.dtype], splits)
    st = fa.fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o1.data_ptr(),
                                   l1.data_ptr(), *args, stream)
    assert st == 0, fa.fa_status_string(st)
    need = fa.fa_splitkv_workspace_bytes(w.B, w.H, w.M, w.D, splits)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=dev)
    st = fa.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(),
                           *args, ws.data_ptr(), need, stream)
    assert st == 0, fa.fa_status_string(st)
    torch.cuda.synchronize()
    return qc, kc, vc, o1, l1, o2, l2


@pytest.mark.parametrize("first,second", [
    ((Workload("noalloc_bf16_causal", 1, 4, 256, 4000, 128, "bf16", True, 1 / math.sqrt(128), 6101), 8),
     (Workload("noalloc_f16_small", 1, 2, 64, 1000, 64, "f16", False, 0.125, 6102), 4)),
])
def test_noalloc_matches_workspace_entry_point(first, second):
    import torch

    for w, splits in (first, second):
        print(f"CASE {w} splits={splits}", flush=True)
        assert fa.fa_splitkv_workspace_bytes(w.B, w.H, w.M, w.D, splits) <= fa.NOALLOC_MAX_BYTES
        qc, kc, vc, o1, l1, o2, l2 = _run_both(w, splits)
        assert not torch.isnan(o1).any() and not torch.isnan(l1).any()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        O_ref, L_ref = oracle.attention(_flat(qc), _flat(kc), _flat(vc), w.scale, w.causal)
        check(f"{w.name}-noalloc", w.dtype, _flat(o1.double()).cpu().numpy(),
              _flat(l1).cpu().numpy(), O_ref, L_ref)


def test_noalloc_refuses_beyond_its_scratch():
    import torch

    dev = torch.device("cuda:0")
    q = torch.zeros(1, 1024, 512, 64, dtype=torch.float16, device=dev)
    lse = torch.zeros(1, 1024, 512, device=dev)
    st = fa.fa_fwd_splitkv_noalloc(q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(),
                                   lse.data_ptr(), 1, 1024, 512, 512, 64, 0.125, 0, fa.DTYPE_F16, 4,
                                   None)
    assert st == 10
