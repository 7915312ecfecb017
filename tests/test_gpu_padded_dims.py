"""Head dims that are multiples of 8 other than the fast sizes and 32 (8 ... 120):
the forward runs the pipelined kernel of the next size up (64, 96 or 128) with the
feature chunks past D left out of every load and copy (zero in registers and
LDS) and out of the store.  Checked against the fp64 oracle on the four-wave
launch (small grids), the eight-wave persistent launch (several items per
workgroup), ragged query and key tails, M > N causal rows that see no key,
zero and negative scales; outputs are prefilled with NaN, so an unwritten
element fails.  The backward pads 40 ... 120 the same way."""

import math

import numpy as np
import pytest

import oracle
from gpu_calls import nan_fwd
from parity import check
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

PADDED_D = [40, 48, 56, 72, 80, 88, 104, 112, 120]  # forward and backward
PADDED_D_FWD = [8, 16, 24] + PADDED_D  # below 32 only the forward pads


def _run(w, splits=None):
    import torch

    print(f"CASE {w.name} B={w.B} H={w.H} M={w.M} N={w.N} D={w.D} {w.dtype} "
          f"causal={w.causal} scale={w.scale:+.4f} splits={splits}", flush=True)
    qc, kc, vc = make_inputs(w)
    dev = torch.device("cuda:0")
    o, lse = nan_fwd(qc.to(dev), kc.to(dev), vc.to(dev), causal=w.causal, scale=w.scale,
                     splits=splits)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(qc.double().numpy(), kc.double().numpy(),
                                    vc.double().numpy(), w.scale, w.causal)
    BH = w.B * w.H
    check(w.name, w.dtype, o.cpu().double().numpy().reshape(BH, w.M, w.D),
          lse.cpu().double().numpy().reshape(BH, w.M), O_ref.reshape(BH, w.M, w.D),
          L_ref.reshape(BH, w.M))
    return o, lse


@pytest.mark.parametrize("D", PADDED_D_FWD)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_padded_dims_small_grid(D, dtype, causal):
    """Four-wave launch: 2 x 3 heads, 300 rows (a ragged 128-row tile), 333 keys
    (a ragged 64-key tile); causal with M > N leaves 33 rows with no key."""
    M, N = (333, 300) if causal else (300, 333)
    _run(Workload(f"pad_small_{dtype}_D{D}_c{int(causal)}", 2, 3, M, N, D, dtype, causal,
                  1 / math.sqrt(D), 300 + D))


@pytest.mark.parametrize("D,dtype,causal", [(80, "bf16", True), (112, "bf16", True),
                                            (120, "f16", False), (48, "f16", True)])
def test_padded_dims_persistent(D, dtype, causal):
    """4 x 32 heads of 1000 rows: more items than CUs, so the eight-wave launch
    (D above 64) runs several items per workgroup; 200 keys, a ragged tail."""
    _run(Workload(f"pad_persist_{dtype}_D{D}_c{int(causal)}", 4, 32, 1000, 200, D, dtype, causal,
                  1 / math.sqrt(D), 400 + D))


@pytest.mark.parametrize("D,dtype,causal,M,N,splits", [
    (80, "bf16", True, 100, 3000, 3), (48, "f16", False, 1, 5000, 8), (120, "bf16", True, 16, 700, 5)])
def test_padded_dims_split_kv(D, dtype, causal, M, N, splits):
    """Split-KV on the padded path: the chunks' fp32 partials (rows of D
    features in the workspace) and the LSE merge; decode-like shapes."""
    _run(Workload(f"pad_split_{dtype}_D{D}_c{int(causal)}", 2, 4, M, N, D, dtype, causal,
                  1 / math.sqrt(D), 700 + D), splits=splits)


@pytest.mark.parametrize("scale", [0.0, -0.2])
def test_padded_dims_scale_sign(scale):
    """Zero scale (uniform weights over the visible keys) and a negative scale on
    the padded path: the sign fold acts on Q's padding chunks too."""
    _run(Workload(f"pad_scale_{scale:+.1f}", 2, 2, 200, 260, 72, "bf16", True, scale, 77))


def test_padded_matches_general_kernel():
    """The padded fast kernel and the general kernel agree within the bound on
    the same inputs (both are checked against the oracle above; this compares
    the two kernels directly, element by element)."""
    import torch

    w = Workload("pad_vs_general", 2, 4, 257, 515, 104, "bf16", True, 1 / math.sqrt(104), 5)
    qc, kc, vc = make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    o1, l1 = nan_fwd(q, k, v, causal=True, scale=w.scale)
    o2, l2 = nan_fwd(q, k, v, causal=True, scale=w.scale, general=True)
    torch.cuda.synchronize()
    assert not torch.isnan(o1).any() and not torch.isnan(o2).any()
    assert (o1.float() - o2.float()).abs().max().item() <= 2e-2
    assert np.abs((l1 - l2).cpu().numpy()).max() <= 2e-4


def _run_bwd(w):
    import torch

    from gpu_calls import nan_bwd
    from oracle.definition import scale_as_kernel
    from parity_bwd import bounds, check as check_bwd
    from workloads import make_dout

    print(f"CASE bwd {w.name} B={w.B} H={w.H} M={w.M} N={w.N} D={w.D} {w.dtype} "
          f"causal={w.causal}", flush=True)
    qc, kc, vc = make_inputs(w)
    gc = make_dout(w)
    dev = torch.device("cuda:0")
    q, k, v, g = qc.to(dev), kc.to(dev), vc.to(dev), gc.to(dev)
    o, lse = nan_fwd(q, k, v, causal=w.causal, scale=w.scale)
    dq, dk, dv = nan_bwd(q, k, v, o, lse, g, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    s = scale_as_kernel(w.scale)
    flat = lambda x: x.reshape(-1, *x.shape[2:])
    q64, k64, v64, g64 = (flat(x.double()).numpy() for x in (qc, kc, vc, gc))
    o_gpu, l_gpu = flat(o.cpu().double()).numpy(), flat(lse.cpu().double()).numpy()
    got = [flat(x.cpu().double()).numpy() for x in (dq, dk, dv)]
    for hh in range(q64.shape[0]):
        rq, rk, rv, parts = oracle.head_bwd(q64[hh], k64[hh], v64[hh], g64[hh], s, w.causal,
                                            return_parts=True)
        check(f"{w.name} head {hh} o", w.dtype, o_gpu[hh], l_gpu[hh], parts["O"], parts["lse"],
              verbose=False)
        bq, bk, bv = bounds(parts, q64[hh], k64[hh], g64[hh], s, w.dtype)
        check_bwd(f"{w.name} head {hh} dq", w.dtype, got[0][hh], rq, bq, verbose=False)
        check_bwd(f"{w.name} head {hh} dk", w.dtype, got[1][hh], rk, bk, verbose=False)
        check_bwd(f"{w.name} head {hh} dv", w.dtype, got[2][hh], rv, bv, verbose=False)


@pytest.mark.parametrize("D", PADDED_D)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_padded_dims_backward(D, dtype, causal):
    """The fast dK/dV and dQ kernels of the next size up with zero padding
    chunks: 2 x 2 heads, ragged 64-row query and 128-row key tiles; causal with
    M > N leaves rows with no key (their dQ is 0)."""
    M, N = (270, 200) if causal else (200, 270)
    _run_bwd(Workload(f"pad_bwd_{dtype}_D{D}_c{int(causal)}", 2, 2, M, N, D, dtype, causal,
                      1 / math.sqrt(D), 500 + D))


@pytest.mark.parametrize("D,dtype", [(112, "bf16"), (80, "f16")])
def test_padded_dims_backward_persistent(D, dtype):
    """More key tiles than CUs (4 x 32 heads x 3 tiles of 128 keys): the dK/dV
    kernel at D above 64 loops over several items per workgroup; 300 queries
    give the 8-wave dQ kernel two query tiles per head."""
    _run_bwd(Workload(f"pad_bwd_persist_{dtype}_D{D}", 4, 32, 300, 300, D, dtype, True,
                      1 / math.sqrt(D), 600 + D))
