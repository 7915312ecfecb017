"""Parity of fa_fwd, fa_fwd_splitkv and fa_bwd with the fp64 oracle on a
seeded sweep of random shapes: every dtype, head dims on and off the fast
paths (1 to 128), M and N from one row to several tiles with ragged tails,
M > N and M < N under the bottom-right causal mask, and positive, negative
and zero scales.  The case list is drawn once from a fixed seed, so every run
checks the same cases; each case's parameters are in its test id.  A second
draw takes its head dims from the multiples of 8 that the 16-bit kernels
zero-pad to the next fast size.  Outputs
are prefilled with NaN (gpu_calls), so an element a kernel fails to write
fails the comparison."""

import math

import numpy as np
import pytest

import oracle
from gpu_calls import nan_bwd, nan_fwd
from oracle.definition import scale_as_kernel
from parity import check
from parity_bwd import bounds, check as check_bwd
from workloads import Workload, make_dout, make_inputs

pytestmark = pytest.mark.gpu

D_CHOICES = [1, 7, 16, 33, 40, 64, 64, 65, 96, 96, 100, 127, 128, 128]
# Multiples of 8 that the 16-bit paths zero-pad to the next fast size.
D_PADDED = [8, 24, 48, 56, 72, 80, 88, 104, 112, 120]


def _cases(n: int, seed: int, d_choices=D_CHOICES, tag="r"):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = ("f32", "f16", "bf16")[i % 3]
        D = int(rng.choice(d_choices))
        M = int(rng.integers(1, 600))
        N = int(rng.integers(1, 800))
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 4))
        causal = bool(rng.integers(0, 2))
        kind = int(rng.integers(0, 6))
        if kind < 4:
            scale = 1.0 / math.sqrt(D)
        elif kind == 4:
            scale = 0.0
        else:
            scale = -float(rng.uniform(0.05, 0.5))
        splits = int(rng.choice([0, 0, 2, 5]))
        name = (f"{tag}{i}_{dtype}_B{B}H{H}_M{M}_N{N}_D{D}_{'causal' if causal else 'full'}"
                f"_s{scale:+.3f}_sp{splits}")
        out.append((Workload(name=name, B=B, H=H, M=M, N=N, D=D, dtype=dtype, causal=causal,
                             scale=scale, seed=7000 + i), splits))
    return out


FWD_CASES = _cases(48, 20261203) + _cases(24, 20261205, D_PADDED, "p")
BWD_CASES = [w for w, _ in _cases(24, 20261204) + _cases(12, 20261206, D_PADDED, "p")]


def _flat(x):
    return x.reshape(-1, *x.shape[2:])


@pytest.mark.parametrize("w,splits", FWD_CASES, ids=[w.name for w, _ in FWD_CASES])
def test_random_shape_forward(w, splits):
    import torch

    print(f"CASE {w.name}", flush=True)
    qc, kc, vc = make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    o, lse = nan_fwd(q, k, v, causal=w.causal, scale=w.scale, splits=splits or None)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(qc.double().numpy(), kc.double().numpy(),
                                    vc.double().numpy(), w.scale, w.causal)
    check(w.name, w.dtype, _flat(o.cpu().double()).numpy(), _flat(lse.cpu().double()).numpy(),
          O_ref.reshape(-1, w.M, w.D), L_ref.reshape(-1, w.M))


@pytest.mark.parametrize("w", BWD_CASES, ids=[w.name for w in BWD_CASES])
def test_random_shape_backward(w):
    import torch

    print(f"CASE {w.name}", flush=True)
    qc, kc, vc = make_inputs(w)
    gc = make_dout(w)
    dev = torch.device("cuda:0")
    q, k, v, g = qc.to(dev), kc.to(dev), vc.to(dev), gc.to(dev)
    o, lse = nan_fwd(q, k, v, causal=w.causal, scale=w.scale)
    dq, dk, dv = nan_bwd(q, k, v, o, lse, g, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    s = scale_as_kernel(w.scale)
    q64, k64, v64, g64 = (_flat(x.double()).numpy() for x in (qc, kc, vc, gc))
    o_gpu, l_gpu = _flat(o.cpu().double()).numpy(), _flat(lse.cpu().double()).numpy()
    got = [_flat(x.cpu().double()).numpy() for x in (dq, dk, dv)]
    for h in range(q64.shape[0]):
        rq, rk, rv, parts = oracle.head_bwd(q64[h], k64[h], v64[h], g64[h], s, w.causal,
                                            return_parts=True)
        # the backward consumes this forward output; its bound is the forward's
        check(f"{w.name} head {h} o", w.dtype, o_gpu[h], l_gpu[h], parts["O"], parts["lse"],
              verbose=False)
        bq, bk, bv = bounds(parts, q64[h], k64[h], g64[h], s, w.dtype)
        check_bwd(f"{w.name} head {h} dq", w.dtype, got[0][h], rq, bq, verbose=False)
        check_bwd(f"{w.name} head {h} dk", w.dtype, got[1][h], rk, bk, verbose=False)
        check_bwd(f"{w.name} head {h} dv", w.dtype, got[2][h], rv, bv, verbose=False)
