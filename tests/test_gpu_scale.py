"""Any finite scale through the C ABI, on every kernel path: zero (uniform
weights over the visible keys, LSE = ln #visible) and negative scales
(S = scale * Q K^T weights small scores up), forward, split-KV and backward,
against the fp64 oracle under the standard per-element bounds.  The oracle's
handling of these scales is pinned on the CPU (tests/oracle_pins.py:
pin_zero_scale_uniform, pin_negative_scale; tests/test_oracle_backward.py:
test_gradients_any_finite_scale)."""

import math

import numpy as np
import pytest

import oracle
from gpu_calls import nan_bwd, nan_fwd
from oracle.definition import scale_as_kernel
from parity import check
from parity_bwd import bounds
from parity_bwd import check as check_bwd
from workloads import Workload, make_dout, make_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"CASE {msg}", flush=True)


def _flat(x):
    return x.reshape(-1, *x.shape[2:])


# (label, B, H, M, N, D, dtype, causal, extra call arguments): one line per kernel path
FWD_PATHS = [
    ("pipe8_bf16_d128_causal", 1, 3, 600, 700, 128, "bf16", True, {}),
    ("pipe4_f16_d64", 2, 2, 300, 333, 64, "f16", False, {}),
    ("pipe8_f16_d96_causal_mgtn", 1, 2, 500, 300, 96, "f16", True, {}),
    ("general_bf16_d100_causal", 1, 2, 200, 260, 100, "bf16", True, {}),
    ("general_f16_d128", 1, 2, 150, 200, 128, "f16", False, {"general": True}),
    ("f32_d128", 1, 2, 300, 200, 128, "f32", True, {}),
    ("f32_keysplit_d64", 1, 1, 100, 700, 64, "f32", True, {}),
    ("split_bf16_d128_causal", 1, 2, 200, 1500, 128, "bf16", True, {"splits": 4}),
    ("split_f16_d65", 1, 1, 100, 900, 65, "f16", False, {"splits": 3}),
    ("split_f32_d32_causal", 1, 1, 80, 500, 32, "f32", True, {"splits": 5}),
]
SCALES = [0.0, -1.0, -0.05]  # multiples of 1/sqrt(D) for the nonzero ones


@pytest.mark.parametrize("mult", SCALES, ids=["zero", "neg", "neg_small"])
@pytest.mark.parametrize("path", FWD_PATHS, ids=[p[0] for p in FWD_PATHS])
def test_forward_any_finite_scale(path, mult):
    import torch

    label, B, H, M, N, D, dtype, causal, extra = path
    scale = mult / math.sqrt(D)
    w = Workload(f"scale_{label}", B, H, M, N, D, dtype, causal, scale, 5300 + D)
    _say(f"{w} {extra}")
    qc, kc, vc = make_inputs(w)
    dev = torch.device("cuda:0")
    o, lse = nan_fwd(qc.to(dev), kc.to(dev), vc.to(dev), causal=causal, scale=scale, **extra)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention(_flat(qc), _flat(kc), _flat(vc), scale, causal)
    check(f"{label} scale={scale:.4g}", dtype, _flat(o.double()).cpu().numpy(),
          _flat(lse).cpu().numpy(), O_ref, L_ref)
    if mult == 0.0:
        # uniform weights: LSE = ln(#visible keys) for every row that sees a key
        vis = np.array([N if not causal else max(0, min(N, i + N - M + 1)) for i in range(M)])
        L = _flat(lse).cpu().numpy()
        ok = vis > 0
        assert np.abs(L[:, ok] - np.log(vis[ok])[None, :]).max() <= 1e-4


BWD_PATHS = [
    ("fast_bf16_d128_causal", 1, 2, 300, 260, 128, "bf16", True),
    ("fast_f16_d64", 1, 2, 200, 333, 64, "f16", False),
    ("general_bf16_d40_causal", 1, 2, 130, 200, 40, "bf16", True),
    ("f32_d64_causal", 1, 2, 200, 260, 64, "f32", True),
]


@pytest.mark.parametrize("mult", [0.0, -1.0], ids=["zero", "neg"])
@pytest.mark.parametrize("path", BWD_PATHS, ids=[p[0] for p in BWD_PATHS])
def test_backward_any_finite_scale(path, mult):
    import torch

    label, B, H, M, N, D, dtype, causal = path
    scale = mult / math.sqrt(D)
    w = Workload(f"scale_bwd_{label}", B, H, M, N, D, dtype, causal, scale, 5400 + D)
    _say(f"{w}")
    qc, kc, vc = make_inputs(w)
    gc = make_dout(w)
    dev = torch.device("cuda:0")
    q, k, v, g = qc.to(dev), kc.to(dev), vc.to(dev), gc.to(dev)
    o, lse = nan_fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = nan_bwd(q, k, v, o, lse, g, causal=causal, scale=scale)
    torch.cuda.synchronize()
    s = scale_as_kernel(scale)
    f64 = lambda x: _flat(x.double().cpu()).numpy()  # noqa: E731
    q64, k64, v64, g64 = f64(qc), f64(kc), f64(vc), f64(gc)
    o64, l64 = f64(o), _flat(lse.cpu().double()).numpy()
    dq64, dk64, dv64 = f64(dq), f64(dk), f64(dv)
    for h in range(B * H):
        rq, rk, rv, parts = oracle.head_bwd(q64[h], k64[h], v64[h], g64[h], s, causal,
                                            return_parts=True)
        check(f"{label} head {h} o", dtype, o64[h], l64[h], parts["O"], parts["lse"],
                  verbose=False)
        bq, bk, bv = bounds(parts, q64[h], k64[h], g64[h], s, dtype)
        check_bwd(f"{label} scale={scale:.4g} head {h} dq", dtype, dq64[h], rq, bq)
        check_bwd(f"{label} scale={scale:.4g} head {h} dk", dtype, dk64[h], rk, bk)
        check_bwd(f"{label} scale={scale:.4g} head {h} dv", dtype, dv64[h], rv, bv)
        if mult == 0.0:
            assert np.all(dq64[h] == 0.0) and np.all(dk64[h] == 0.0)
