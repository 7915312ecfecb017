"""Parity of the HIP backward pass (fa_bwd through the C ABI) with the fp64
oracle's gradients, on seeded inputs: the forward pass runs on the GPU first
(as a caller would), then fa_bwd with a seeded incoming gradient.  The
per-element error bound is derived in tests/parity_bwd.py."""

import numpy as np
import pytest

import io_aware_tiled_fa_amd as fa
import oracle
from oracle.definition import scale_as_kernel
from gpu_calls import nan_bwd, nan_fwd
from parity import check as check_fwd
from parity_bwd import bounds, check
from workloads import WORKLOADS, Workload, make_dout, make_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"CASE {msg}", flush=True)


def _gpu_fwd_bwd(w, qc, kc, vc, gc):
    import torch

    dev = torch.device("cuda:0")
    q, k, v, g = qc.to(dev), kc.to(dev), vc.to(dev), gc.to(dev)
    o, lse = nan_fwd(q, k, v, causal=w.causal, scale=w.scale)
    dq, dk, dv = nan_bwd(q, k, v, o, lse, g, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def _flat(x):
    return x.reshape(-1, *x.shape[2:])


def _check_heads(w, heads=None):
    qc, kc, vc = make_inputs(w)
    gc = make_dout(w)
    o, lse, dq, dk, dv = _gpu_fwd_bwd(w, qc, kc, vc, gc)
    q64, k64, v64 = (_flat(x.double()).numpy() for x in (qc, kc, vc))
    g64 = _flat(gc.double()).numpy()
    o_gpu = _flat(o.cpu().double()).numpy()
    l_gpu = _flat(lse.cpu().double()).numpy()
    dq_gpu, dk_gpu, dv_gpu = (_flat(x.cpu().double()).numpy() for x in (dq, dk, dv))
    s = scale_as_kernel(w.scale)
    nh = q64.shape[0]
    heads = range(nh) if heads is None else heads
    reps = []
    for h in heads:
        rq, rk, rv, parts = oracle.head_bwd(q64[h], k64[h], v64[h], g64[h], s, w.causal,
                                            return_parts=True)
        # the forward output the backward consumes is within the forward's bound,
        # from which the backward's bound on Delta is derived
        check_fwd(f"{w.name} head {h} o", w.dtype, o_gpu[h], l_gpu[h], parts["O"], parts["lse"],
                  verbose=False)
        bq, bk, bv = bounds(parts, q64[h], k64[h], g64[h], s, w.dtype)
        reps.append(check(f"{w.name} head {h} dq", w.dtype, dq_gpu[h], rq, bq, verbose=False))
        reps.append(check(f"{w.name} head {h} dk", w.dtype, dk_gpu[h], rk, bk, verbose=False))
        reps.append(check(f"{w.name} head {h} dv", w.dtype, dv_gpu[h], rv, bv, verbose=False))
        if w.causal and w.M > w.N:  # rows without a visible key: dq exactly 0
            assert np.all(dq_gpu[h][: w.M - w.N] == 0.0)
    for name in ("dq", "dk", "dv"):
        rs = [r for r in reps if r["case"].endswith(name)]
        print(f"PARITY_BWD case={w.name} grad={name} heads={len(rs)} "
              f"max_err={max(r['max_err'] for r in rs):.3e} "
              f"max_ref={max(r['max_ref'] for r in rs):.3e} "
              f"max_err_over_allow={max(r['max_err_over_allow'] for r in rs):.3f}", flush=True)
    return reps


def _wl(name, B, H, M, N, D, dtype, causal, seed):
    return Workload(name=name, B=B, H=H, M=M, N=N, D=D, dtype=dtype, causal=causal,
                    scale=1.0 / np.sqrt(D), seed=seed)


SMALL = [
    _wl("bwd_small_bf16", 1, 2, 100, 150, 64, "bf16", False, 3101),
    _wl("bwd_small_f16_causal_mltn", 1, 2, 150, 100, 64, "f16", True, 3102),
    _wl("bwd_sq_bf16_causal", 2, 1, 200, 200, 128, "bf16", True, 3103),
    _wl("bwd_ragged_f16_causal", 1, 1, 77, 333, 96, "f16", True, 3104),
    _wl("bwd_d1_bf16", 1, 1, 70, 90, 1, "bf16", True, 3105),
    _wl("bwd_d8_f16", 1, 2, 65, 129, 8, "f16", False, 3106),
    _wl("bwd_d40_bf16", 1, 1, 130, 257, 40, "bf16", True, 3107),
    _wl("bwd_d65_f16", 1, 1, 64, 64, 65, "f16", False, 3108),
    _wl("bwd_d100_bf16", 1, 1, 129, 130, 100, "bf16", True, 3109),
    _wl("bwd_d32_f16_causal", 1, 1, 256, 256, 32, "f16", True, 3110),
    _wl("bwd_m1_bf16", 1, 1, 1, 300, 64, "bf16", False, 3111),
    _wl("bwd_n1_f16", 1, 1, 300, 1, 64, "f16", False, 3112),
    _wl("bwd_empty_rows_f16", 1, 2, 300, 100, 64, "f16", True, 3113),
    # fast dK/dV path: ragged query and key tails, M > N causal, many query tiles
    _wl("bwd_fast_d128_ragged_bf16", 1, 2, 337, 261, 128, "bf16", False, 3114),
    _wl("bwd_fast_d96_causal_mgtn_f16", 1, 1, 700, 450, 96, "f16", True, 3115),
    _wl("bwd_fast_d64_many_tiles_bf16", 1, 1, 1100, 1030, 64, "bf16", True, 3116),
]


# fp32: P and dS stay fp32 (fa_bwd on v_mfma_f32_32x32x2f32)
F32 = [
    _wl("bwd_f32_d64", 1, 2, 100, 150, 64, "f32", False, 3131),
    _wl("bwd_f32_causal_mgtn_d32", 1, 1, 150, 100, 32, "f32", True, 3132),
    _wl("bwd_f32_causal_d128", 1, 2, 200, 200, 128, "f32", True, 3133),
    _wl("bwd_f32_d1", 1, 1, 70, 90, 1, "f32", True, 3134),
    _wl("bwd_f32_d40_ragged", 1, 1, 130, 257, 40, "f32", False, 3135),
    _wl("bwd_f32_d65", 1, 1, 64, 64, 65, "f32", True, 3136),
    _wl("bwd_f32_m1", 1, 1, 1, 300, 96, "f32", False, 3137),
    _wl("bwd_f32_n1", 1, 1, 300, 1, 64, "f32", False, 3138),
    _wl("bwd_f32_single_head_shape", 1, 1, 256, 1024, 64, "f32", False, 3139),
]
SMALL = SMALL + F32


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_bwd_small_shapes(w):
    _say(f"{w}")
    _check_heads(w)


def test_bwd_gpt2_medium_shape():
    """GPT-2-medium attention shapes (fp16, D = 64, N = 1024), on 4 heads."""
    w = WORKLOADS["gpt2_medium_f16"].with_(B=1, H=4)
    _say(f"{w}")
    _check_heads(w)


def test_bwd_causal_prefill_two_heads():
    """The headline shape (bf16, D = 128, M = N = 4096, causal) on two full heads."""
    w = WORKLOADS["causal_prefill_bf16"].with_(B=1, H=2)
    _say(f"{w}")
    _check_heads(w)


def test_bwd_stress_large_logits():
    """fp16 with Q scaled by 8 (peaked rows), M != N, causal bottom-right."""
    w = WORKLOADS["stress_f16_causal"].with_(B=1, H=2)
    _say(f"{w}")
    _check_heads(w)


@pytest.mark.parametrize("w", [
    # more (head, tile) items than workgroups: the persistent dK/dV and dQ
    # launches, with item counts that do not divide evenly over the XCDs
    _wl("bwd_persistent_bf16_causal", 3, 27, 1024, 1024, 128, "bf16", True, 3121),
    _wl("bwd_persistent_f16_d96", 2, 37, 500, 700, 96, "f16", False, 3122),
], ids=lambda w: w.name)
def test_bwd_persistent_launch(w):
    _say(f"{w}")
    nh = w.B * w.H
    _check_heads(w, heads=sorted({0, 1, nh // 3, nh // 2, nh - 2, nh - 1}))


def test_bwd_no_keys_and_no_queries():
    import torch

    dev = torch.device("cuda:0")
    _say("bwd N=0 and M=0")
    # N = 0: every row is empty, dq must be all zeros
    q = torch.randn(1, 2, 40, 64, device=dev).half()
    g = torch.randn(1, 2, 40, 64, device=dev).half()
    e = torch.empty(1, 2, 0, 64, device=dev).half()
    o, lse = fa.fwd(q, e, e, causal=False)
    dq = torch.full_like(q, 7.0)
    dq, dk, dv = fa.bwd(q, e, e, o, lse, g, dq=dq)
    torch.cuda.synchronize()
    assert torch.all(dq == 0)
    # M = 0: no query sees any key, dk and dv must be all zeros
    k = torch.randn(1, 2, 70, 64, device=dev).half()
    qe = torch.empty(1, 2, 0, 64, device=dev).half()
    lse0 = torch.empty(1, 2, 0, device=dev)
    dk = torch.full_like(k, 7.0)
    dv = torch.full_like(k, 7.0)
    fa.bwd(qe, k, k, qe, lse0, qe, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)


def test_bwd_sum_rules_and_determinism():
    """Rows of dS sum to 0, so dK summed over keys is ~0; dV summed over keys
    equals dO summed over the rows that see a key; two runs are bit-identical."""
    import torch

    w = _wl("bwd_props_bf16", 1, 2, 500, 700, 128, "bf16", True, 3120)
    _say(f"{w}")
    qc, kc, vc = make_inputs(w)
    gc = make_dout(w)
    o, lse, dq, dk, dv = _gpu_fwd_bwd(w, qc, kc, vc, gc)
    _, _, dq2, dk2, dv2 = _gpu_fwd_bwd(w, qc, kc, vc, gc)
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    dv_sum = dv.double().sum(dim=2).cpu()
    g_sum = gc.double().sum(dim=2)
    scale_dv = dv.double().abs().sum(dim=2).cpu().max().item()
    assert (dv_sum - g_sum).abs().max().item() <= 2e-2 * scale_dv + 1e-3
    dk_sum = dk.double().sum(dim=2).cpu()
    scale_dk = dk.double().abs().sum(dim=2).cpu().max().item()
    assert dk_sum.abs().max().item() <= 2e-2 * scale_dk + 1e-3


@pytest.mark.parametrize("D,BH", [(128, 16385), (112, 18725)])
def test_bwd_tensors_beyond_2_31_elements(D, BH):
    """Forward and backward with Q, K, V, dO and the gradients of more than 2^31
    elements each (BH heads of 1024 x D, bf16, causal; D = 112 runs the fast
    kernels zero-padded to 128): every gradient of the first head, the heads on
    either side of the 2^31-element offset and the last head against the
    oracle.  Inputs are drawn on the GPU (seeded)."""
    import torch
    from workloads import make_dout_device, make_inputs_device

    w = _wl(f"bwd_big_bf16_causal_d{D}", 1, BH, 1024, 1024, D, "bf16", True, 3201)
    per = w.M * w.D
    assert w.H * per > 2**31
    _say(f"{w} ({w.H * per} elements per tensor)")
    dev = torch.device("cuda:0")
    q, k, v = make_inputs_device(w, dev)
    g = make_dout_device(w, dev)
    o, lse = nan_fwd(q, k, v, causal=w.causal, scale=w.scale)
    dq, dk, dv = nan_bwd(q, k, v, o, lse, g, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    s = scale_as_kernel(w.scale)
    for h in sorted({0, 2**31 // per - 1, 2**31 // per, w.H - 1}):
        q64, k64, v64, g64 = (x[0, h].double().cpu().numpy() for x in (q, k, v, g))
        o_h = o[0, h].double().cpu().numpy()
        rq, rk, rv, parts = oracle.head_bwd(q64, k64, v64, g64, s, w.causal, return_parts=True)
        check_fwd(f"{w.name} head {h} o", w.dtype, o_h, lse[0, h].double().cpu().numpy(),
                  parts["O"], parts["lse"], verbose=False)
        bq, bk, bv = bounds(parts, q64, k64, g64, s, w.dtype)
        for name, got, ref, bnd in (("dq", dq, rq, bq), ("dk", dk, rk, bk), ("dv", dv, rv, bv)):
            check(f"{w.name} head {h} {name}", w.dtype, got[0, h].double().cpu().numpy(), ref, bnd)
    del q, k, v, g, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
