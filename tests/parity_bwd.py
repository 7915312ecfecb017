"""Comparison of the HIP backward pass with the fp64 oracle (shared by the GPU tests).

The pages state no accuracy for gradients, so the bound is derived from the
arithmetic of the kernels, element by element, from exact (oracle) quantities:

* P is rebuilt in fp32 and rounded to the input type (unit roundoff u: 2^-8 for
  bf16, 2^-11 for fp16; fp32 inputs keep P and dS in fp32, u = 2^-24) before
  dV = P^T dO:                                          |err dV| <= u P^T |dO|
* Delta uses the forward output the caller passes, which the tests check
  against the forward's own per-element bound |O_gpu - O| <= TOL_O + 1/2 ulp(O)
  (tests/parity.py); so e_D[i] = sum_d |dO_id| (TOL_O + 1/2 ulp(O_id)), from
  stated bounds and exact values only; dS = P (dP - Delta) is rounded to the
  input type before its products:       |err dS| <= E = u |dS| + P e_D[:, None]
* dK = s dS^T Q and dQ = s dS K:        |err dK| <= |s| E^T |Q|,  |err dQ| <= |s| E |K|

The test allows twice this first-order bound, plus half an ulp of the output
type at the exact value (the final rounding) and 1e-5 of the largest exact
value (fp32 accumulation over up to 65536 terms).  A dropped term, a wrong
sign, a transposed operand or a missing scale is larger by orders of
magnitude.  Each check reports the raw max error, the max error relative to the
bound, and the count above it.
"""

from __future__ import annotations

import numpy as np

from parity import TOL_O, half_ulp

UNIT = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8, "f32": 2.0 ** -24}


def bounds(parts: dict, q, k, dout, s: float, dtype: str):
    """Per-element error bounds (dq, dk, dv) for one head from the oracle's parts
    and the forward's stated per-element bound on O (never from GPU output)."""
    u = UNIT[dtype]
    P, dS, O = parts["P"], parts["dS"], parts["O"]
    ad = np.abs(dout)
    e_o = TOL_O[dtype] + half_ulp(O, dtype)
    e_delta = np.sum(ad * e_o, axis=1) + 2.0 ** -22 * np.sum(np.abs(dout * O), axis=1)
    E = u * np.abs(dS) + P * e_delta[:, None]
    b_dv = u * (P.T @ ad)
    b_dk = abs(s) * (E.T @ np.abs(q))
    b_dq = abs(s) * (E @ np.abs(k))
    return b_dq, b_dk, b_dv


def check(name: str, dtype: str, got, ref, bound, *, verbose: bool = True) -> dict:
    """Assert |got - ref| <= 2 bound + half ulp(ref) + 1e-5 max|ref| elementwise."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape == bound.shape
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    allow = 2.0 * bound + half_ulp(ref, dtype) + 1e-5 * float(np.abs(ref).max(initial=0.0))
    rep = {
        "case": name, "dtype": dtype,
        "max_err": float(err.max(initial=0.0)),
        "max_ref": float(np.abs(ref).max(initial=0.0)),
        "max_err_over_allow": float((err / allow).max(initial=0.0)) if err.size else 0.0,
        "above": int((err > allow).sum()),
        "n": int(err.size),
    }
    if verbose:
        print("PARITY_BWD " + " ".join(f"{k}={v}" for k, v in rep.items()), flush=True)
    assert rep["above"] == 0, rep
    return rep
