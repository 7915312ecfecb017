"""Comparison of the HIP path's outputs with the oracle's (shared by the GPU tests).

Tolerance (stated in the test, applied per element):

    |O_gpu - O_ref| <= TOL[dtype] + 1/2 ulp_dtype(O_ref)
    |LSE_gpu - LSE_ref| <= 1e-4, and -inf exactly where the oracle has -inf

TOL is 1e-5 (fp32), 2e-3 (fp16), 1e-2 (bf16) on O and 1e-4 on LSE.  The half
ulp term is the rounding of the exact result to the output dtype, which alone
can exceed the bare bound (bf16 outputs with |O| >= 4 have a half ulp of
2^-6 = 0.0156 > 1e-2); the bound therefore applies to the error beyond that
final rounding.  Each check also reports the raw max error, the rounding floor
max|rnd(O_ref) - O_ref| and how many elements exceed the bare bound, so either
reading can be applied by the reader.
"""

from __future__ import annotations

import numpy as np

TOL_O = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}
TOL_LSE = 1e-4


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Half the spacing of `dtype` numbers at |x| (subnormal spacing near 0)."""
    ax = np.abs(x)
    e = np.frexp(ax)[1]  # |x| = m * 2^e, m in [0.5, 1)
    mant, emin = {"f32": (23, -126), "f16": (10, -14), "bf16": (7, -126)}[dtype]
    e = np.maximum(e - 1, emin)  # unbiased exponent of the binade, clamped at the subnormal range
    return np.ldexp(1.0, e - mant - 1)


def rounded(x: np.ndarray, dtype: str) -> np.ndarray:
    import torch

    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    return torch.from_numpy(np.ascontiguousarray(x)).to(tdt).double().numpy()


def check(name: str, dtype: str, O_gpu, L_gpu, O_ref, L_ref, *, verbose: bool = True) -> dict:
    """Assert parity and return the report numbers."""
    O_gpu = np.asarray(O_gpu, dtype=np.float64)
    L_gpu = np.asarray(L_gpu, dtype=np.float64)
    O_ref = np.asarray(O_ref, dtype=np.float64)
    L_ref = np.asarray(L_ref, dtype=np.float64)
    assert O_gpu.shape == O_ref.shape and L_gpu.shape == L_ref.shape
    assert np.all(np.isfinite(O_gpu)), f"{name}: non-finite O"
    err = np.abs(O_gpu - O_ref)
    bound = TOL_O[dtype] + half_ulp(O_ref, dtype)
    floor = float(np.abs(rounded(O_ref, dtype) - O_ref).max(initial=0.0))
    rep = {
        "case": name, "dtype": dtype,
        "o_max_err": float(err.max(initial=0.0)),
        "o_round_floor": floor,
        "o_above_bare_tol": int((err > TOL_O[dtype]).sum()),
        "o_above_bound": int((err > bound).sum()),
        "n": int(err.size),
    }
    inf_ref = np.isneginf(L_ref)
    assert np.array_equal(np.isneginf(L_gpu), inf_ref), f"{name}: -inf LSE rows differ"
    fin = ~inf_ref
    lerr = np.abs(L_gpu[fin] - L_ref[fin])
    rep["lse_max_err"] = float(lerr.max(initial=0.0))
    rep["empty_rows"] = int(inf_ref.sum())
    if inf_ref.any():
        # rows without a visible key: O must be exactly zero
        Oz = O_gpu.reshape(-1, O_gpu.shape[-1])[inf_ref.reshape(-1)]
        assert np.all(Oz == 0.0), f"{name}: empty rows not zero"
    if verbose:
        print("PARITY " + " ".join(f"{k}={v}" for k, v in rep.items()), flush=True)
    assert rep["o_above_bound"] == 0, rep
    assert rep["lse_max_err"] <= TOL_LSE, rep
    return rep
