"""Plant plausible mistakes in the oracle's definition (on the CPU) and check that
at least one pin catches each.  A pin 'catches' a mutant when it raises."""

import math

import numpy as np
import pytest

import oracle
import oracle.backward as ob
import oracle.definition as oa
import oracle.split as osp
from oracle_pins import PINS

_orig_scores = oa.scores
_orig_softmax = oa.masked_softmax
_orig_mask = oa.visible_mask


def _softmax_no_max(S, vis):
    e = np.where(vis, np.exp(np.where(vis, S, -np.inf)), 0.0)
    l = e.sum(axis=1)
    with np.errstate(all="ignore"):
        return e / l[:, None], S.max(axis=1), np.log(l)


def _softmax_lse_no_m(S, vis):
    P, m, lse = _orig_softmax(S, vis)
    return P, m, lse - np.where(np.isfinite(m), m, 0.0)


def _softmax_log2(S, vis):
    P, m, lse = _orig_softmax(S, vis)
    mm = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(all="ignore"):
        return P, m, mm + (lse - mm) / math.log(2.0)


def _softmax_unnormalised(S, vis):
    P, m, lse = _orig_softmax(S, vis)
    return P * np.exp(np.where(np.isfinite(lse), lse - np.where(np.isfinite(m), m, 0), 0))[:, None], m, lse


def _softmax_sign(S, vis):
    Sm = np.where(vis, S, -np.inf)
    m = Sm.max(axis=1)
    e = np.where(vis, np.exp(np.where(vis, m[:, None] - S, 0.0)), 0.0)
    l = e.sum(axis=1)
    with np.errstate(all="ignore"):
        return e / l[:, None], m, m + np.log(l)


def _softmax_empty_nan(S, vis):
    Sm = np.where(vis, S, -np.inf)
    m = Sm.max(axis=1)
    with np.errstate(all="ignore"):
        e = np.where(vis, np.exp(Sm - m[:, None]), 0.0)
        l = e.sum(axis=1)
        return e / l[:, None], m, m + np.log(l)


def _softmax_drop_last_key(S, vis):
    vis = vis.copy()
    vis[:, -1] = False if vis.shape[1] > 1 else vis[:, -1]
    return _orig_softmax(S, vis)


MUTANTS = {
    "scores_without_scale": ("scores", lambda q, k, s: q @ k.T),
    "scores_scale_inverted": ("scores", lambda q, k, s: (q @ k.T) / s),
    "scores_scale_sqrt": ("scores", lambda q, k, s: math.sqrt(s) * (q @ k.T)),
    "scores_transposed": ("scores", lambda q, k, s: s * (k @ q.T)),
    "scores_drop_last_feature": ("scores", lambda q, k, s: s * (q[:, :-1] @ k[:, :-1].T)
                                 if q.shape[1] > 1 else s * (q @ k.T) * 0.0),
    "mask_top_left": ("visible_mask", lambda rows, N, M, causal: _orig_mask(rows, N, N, causal)),
    "mask_off_by_one": ("visible_mask", lambda rows, N, M, causal:
                        _orig_mask(rows, N, M, causal) if not causal else
                        np.arange(N)[None, :] < np.asarray(rows)[:, None] + (N - M)),
    "mask_inverted_side": ("visible_mask", lambda rows, N, M, causal:
                           _orig_mask(rows, N, M, causal) if not causal else
                           np.arange(N)[None, :] >= np.asarray(rows)[:, None] + (N - M)),
    "mask_ignored": ("visible_mask", lambda rows, N, M, causal: _orig_mask(rows, N, M, False)),
    "softmax_no_max_subtraction": ("masked_softmax", _softmax_no_max),
    "lse_missing_max": ("masked_softmax", _softmax_lse_no_m),
    "lse_in_log2": ("masked_softmax", _softmax_log2),
    "p_not_normalised": ("masked_softmax", _softmax_unnormalised),
    "exponent_sign_flipped": ("masked_softmax", _softmax_sign),
    "empty_row_unguarded": ("masked_softmax", _softmax_empty_nan),
    "last_key_dropped": ("masked_softmax", _softmax_drop_last_key),
}


def _bf16(s):
    import torch

    return float(torch.tensor(s, dtype=torch.float64).to(torch.bfloat16).double())


# Wrong roundings of the fp32 scale argument, planted in every module that
# binds the helper (the definition, the split and backward oracles, the package).
SCALE_MUTANTS = {
    "scale_rounded_to_fp16": lambda s: float(np.float16(s)),
    "scale_rounded_to_bf16": _bf16,
    "scale_not_rounded": lambda s: float(s),
    "scale_sign_dropped": lambda s: abs(float(np.float32(s))),
}


@pytest.mark.parametrize("name", sorted(SCALE_MUTANTS))
def test_scale_mutant_is_caught(name, monkeypatch):
    fn = SCALE_MUTANTS[name]
    for mod in (oa, ob, osp, oracle):
        monkeypatch.setattr(mod, "scale_as_kernel", fn)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception:  # noqa: BLE001 - any failure of a pin counts as caught
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(oa, attr, fn)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception:  # noqa: BLE001 - any failure of a pin counts as caught
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
