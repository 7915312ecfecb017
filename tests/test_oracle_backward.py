"""Pins of the backward oracle (oracle/backward.py), CPU only.

The gradient formulas are not printed on the pages, so they are pinned against
things that do not use them:

* central finite differences of the forward definition (oracle.attention),
  whose own pins live in test_oracle_pins.py;
* closed forms that follow from the definition (N = 1, equal keys, sums over
  keys);
* the rebuild of P from the saved LSE, the check of the Module 08 page's Step 6
  ("memory footprint and recomputation"), where rebuilt tiles matched the
  stored P to rounding error;
* mutants with one plausible mistake each, which the finite-difference pin must
  reject.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle.definition import masked_softmax, scores, visible_mask

SCALE = 0.5  # exact in fp32, so the oracle's fp32-rounded scale is this value


def _loss(q, k, v, g, causal, scale=SCALE):
    O, _ = oracle.attention(q, k, v, scale, causal)
    return float(np.sum(O * g))


def _fd_grads(q, k, v, g, causal, h=1e-6, scale=SCALE):
    """Central differences of sum(O * g) with respect to every input element."""
    grads = []
    for which in range(3):
        xs = [q.copy(), k.copy(), v.copy()]
        gx = np.zeros_like(xs[which])
        it = np.nditer(gx, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = [x.copy() for x in xs]
            xm = [x.copy() for x in xs]
            xp[which][idx] += h
            xm[which][idx] -= h
            gx[idx] = (_loss(*xp, g, causal, scale) - _loss(*xm, g, causal, scale)) / (2 * h)
        grads.append(gx)
    return grads


SHAPES = [  # (M, N, D, causal)
    (1, 1, 1, False),
    (3, 5, 2, False),
    (5, 3, 4, False),
    (4, 4, 3, True),
    (3, 7, 2, True),   # M < N: bottom-right mask, every row sees keys
    (6, 3, 2, True),   # M > N: rows 0..2 see no key
    (7, 7, 4, True),
]


def _inputs(M, N, D, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((M, D))
    k = rng.standard_normal((N, D))
    v = rng.standard_normal((N, D))
    g = rng.standard_normal((M, D))
    return q, k, v, g


@pytest.mark.parametrize("M,N,D,causal", SHAPES)
def test_gradients_match_finite_differences(M, N, D, causal):
    q, k, v, g = _inputs(M, N, D, 100 + M * 10 + N)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, SCALE, causal)
    fq, fk, fv = _fd_grads(q, k, v, g, causal)
    for a, b in ((dq, fq), (dk, fk), (dv, fv)):
        assert np.max(np.abs(a - b)) <= 1e-7 * max(1.0, np.max(np.abs(b)))


@pytest.mark.parametrize("scale", [0.0, -0.75])
@pytest.mark.parametrize("M,N,D,causal", [(3, 5, 2, False), (6, 3, 2, True)])
def test_gradients_any_finite_scale(M, N, D, causal, scale):
    """Zero and negative scales (exact in fp32): the gradients still match
    central differences of the forward definition; at scale 0 dq and dk vanish
    (the scores do not depend on q or k)."""
    q, k, v, g = _inputs(M, N, D, 200 + M * 10 + N)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, scale, causal)
    fq, fk, fv = _fd_grads(q, k, v, g, causal, scale=scale)
    for a, b in ((dq, fq), (dk, fk), (dv, fv)):
        assert np.max(np.abs(a - b)) <= 1e-7 * max(1.0, np.max(np.abs(b)))
    if scale == 0.0:
        assert np.all(dq == 0.0) and np.all(dk == 0.0)


def _mutant(q, k, v, g, causal, defect):
    """head_bwd with one deliberate mistake (negative controls of the FD pin)."""
    s = SCALE
    M, N = q.shape[0], k.shape[0]
    vis = visible_mask(np.arange(M), N, M, causal)
    P, _, _ = masked_softmax(scores(q, k, s), vis)
    O = P @ v
    dP = g @ v.T
    delta = np.sum(g * O, axis=1)
    dV = P.T @ g
    if defect == "no_delta":
        dS = P * dP
    elif defect == "delta_sign":
        dS = P * (dP + delta[:, None])
    else:
        dS = P * (dP - delta[:, None])
    dQ = s * (dS @ k)
    dK = s * (dS.T @ q)
    if defect == "dk_untransposed":
        dK = s * (dS @ q)
    elif defect == "dq_no_scale":
        dQ = dS @ k
    elif defect == "dv_untransposed":
        dV = P @ g
    elif defect == "delta_from_dp":  # Delta as a plain row sum of dP, without the P weights
        dS = P * (dP - dP.sum(axis=1)[:, None])
        dQ = s * (dS @ k)
        dK = s * (dS.T @ q)
    return dQ, dK, dV


@pytest.mark.parametrize("defect", ["no_delta", "delta_sign", "dk_untransposed", "dq_no_scale",
                                    "dv_untransposed", "delta_from_dp"])
def test_finite_differences_reject_mutants(defect):
    q, k, v, g = _inputs(4, 4, 3, 7)
    mq, mk, mv = _mutant(q, k, v, g, False, defect)
    fq, fk, fv = _fd_grads(q, k, v, g, False)
    worst = max(np.max(np.abs(mq - fq)), np.max(np.abs(mk - fk)), np.max(np.abs(mv - fv)))
    assert worst > 1e-3
    # and the unmutated formulas pass on the same inputs
    dq, dk, dv = _mutant(q, k, v, g, False, "none")
    assert max(np.max(np.abs(dq - fq)), np.max(np.abs(dk - fk)), np.max(np.abs(dv - fv))) < 1e-7


def test_single_key_closed_form():
    # N = 1: P = 1 on every row, so dS = 0 (dQ = dK = 0) and dV_0 = sum_i dO_i.
    q, k, v, g = _inputs(5, 1, 3, 11)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, SCALE, False)
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    np.testing.assert_allclose(dv[0], g.sum(axis=0), rtol=0, atol=1e-14)


def test_equal_keys_give_zero_dq():
    # All keys equal: every row of S is constant, dS rows sum to 0, dQ = s*K_0*sum_j dS = 0.
    q, k, v, g = _inputs(6, 5, 4, 12)
    k[:] = k[0]
    dq, _, _ = oracle.attention_bwd(q, k, v, g, SCALE, False)
    assert np.max(np.abs(dq)) < 1e-14


@pytest.mark.parametrize("M,N,causal", [(9, 13, False), (13, 9, True), (11, 11, True)])
def test_sums_over_keys(M, N, causal):
    # Rows of P sum to 1 (or are empty): sum_j dV_j = sum of dO over non-empty rows.
    # Rows of dS sum to 0: sum_j dK_j = s * sum_i Q_i * sum_j dS_ij = 0.
    q, k, v, g = _inputs(M, N, 5, 13)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, SCALE, causal)
    nonempty = visible_mask(np.arange(M), N, M, causal).any(axis=1)
    np.testing.assert_allclose(dv.sum(axis=0), g[nonempty].sum(axis=0), rtol=0, atol=1e-12)
    assert np.max(np.abs(dk.sum(axis=0))) < 1e-12


def test_empty_rows_have_zero_dq_and_do_not_reach_dk_dv():
    M, N = 8, 3  # causal bottom-right: rows 0..4 see no key
    q, k, v, g = _inputs(M, N, 2, 14)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, SCALE, True)
    assert np.all(dq[:5] == 0.0)
    g2 = g.copy()
    g2[:5] = 123.0
    _, dk2, dv2 = oracle.attention_bwd(q, k, v, g2, SCALE, True)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2)


def test_rebuilt_p_matches_stored_p():
    # Module 08, Step 6: N = 1000, d = 64, standard normal Q and K; P rebuilt as
    # exp(S - L) from Q, K and the saved L matches the materialised P to rounding
    # error (the page printed 5.20e-17 for its draw).
    rng = np.random.default_rng(0)
    N, d = 1000, 64
    Q, K = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    scale = 1.0 / np.sqrt(d)  # 0.125: exact in fp32
    _, L, _, P = oracle.attention(Q, K, K, scale, False, return_sp=True)
    Pr = oracle.recompute_p(Q, K, L, scale, False)
    assert np.max(np.abs(Pr - P)) < 1e-15
    # causal with empty rows: rebuilt rows with L = -inf are exactly 0
    Qc, Kc = Q[:40], K[:25]
    _, Lc, _, Pc = oracle.attention(Qc, Kc, Kc, scale, True, return_sp=True)
    Prc = oracle.recompute_p(Qc, Kc, Lc, scale, True)
    assert np.max(np.abs(Prc - Pc)) < 1e-15
    assert np.all(Prc[:15] == 0.0)


def test_batched_heads_match_single_heads():
    rng = np.random.default_rng(15)
    q = rng.standard_normal((2, 3, 6, 4))
    k = rng.standard_normal((2, 3, 9, 4))
    v = rng.standard_normal((2, 3, 9, 4))
    g = rng.standard_normal((2, 3, 6, 4))
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, SCALE, True)
    for b in range(2):
        for h in range(3):
            a = oracle.attention_bwd(q[b, h], k[b, h], v[b, h], g[b, h], SCALE, True)
            assert np.array_equal(a[0], dq[b, h]) and np.array_equal(a[1], dk[b, h])
            assert np.array_equal(a[2], dv[b, h])
