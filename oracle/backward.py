"""Gradients of exact attention in fp64: the backward pass by recomputation.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``): callable only from tests,
``smoke()`` and the benchmark's CPU-baseline leg.

What the pages fix ("Module 08: FlashAttention and Memory-Efficient Kernels",
section "The backward pass: recompute instead of store" and Step 6 "memory
footprint and recomputation"): the forward pass keeps O and one number per row,
L = m + log(l); the backward pass rebuilds each tile of P as exp(S - L) from Q
and K instead of reading a stored N x N matrix.  Counting N x N x d matrix
products (the page's exercise "Price the recomputation"), the standard backward
has four and recomputation adds QK^T once more.

What the pages do not print: the gradient formulas.  They are the chain rule
applied to the definition in :mod:`oracle.definition` (a scalar loss with
dO = dLoss/dO given), with the softmax Jacobian
dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik):

    P        = exp(S - LSE) on visible entries, 0 elsewhere (recomputed)
    dV       = P^T dO
    dP       = dO V^T
    Delta_i  = sum_d dO[i, d] O[i, d]        (= sum_j P_ij dP_ij)
    dS       = P * (dP - Delta[:, None])
    dQ       = s dS K
    dK       = s dS^T Q

A row with no visible key has P = 0, so it contributes nothing and its dQ row
is 0.  Every formula is pinned in ``tests/test_oracle_backward.py`` against
central finite differences of the forward definition (which does not use these
formulas), against closed forms, and by mutants that each pin must reject.
"""

from __future__ import annotations

import numpy as np

from .definition import _as_f64, masked_softmax, scale_as_kernel, scores, visible_mask

__all__ = ["recompute_p", "attention_bwd", "head_bwd"]


def recompute_p(q, k, lse, scale: float, causal: bool) -> np.ndarray:
    """P rebuilt from Q, K and the saved per-row LSE: exp(S - LSE) where visible.

    One head: q [M, D], k [N, D], lse [M] -> P [M, N] (fp64).  Rows with
    LSE = -inf (no visible key) give P = 0.  This is the rebuild step of the
    Module 08 page's Step 6, applied to the whole matrix at once.
    """
    q, k = _as_f64(q), _as_f64(k)
    lse = np.asarray(lse, dtype=np.float64)
    M, N = q.shape[0], k.shape[0]
    s = scale_as_kernel(scale)
    vis = visible_mask(np.arange(M), N, M, causal)
    S = scores(q, k, s)
    finite = np.isfinite(lse)
    L = np.where(finite, lse, 0.0)
    with np.errstate(over="ignore"):
        P = np.where(vis & finite[:, None], np.exp(S - L[:, None]), 0.0)
    return P


def head_bwd(q, k, v, dout, s: float, causal: bool, return_parts: bool = False):
    """Gradients for one head (fp64 arrays): returns (dq, dk, dv[, parts])."""
    M, N = q.shape[0], k.shape[0]
    vis = visible_mask(np.arange(M), N, M, causal)
    S = scores(q, k, s)
    P, _, lse = masked_softmax(S, vis)
    O = P @ v
    dV = P.T @ dout
    dP = dout @ v.T
    delta = np.sum(dout * O, axis=1)
    dS = P * (dP - delta[:, None])
    dQ = s * (dS @ k)
    dK = s * (dS.T @ q)
    if return_parts:
        return dQ, dK, dV, dict(P=P, dP=dP, dS=dS, delta=delta, O=O, lse=lse, S=S)
    return dQ, dK, dV


def attention_bwd(q, k, v, dout, scale: float, causal: bool = False, return_parts: bool = False):
    """Gradients of attention for q [..., M, D], k/v [..., N, D], dout [..., M, D].

    Leading dimensions are heads.  Returns (dq, dk, dv) in fp64 with the shapes
    of q, k, v; with ``return_parts`` also a list of per-head dicts holding P,
    dP, dS, Delta, O and LSE.
    """
    q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    s = scale_as_kernel(scale)
    lead = q.shape[:-2]
    M, D = q.shape[-2:]
    N = k.shape[-2]
    nh = int(np.prod(lead, dtype=np.int64))
    qf, kf = q.reshape(nh, M, D), k.reshape(nh, N, D)
    vf, gf = v.reshape(nh, N, v.shape[-1]), dout.reshape(nh, M, v.shape[-1])
    dq, dk, dv = np.empty_like(qf), np.empty_like(kf), np.empty_like(vf)
    parts = []
    for h in range(nh):
        res = head_bwd(qf[h], kf[h], vf[h], gf[h], s, causal, return_parts)
        dq[h], dk[h], dv[h] = res[0], res[1], res[2]
        if return_parts:
            parts.append(res[3])
    out = (dq.reshape(q.shape), dk.reshape(k.shape), dv.reshape(v.shape))
    return out + (parts,) if return_parts else out
