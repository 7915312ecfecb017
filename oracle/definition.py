"""Exact attention by its definition, in fp64, materialising S and P.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``): callable only from tests,
``smoke()`` and the benchmark's CPU-baseline leg.

What is computed, per (batch, head), following the definition of standard
attention on the "Module 08: FlashAttention and Memory-Efficient Kernels" page
(section "Where the time goes in standard attention" and the ``softmax`` /
``standard_attention`` functions of its Step 1) and the problem statement on the
"FlashAttention in Triton" page (section "First, what does attention actually
do?": Q has M rows, K and V have N rows, all of width D, O is M x D):

    S[i, j]  = s * sum_d Q[i, d] K[j, d]            (s = the scale, see below)
    vis(i,j) = not causal  or  j <= i + (N - M)      (bottom-right aligned mask)
    m[i]     = max_{j visible} S[i, j]
    P[i, j]  = exp(S[i, j] - m[i]) / sum_{j' visible} exp(S[i, j'] - m[i])
               for visible j, and 0 otherwise
    O[i, :]  = sum_j P[i, j] V[j, :]
    LSE[i]   = m[i] + log(sum_{j visible} exp(S[i, j] - m[i]))

The log-sum-exp is the one number per row kept for the backward pass
("The backward pass: recompute instead of store" on the Module 08 page:
L = m + log(l)).

Readings where the pages are silent:

* Causal alignment when M != N: the pages only show square masks (``np.tril`` /
  ``cols <= rows``).  Bottom-right alignment ``j <= i + N - M`` is used; it is
  the same mask when M == N.
* A row with no visible key (possible only when causal and M > N): the pages
  name the NaN failure and the guard "clamp an infinite running max to 0"
  (Module 08, "Common mistakes"), but no output value.  With the clamp the sum
  is 0, so LSE = 0 + log 0 = -inf; O is 0/0 and is defined here as 0.
* The scale is the fp32 value the kernel receives, widened exactly:
  ``s = float64(float32(scale))``.
* Inputs in fp16/bf16/fp32 are widened exactly to fp64 before any arithmetic.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "scale_as_kernel",
    "visible_mask",
    "scores",
    "masked_softmax",
    "attention",
    "attention_rows",
]


def scale_as_kernel(scale: float) -> float:
    """The scale as the library receives it (an fp32 argument), widened to fp64."""
    return float(np.float64(np.float32(scale)))


def visible_mask(rows: np.ndarray, N: int, M: int, causal: bool) -> np.ndarray:
    """Boolean [len(rows), N]: key j is visible to query row i.

    Non-causal: every key.  Causal: ``j <= i + (N - M)`` (bottom-right corner
    alignment; identical to the pages' lower-triangular mask when M == N).
    """
    rows = np.asarray(rows, dtype=np.int64)
    if not causal:
        return np.ones((rows.shape[0], N), dtype=bool)
    cols = np.arange(N, dtype=np.int64)[None, :]
    return cols <= (rows[:, None] + (N - M))


def scores(q: np.ndarray, k: np.ndarray, s: float) -> np.ndarray:
    """S = s * Q K^T for one head, fp64.  q: [R, D], k: [N, D] -> [R, N]."""
    return s * (q @ k.T)


def masked_softmax(S: np.ndarray, vis: np.ndarray):
    """Row softmax of S over the visible entries (stable form: subtract the row max).

    Returns (P, m, lse).  A row with no visible entry gets P = 0, m = -inf and
    lse = -inf (the clamped-max reading described in the module docstring).
    """
    Sm = np.where(vis, S, -np.inf)
    m = np.max(Sm, axis=1, initial=-np.inf)  # N = 0 leaves every row empty
    empty = ~vis.any(axis=1)
    m_safe = np.where(empty, 0.0, m)
    e = np.where(vis, np.exp(Sm - m_safe[:, None]), 0.0)
    l = e.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        P = np.where(empty[:, None], 0.0, e / np.where(empty, 1.0, l)[:, None])
        lse = m_safe + np.log(l)  # log(0) = -inf for an empty row
    return P, m, lse


def _as_f64(x) -> np.ndarray:
    """Exact widening of a numpy array or torch CPU tensor (fp16/bf16/fp32/fp64)."""
    if hasattr(x, "detach"):  # torch tensor: bf16 has no numpy dtype, widen in torch
        import torch

        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _head(q, k, v, s, causal, rows, return_sp=False):
    M = q.shape[0]
    N = k.shape[0]
    vis = visible_mask(rows, N, M, causal)
    S = scores(q[rows], k, s)
    P, m, lse = masked_softmax(S, vis)
    O = P @ v
    if return_sp:
        return O, lse, S, P
    return O, lse


def attention(q, k, v, scale: float, causal: bool = False, return_sp: bool = False):
    """Full attention for q [..., M, D], k/v [..., N, D] (leading dims are heads).

    Returns (O [..., M, D], LSE [..., M]) in fp64; with ``return_sp`` also the
    materialised S and P ([..., M, N]).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    s = scale_as_kernel(scale)
    lead = q.shape[:-2]
    M, D = q.shape[-2:]
    N = k.shape[-2]
    nh = int(np.prod(lead, dtype=np.int64))
    qf = q.reshape(nh, M, D)
    kf = k.reshape(nh, N, k.shape[-1])
    vf = v.reshape(nh, N, v.shape[-1])
    Dv = vf.shape[-1]
    O = np.empty((qf.shape[0], M, Dv))
    L = np.empty((qf.shape[0], M))
    Ss, Ps = [], []
    rows = np.arange(M)
    for h in range(qf.shape[0]):
        res = _head(qf[h], kf[h], vf[h], s, causal, rows, return_sp)
        O[h], L[h] = res[0], res[1]
        if return_sp:
            Ss.append(res[2])
            Ps.append(res[3])
    O = O.reshape(*lead, M, Dv)
    L = L.reshape(*lead, M)
    if return_sp:
        S = np.stack(Ss).reshape(*lead, M, N)
        P = np.stack(Ps).reshape(*lead, M, N)
        return O, L, S, P
    return O, L


def attention_rows(q, k, v, scale: float, causal: bool, rows):
    """Attention for selected query rows only, one head at a time.

    q: [H, M, D], k/v: [H, N, D] (leading dims already flattened to H heads).
    rows: [H, R] int array (the rows to compute for each head) or [R] shared.
    Returns (O [H, R, D], LSE [H, R]) in fp64.  Each selected row is computed
    against all N keys exactly as in :func:`attention`.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    s = scale_as_kernel(scale)
    H = q.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    if rows.ndim == 1:
        rows = np.broadcast_to(rows, (H, rows.shape[0]))
    R = rows.shape[1]
    O = np.empty((H, R, v.shape[-1]))
    L = np.empty((H, R))
    for h in range(H):
        O[h], L[h] = _head(q[h], k[h], v[h], s, causal, rows[h])
    return O, L
