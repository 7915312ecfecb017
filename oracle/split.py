"""Attention over key chunks and the merge of the partial results, in fp64.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``): callable only from tests,
``smoke()`` and the benchmark's CPU-baseline leg.

The merge is the concatenation algebra the "Module 08: FlashAttention and
Memory-Efficient Kernels" page states in "Tiling and the online softmax": the
softmax of a concatenation follows from the maxima and sums of its pieces.  For
key chunks g with partial results (O_g, LSE_g) -- attention restricted to the
chunk's keys, O_g already normalised over them -- the full result is

    LSE = log sum_g exp(LSE_g),     O = sum_g exp(LSE_g - LSE) * O_g,

computed with the largest LSE_g subtracted first.  A chunk in which a row sees
no key has LSE_g = -inf and weight 0; a row that sees no key in any chunk ends
with LSE = -inf and O = 0, the same reading as the definition's empty row.

Visibility stays global: key j (in the whole [0, N)) is visible to row i iff
not causal or j <= i + N - M, whichever chunk holds it.
"""

from __future__ import annotations

import numpy as np

from .definition import _as_f64, masked_softmax, scale_as_kernel, scores, visible_mask

__all__ = ["partial_attention", "merge_partials", "split_attention"]


def partial_attention(q, k, v, scale: float, causal: bool, lo: int, hi: int):
    """(O_g, LSE_g) of one head over the keys [lo, hi), with the global mask.

    q [M, D], k/v [N, D] (the whole key range) -> O_g [M, D], LSE_g [M] (fp64).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    M, N = q.shape[0], k.shape[0]
    s = scale_as_kernel(scale)
    vis = visible_mask(np.arange(M), N, M, causal)[:, lo:hi]
    S = scores(q, k[lo:hi], s)
    P, _, lse = masked_softmax(S, vis)
    return P @ v[lo:hi], lse


def merge_partials(O_parts, L_parts):
    """Merge partial results: O_parts [G, M, D], L_parts [G, M] -> (O [M, D], LSE [M])."""
    O_parts = np.asarray(O_parts, dtype=np.float64)
    L_parts = np.asarray(L_parts, dtype=np.float64)
    m = np.max(L_parts, axis=0, initial=-np.inf)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(L_parts - m_safe[None, :])          # exp(-inf) = 0 for empty chunks
    total = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = m_safe + np.log(total)                # -inf where every chunk is empty
        O = np.where(empty[:, None], 0.0,
                     np.einsum("gm,gmd->md", w, O_parts) / np.where(empty, 1.0, total)[:, None])
    return O, lse


def split_attention(q, k, v, scale: float, causal: bool, bounds):
    """Attention of one head computed chunk by chunk and merged.

    bounds: increasing key positions [0 = b_0, b_1, ..., b_G = N]; chunk g is
    [b_g, b_{g+1}).  Returns (O, LSE) as :func:`oracle.attention` would.
    """
    parts = [partial_attention(q, k, v, scale, causal, lo, hi)
             for lo, hi in zip(bounds[:-1], bounds[1:])]
    return merge_partials([p[0] for p in parts], [p[1] for p in parts])
