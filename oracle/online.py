"""The streaming (online-softmax) recurrence, written out step by step in fp64.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).  Nothing here is the
reference result: :func:`oracle.definition.attention` is.  These functions exist
so that the recurrence the HIP kernel implements can itself be pinned - against
the pages' printed trace and worked example, and against the definition for
every block split - and so that the failure modes the pages name can be planted
and shown to be caught.

Recurrence (per query row, per new tile ``c`` of scaled scores), as described in
"Tiling and the online softmax" on the Module 08 page and "How can softmax work
a tile at a time?" on the FlashAttention-in-Triton page:

    m_new = max(m, max(c))
    alpha = exp(m - m_new)               (rescales everything seen so far)
    p     = exp(c - m_new)
    l     = l * alpha + sum(p)
    acc   = acc * alpha + p V_tile       (acc is kept un-normalised)
    m     = m_new
    ...after the last tile:  O = acc / l,  LSE = m + log(l)

starting from m = -inf, l = 0, acc = 0.  The loop order is the one where the
outer loop runs over blocks of Q and the inner loop over blocks of K/V with a
single final division (the arrangement the Module 08 page describes for
FlashAttention-2 in "Related ideas" and asks for in its "Project").

Base two (the "FlashAttention-style kernel" page, "The loop"): the scale is
multiplied by log2(e) once so that every exponential is exp2; the max and all
differences are then in base-2 units and LSE = ln(2) * (m2 + log2(l)).

Failure modes the pages name, available as switches for negative-control tests:

* ``rescale=False``: the ``acc * alpha`` / ``l * alpha`` terms dropped ("Things
  that break"; Module 08 Step 3's "without rescaling").
* ``alpha_base_e=True``: alpha computed with base e in a base-two loop ("Things
  that break": off by a smooth factor).
* ``guard=False``: no clamp of an all-masked running max, so -inf - (-inf)
  gives NaN (Module 08 Step 3 and "Common mistakes").
* ``sentinel=-1e6``: masking with a finite sentinel instead of -inf ("Causal
  masking": the sentinel becomes the max and inflates the running sum).
* ``reverse=True``: visit K/V blocks last-to-first (Module 08 "Practice" 2).
"""

from __future__ import annotations

import math

import numpy as np

__all__ = ["online_softmax_trace", "tiled_attention", "LOG2E", "LN2"]

LOG2E = 1.0 / math.log(2.0)
LN2 = math.log(2.0)


def online_softmax_trace(x, chunk, rescale: bool = True):
    """Stream one row of scores in chunks; return (m, l, history).

    ``chunk`` is a chunk length, or a sequence of chunk lengths (any split of
    the row).  ``history`` holds (m, l) after each chunk.  Natural-base, as in
    the Module 08 page's Step 3.  With ``rescale=False`` the old sum is not
    multiplied by exp(m_old - m_new) (the mistake that step demonstrates).
    """
    x = np.asarray(x, dtype=np.float64)
    if isinstance(chunk, (int, np.integer)):
        bounds = list(range(0, x.shape[0], int(chunk))) + [x.shape[0]]
    else:
        bounds = list(np.concatenate([[0], np.cumsum(chunk)]).astype(int))
        if bounds[-1] != x.shape[0]:
            raise ValueError("chunk lengths must sum to the row length")
    m, l = -np.inf, 0.0
    hist = []
    for start, stop in zip(bounds[:-1], bounds[1:]):
        c = x[start:stop]
        m_new = max(m, c.max())
        if rescale:
            l = l * np.exp(m - m_new) + np.exp(c - m_new).sum()
        else:
            l = l + np.exp(c - m_new).sum()
        m = m_new
        hist.append((m, l))
    return m, l, hist


def tiled_attention(q, k, v, scale: float, causal: bool = False,
                    block_m: int = 16, block_n: int = 16, *,
                    base2: bool = True, rescale: bool = True,
                    alpha_base_e: bool = False, guard: bool = True,
                    sentinel: float | None = None, reverse: bool = False,
                    skip_masked_tiles: bool = True, history: list | None = None):
    """Tiled exact attention for one head by the online recurrence (fp64).

    q: [M, D], k: [N, D], v: [N, Dv].  Returns (O, LSE, m, l) where m is in the
    base used (base-2 units when ``base2``) and LSE is natural log.  A row that
    never saw a visible key returns O = 0 and LSE = -inf when ``guard`` is on.

    Causal mask: key j visible to row i iff ``j <= i + (N - M)``.  With
    ``skip_masked_tiles`` a (Q block, K/V block) pair whose keys are all beyond
    every row's diagonal is skipped through the loop bounds, as a kernel does.
    ``history`` (if a list) receives (m, l, acc) copies after every K/V block
    for the first row block, for worked-example checks.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    M, N = q.shape[0], k.shape[0]
    s = float(np.float64(np.float32(scale)))
    c = s * LOG2E if base2 else s
    ex = np.exp2 if base2 else np.exp
    ex_alpha = np.exp if alpha_base_e else ex
    mask_value = -np.inf if sentinel is None else sentinel

    O = np.zeros((M, v.shape[1]))
    LSE = np.zeros(M)
    m_out = np.zeros(M)
    l_out = np.zeros(M)
    for i0 in range(0, M, block_m):
        rows = np.arange(i0, min(i0 + block_m, M))
        m = np.full(rows.shape[0], -np.inf)
        l = np.zeros(rows.shape[0])
        acc = np.zeros((rows.shape[0], v.shape[1]))
        starts = list(range(0, N, block_n))
        if reverse:
            starts = starts[::-1]
        for j0 in starts:
            cols = np.arange(j0, min(j0 + block_n, N))
            if causal and skip_masked_tiles and j0 > rows[-1] + (N - M):
                continue  # every key of this block is beyond every row's diagonal
            t = c * (q[rows] @ k[cols].T)
            if causal:
                vis = cols[None, :] <= rows[:, None] + (N - M)
                t = np.where(vis, t, mask_value)
            m_new = np.maximum(m, t.max(axis=1))
            m_use = np.where(np.isneginf(m_new), 0.0, m_new) if guard else m_new
            with np.errstate(invalid="ignore", over="ignore"):
                alpha = ex_alpha(m - m_use)
                p = ex(t - m_use[:, None])
            if rescale:
                l = l * alpha + p.sum(axis=1)
                acc = acc * alpha[:, None] + p @ v[cols]
            else:
                l = l + p.sum(axis=1)
                acc = acc + p @ v[cols]
            m = m_new
            if history is not None and i0 == 0:
                history.append((m.copy(), l.copy(), acc.copy()))
        with np.errstate(invalid="ignore", divide="ignore"):
            if guard:
                empty = l == 0.0
                O[rows] = np.where(empty[:, None], 0.0, acc / np.where(empty, 1.0, l)[:, None])
                m_fin = np.where(np.isneginf(m), 0.0, m)
            else:
                O[rows] = acc / l[:, None]
                m_fin = m
            lse = (m_fin + np.log2(l)) * LN2 if base2 else m_fin + np.log(l)
        LSE[rows] = lse
        m_out[rows] = m
        l_out[rows] = l
    return O, LSE, m_out, l_out
