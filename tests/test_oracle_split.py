"""Pins of the chunked attention and merge helpers (oracle/split.py), CPU only.

* The three-key worked example of "FlashAttention in Triton", section "How can
  softmax work a tile at a time?", read in chunks of two keys then one: the
  merge must land on the printed l, O (and the exact LSE).
* Merged chunks equal the definition (oracle.attention) for random chunkings,
  both mask modes, both ways of M != N.
* Closed forms: one chunk is the definition itself; chunks a row cannot see
  carry weight 0; rows that see nothing anywhere are O = 0, LSE = -inf.
* Mutants of the merge (no max subtraction, no normalisation, plain average)
  must fail.
"""

from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle
from oracle.split import merge_partials, partial_attention, split_attention

HERE = os.path.dirname(os.path.abspath(__file__))


def test_worked_example_in_two_chunks():
    g = json.load(open(os.path.join(HERE, "golden", "worked_example_three_keys.json")))
    Q, K, V = (np.array(g[x]) for x in ("Q", "K", "V"))
    b = np.cumsum([0] + g["blocks"])  # [0, 2, 3]
    O, L = split_attention(Q, K, V, g["scale"], False, b)
    assert abs(O[0, 0] - g["final"]["O"]) <= g["tol"]
    assert abs(np.exp(L[0] - 3.0) - g["final"]["l"]) <= g["tol"]  # l relative to the max 3
    assert abs(O[0, 0] - 25.752104) < 1e-6 and abs(L[0] - 3.407606) < 1e-6


def _rand(M, N, D, seed, qmul=1.0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((M, D)) * qmul, rng.standard_normal((N, D)), rng.standard_normal((N, D))


@pytest.mark.parametrize("M,N,causal,seed", [
    (17, 50, False, 1), (50, 17, True, 2), (40, 40, True, 3), (9, 200, True, 4), (64, 130, False, 5),
])
def test_merged_chunks_equal_the_definition(M, N, causal, seed):
    q, k, v = _rand(M, N, 8, seed, qmul=3.0)
    O_ref, L_ref = oracle.attention(q, k, v, 0.35, causal)
    rng = np.random.default_rng(100 + seed)
    for G in (1, 2, 3, 7):
        cuts = np.sort(rng.choice(np.arange(1, N), size=min(G - 1, N - 1), replace=False))
        b = np.concatenate([[0], cuts, [N]])
        O, L = split_attention(q, k, v, 0.35, causal, b)
        fin = np.isfinite(L_ref)
        assert np.array_equal(np.isneginf(L), np.isneginf(L_ref))
        assert np.max(np.abs(O - O_ref)) < 1e-13
        assert np.max(np.abs(L[fin] - L_ref[fin]), initial=0.0) < 1e-13


def test_one_chunk_is_the_definition():
    q, k, v = _rand(20, 30, 4, 7)
    O_ref, L_ref = oracle.attention(q, k, v, 0.5, True)
    O, L = split_attention(q, k, v, 0.5, True, [0, 30])
    assert np.array_equal(O, O_ref) and np.array_equal(L, L_ref)


def test_invisible_chunks_and_empty_rows():
    # M = 12 > N = 8, causal: row i sees keys j <= i - 4, rows 0..3 see none.
    q, k, v = _rand(12, 8, 3, 8)
    O1, L1 = partial_attention(q, k, v, 0.5, True, 4, 8)  # keys 4..7: rows 0..7 see none of them
    assert np.all(np.isneginf(L1[:8])) and np.all(O1[:8] == 0.0)
    O, L = split_attention(q, k, v, 0.5, True, [0, 4, 8])
    assert np.all(np.isneginf(L[:4])) and np.all(O[:4] == 0.0)
    O_ref, L_ref = oracle.attention(q, k, v, 0.5, True)
    assert np.max(np.abs(O - O_ref)) < 1e-14


def test_merge_is_order_independent():
    q, k, v = _rand(10, 60, 5, 9, qmul=4.0)
    b = [0, 11, 29, 30, 60]
    parts = [partial_attention(q, k, v, 0.4, False, lo, hi) for lo, hi in zip(b[:-1], b[1:])]
    O1, L1 = merge_partials([p[0] for p in parts], [p[1] for p in parts])
    O2, L2 = merge_partials([p[0] for p in parts[::-1]], [p[1] for p in parts[::-1]])
    assert np.max(np.abs(O1 - O2)) < 1e-14 and np.max(np.abs(L1 - L2)) < 1e-14


def _mutant_merge(O_parts, L_parts, defect):
    O_parts, L_parts = np.asarray(O_parts), np.asarray(L_parts)
    if defect == "average":
        return O_parts.mean(axis=0), np.log(np.exp(L_parts).sum(axis=0))
    w = np.exp(L_parts)  # no max subtraction
    if defect == "unnormalised":
        return np.einsum("gm,gmd->md", w, O_parts), np.log(w.sum(axis=0))
    if defect == "no_max":
        return np.einsum("gm,gmd->md", w, O_parts) / w.sum(axis=0)[:, None], np.log(w.sum(axis=0))
    raise ValueError(defect)


@pytest.mark.parametrize("defect,qmul", [
    ("average", 3.0), ("unnormalised", 3.0),  # wrong algebra at ordinary logits
    ("no_max", 400.0),                         # LSE > 709: exp overflows without the max
])
def test_merge_mutants_fail(defect, qmul):
    q, k, v = _rand(16, 90, 8, 10, qmul=qmul)
    O_ref, L_ref = oracle.attention(q, k, v, 1.0, False)
    b = [0, 30, 60, 90]
    parts = [partial_attention(q, k, v, 1.0, False, lo, hi) for lo, hi in zip(b[:-1], b[1:])]
    with np.errstate(all="ignore"):
        O, L = _mutant_merge([p[0] for p in parts], [p[1] for p in parts], defect)
        bad = (not np.all(np.isfinite(O))) or np.max(np.abs(O - O_ref)) > 1e-6 \
            or (not np.all(np.isfinite(L))) or np.max(np.abs(L - L_ref)) > 1e-6
    assert bad
