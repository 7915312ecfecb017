"""Failure modes the pages name, planted in the oracle's recurrence helper on the
CPU, must be visible to the checks (no GPU).

* "Things that break" (FlashAttention-style kernel page): a dropped acc*alpha is
  right within one tile and wrong beyond it; a base-e alpha in a base-2 loop is
  off by a smooth factor.
* "Causal masking" (same page): a finite -1e6 sentinel on a fully masked tile
  becomes the max and inflates the running sum.
* Module 08 "Practice" 2 and "Common mistakes": a reversed causal loop without
  the clamp of an all-masked max produces NaN rows; with it, none.
"""

import numpy as np

from oracle import attention, tiled_attention


def _data(M, N, D, seed, qmult=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((M, D)) * qmult, rng.standard_normal((N, D)),
            rng.standard_normal((N, D)))


def test_missing_rescale_only_visible_beyond_one_tile():
    q, k, v = _data(16, 64, 8, 1, qmult=3.0)
    O, L = attention(q, k, v, 0.5)
    O1, _, _, _ = tiled_attention(q, k, v, 0.5, block_m=16, block_n=64, rescale=False)
    assert np.abs(O1 - O).max() <= 1e-12          # one tile: still right
    O4, _, _, _ = tiled_attention(q, k, v, 0.5, block_m=16, block_n=16, rescale=False)
    assert np.abs(O4 - O).max() > 1e-2            # four tiles: wrong


def test_base_e_alpha_in_base_two_loop_is_off():
    q, k, v = _data(16, 64, 8, 2, qmult=3.0)
    O, L = attention(q, k, v, 0.5)
    Ob, Lb, _, _ = tiled_attention(q, k, v, 0.5, block_n=16, alpha_base_e=True)
    assert np.abs(Ob - O).max() > 1e-3
    Og, _, _, _ = tiled_attention(q, k, v, 0.5, block_n=16)
    assert np.abs(Og - O).max() <= 1e-12


def _expected_nan_rows(M, N, bm, bn):
    """Rows whose first visited (reversed, not skipped) K/V block has no key they
    can see: their running max is -inf there and -inf - (-inf) poisons them."""
    bad = 0
    for i0 in range(0, M, bm):
        rows = range(i0, min(i0 + bm, M))
        starts = [j0 for j0 in range(0, N, bn) if not j0 > rows[-1] + (N - M)]
        first = max(starts)
        bad += sum(1 for i in rows if first > i + (N - M))
    return bad


def test_reversed_causal_loop_nan_rows_and_guard():
    M = N = 300
    q, k, v = _data(M, N, 64, 3)
    O_bad, _, _, _ = tiled_attention(q, k, v, 1 / 8, True, 64, 100, reverse=True, guard=False)
    nan_rows = int(np.isnan(O_bad).any(axis=1).sum())
    assert nan_rows == _expected_nan_rows(M, N, 64, 100) == 44
    O_ok, L_ok, _, _ = tiled_attention(q, k, v, 1 / 8, True, 64, 100, reverse=True, guard=True)
    O, L = attention(q, k, v, 1 / 8, True)
    assert not np.isnan(O_ok).any()
    assert np.abs(O_ok - O).max() <= 1e-12 and np.abs(L_ok - L).max() <= 1e-12


def test_finite_sentinel_inflates_running_sum():
    # causal with M > N: rows 0..23 see no key, yet their tile is visited (it is
    # not wholly beyond the block's last row).  A -1e6 sentinel becomes their max,
    # every masked lane exponentiates to one and the sum counts masked keys.
    M, N = 40, 16
    q, k, v = _data(M, N, 16, 4)
    O, L = attention(q, k, v, 0.25, True)
    Os, Ls, _, ls = tiled_attention(q, k, v, 0.25, True, 32, 16, sentinel=-1e6)
    Og, Lg, _, lg = tiled_attention(q, k, v, 0.25, True, 32, 16)
    empty = np.arange(M) < M - N
    assert np.all(lg[empty] == 0.0) and np.all(ls[empty] == N)   # sum inflated
    assert np.abs(Os[empty]).max() > 1e-2 and np.all(O[empty] == 0.0)
    assert np.array_equal(Og, np.where(np.isnan(Og), 0, Og)) and np.abs(Og - O).max() <= 1e-12
    # a real key later in the row clears the inflation (alpha underflows to 0)
    Or, _, _, _ = tiled_attention(q[:16], k, v, 0.25, True, 16, 4, reverse=True, sentinel=-1e6)
    Od, _ = attention(q[:16], k, v, 0.25, True)
    assert np.abs(Or - Od).max() <= 1e-12

