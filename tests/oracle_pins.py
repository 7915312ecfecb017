"""Pins of the CPU oracle: checks against values the pages print, closed forms,
invariants, library routines and brute force.  None of them re-derives the
oracle's own formula.  Each function raises (AssertionError or otherwise) when
the oracle is wrong; ``test_oracle_pins.py`` runs them, and
``test_oracle_mutations.py`` plants mistakes in the oracle and checks that at
least one of them fails for every mistake.
"""

from __future__ import annotations

import itertools
import json
import math
import os
import struct

import numpy as np

import oracle
from oracle import attention, attention_rows, online_softmax_trace, tiled_attention
from oracle.definition import masked_softmax

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _f32(x: float) -> float:
    """x rounded to IEEE binary32 (round to nearest even) through its byte
    encoding, independently of the oracle's own rounding helper."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


# ---------------------------------------------------------------- printed values

def pin_worked_example_definition():
    """Three-key worked example (FlashAttention in Triton, 'How can softmax work a
    tile at a time?'): denominator ~1.503, weighted sum ~38.711, output ~25.752."""
    g = _golden("worked_example_three_keys.json")
    Q, K, V = (np.array(g[x]) for x in ("Q", "K", "V"))
    O, L = attention(Q, K, V, g["scale"])
    m = 3.0  # largest scaled score
    l = math.exp(L[0] - m)
    tol = g["tol"]
    assert abs(O[0, 0] - g["final"]["O"]) <= tol, O
    assert abs(l - g["final"]["l"]) <= tol, l
    assert abs(O[0, 0] * l - g["final"]["acc"]) <= tol
    # closed form of the same example (full precision)
    e = [math.exp(1 - 3), math.exp(2 - 3), 1.0]
    exact_O = (10 * e[0] + 20 * e[1] + 30 * e[2]) / sum(e)
    assert abs(O[0, 0] - exact_O) <= 1e-13
    assert abs(L[0] - (3.0 + math.log(sum(e)))) <= 1e-13


def pin_worked_example_recurrence():
    """Same example streamed in blocks of two then one key: the weights after the
    first block are ~[0.368, 1]; after the second they are rescaled to
    ~[0.135, 0.368] and the new key adds 1 (both bases)."""
    g = _golden("worked_example_three_keys.json")
    Q, K, V = (np.array(g[x]) for x in ("Q", "K", "V"))
    tol = g["tol"]
    for base2 in (False, True):
        hist = []
        O, L, m, l = tiled_attention(Q, K, V, g["scale"], block_m=1, block_n=g["blocks"][0],
                                     base2=base2, history=hist)
        assert len(hist) == 2
        (m1, l1, a1), (m2, l2, a2) = hist
        unit = 1.0 / math.log(2.0) if base2 else 1.0
        assert abs(m1[0] / unit - g["after_first_block"]["m"]) <= 1e-12
        assert abs(l1[0] - sum(g["after_first_block"]["weights"])) <= 2 * tol
        w_old = g["after_second_block"]["rescaled_old_weights"]
        assert abs(m2[0] / unit - g["after_second_block"]["m"]) <= 1e-12
        assert abs(l2[0] - (sum(w_old) + g["after_second_block"]["new_weight"])) <= 2 * tol
        assert abs(l2[0] - g["final"]["l"]) <= tol
        assert abs(a2[0, 0] - g["final"]["acc"]) <= tol
        assert abs(O[0, 0] - g["final"]["O"]) <= tol


def pin_online_trace_printed():
    """Module 08 Step 3: seeded row, chunks of four, printed (m, l) per chunk."""
    g = _golden("online_softmax_trace.json")
    x = np.random.default_rng(g["seed"]).standard_normal(g["n"]) * g["multiplier"]
    _, _, hist = online_softmax_trace(x, g["chunk"])
    for (m, l), pm, pl in zip(hist, g["printed_m"], g["printed_l"]):
        assert abs(m - pm) <= g["printed_tol"], (m, pm)
        assert abs(l - pl) <= g["printed_tol"], (l, pl)


def pin_online_trace_equals_definition():
    """Module 08 Step 3: 'max |online - reference|: 0.0' - the streamed (m, l)
    reproduce the one-shot softmax row of the definition exactly."""
    g = _golden("online_softmax_trace.json")
    x = np.random.default_rng(g["seed"]).standard_normal(g["n"]) * g["multiplier"]
    m, l, _ = online_softmax_trace(x, g["chunk"])
    P, _, _ = masked_softmax(x[None, :], np.ones((1, x.shape[0]), dtype=bool))
    assert np.abs(np.exp(x - m) / l - P[0]).max() <= g["max_abs_online_minus_reference"] + 1e-16


def pin_online_trace_without_rescale():
    """Module 08 Step 3: dropping the rescale term gives max error 0.2700173732766699."""
    g = _golden("online_softmax_trace.json")
    x = np.random.default_rng(g["seed"]).standard_normal(g["n"]) * g["multiplier"]
    P, _, _ = masked_softmax(x[None, :], np.ones((1, x.shape[0]), dtype=bool))
    m, l, _ = online_softmax_trace(x, g["chunk"], rescale=False)
    err = np.abs(np.exp(x - m) / l - P[0]).max()
    assert abs(err - g["without_rescaling_max_error"]) <= 1e-15, err
    with np.errstate(invalid="ignore"):
        assert np.isnan(np.exp(-np.inf - -np.inf)) == g["exp_neginf_minus_neginf_is_nan"]


def pin_flop_formula():
    """Module 08 Step 4 prints 256,000,000 matmul FLOPs at N = 1000, d = 64."""
    from workloads import exact_flops, metric_flops, visible_pairs

    g = _golden("flop_count.json")
    N, d = g["N"], g["d"]
    assert metric_flops(1, 1, N, N, d, False) == g["matmul_flops_standard"]
    assert exact_flops(1, 1, N, N, d, False) == g["matmul_flops_tiled"]
    for M, Nk in [(1, 1), (3, 7), (7, 3), (13, 13), (5, 1), (1, 5)]:
        vis = oracle.visible_mask(np.arange(M), Nk, M, True)
        assert visible_pairs(M, Nk, True) == int(vis.sum())
        brute = sum(1 for i in range(M) for j in range(Nk) if j <= i + Nk - M)
        assert brute == int(vis.sum())


# ---------------------------------------------------------------- brute force

def _brute(q, k, v, s, causal):
    """Pure-Python triple loop (math.exp / math.fsum), independent of numpy."""
    M, D = len(q), len(q[0])
    N = len(k)
    O = [[0.0] * len(v[0]) for _ in range(M)]
    L = [0.0] * M
    for i in range(M):
        vis = [j for j in range(N) if (not causal) or j <= i + N - M]
        if not vis:
            L[i] = -math.inf
            continue
        sc = {j: s * math.fsum(q[i][d] * k[j][d] for d in range(D)) for j in vis}
        mx = max(sc.values())
        w = {j: math.exp(sc[j] - mx) for j in vis}
        tot = math.fsum(w.values())
        for c in range(len(v[0])):
            O[i][c] = math.fsum(w[j] * v[j][c] for j in vis) / tot
        L[i] = mx + math.log(tot)
    return O, L


def pin_brute_force():
    """Tiny shapes, M != N both ways, causal and not: definition vs brute force."""
    rng = _rng(7)
    for M, N, D, causal in itertools.product([1, 2, 3, 7, 13], [1, 2, 3, 7, 13], [1, 3, 8],
                                             [False, True]):
        if (M * N * D) % 5 and M != N and D == 3:
            continue  # thin the grid; every (M, N) pair is still covered with D = 1 and 8
        q = rng.standard_normal((M, D)) * 2.0
        k = rng.standard_normal((N, D))
        v = rng.standard_normal((N, D + 1))  # value width differs from D on purpose
        s = 0.7
        O, L = attention(q, k, v, s, causal)
        Ob, Lb = _brute(q.tolist(), k.tolist(), v.tolist(), _f32(s), causal)
        Ob, Lb = np.array(Ob), np.array(Lb)
        assert np.array_equal(np.isneginf(L), np.isneginf(Lb)), (M, N, D, causal)
        fin = np.isfinite(Lb)
        assert np.abs(L[fin] - Lb[fin]).max(initial=0.0) <= 1e-12, (M, N, D, causal)
        assert np.abs(O - Ob).max() <= 1e-12, (M, N, D, causal)


# ---------------------------------------------------------------- library routines

def pin_torch_sdpa_fp64():
    """PyTorch's own CPU scaled_dot_product_attention (math path, fp64) with an
    explicit bottom-right boolean mask, and scipy's logsumexp for LSE."""
    import torch
    import torch.nn.functional as F
    from scipy.special import logsumexp

    rng = _rng(11)
    for M, N, D, causal in [(33, 70, 16, False), (70, 70, 24, True), (40, 90, 8, True),
                            (64, 129, 128, False)]:
        q = rng.standard_normal((2, 3, M, D))
        k = rng.standard_normal((2, 3, N, D))
        v = rng.standard_normal((2, 3, N, D))
        s = 1.0 / math.sqrt(D)
        O, L = attention(q, k, v, s, causal)
        s64 = _f32(s)
        mask = None
        if causal:
            mask = torch.from_numpy(np.arange(N)[None, :] <= np.arange(M)[:, None] + (N - M))
        Ot = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                            torch.from_numpy(v), attn_mask=mask, scale=s64)
        assert np.abs(O - Ot.numpy()).max() <= 1e-12
        S = s64 * np.einsum("bhmd,bhnd->bhmn", q, k)
        if causal:
            S = np.where(mask.numpy(), S, -np.inf)
        assert np.abs(L - logsumexp(S, axis=-1)).max() <= 1e-12


def pin_scipy_softmax_rows():
    """Materialised P equals scipy.special.softmax row by row and sums to 1."""
    from scipy.special import softmax

    rng = _rng(12)
    q = rng.standard_normal((20, 5)) * 3
    k = rng.standard_normal((31, 5))
    v = rng.standard_normal((31, 5))
    O, L, S, P = attention(q, k, v, 0.5, False, return_sp=True)
    assert np.abs(P - softmax(S, axis=-1)).max() <= 1e-14
    assert np.abs(P.sum(axis=-1) - 1.0).max() <= 1e-14
    assert np.abs(O - P @ v).max() <= 1e-14
    assert np.abs(S - _f32(0.5) * (q @ k.T)).max() <= 1e-13


# ---------------------------------------------------------------- the scale argument

def pin_scale_rounded_to_fp32():
    """The library receives the scale as an fp32 argument, so the oracle's scale
    is that fp32 value.  Literal binary32 values (nearest-even rounding):
    1/sqrt(128) -> 0.0883883461356163 (fp16 would give 0.08837890625),
    1/sqrt(96) -> 0.10206207633018494, 0.3 -> 0.30000001192092896; 1/8 and 0 are
    exact."""
    cases = [(1 / math.sqrt(128), 0.0883883461356163), (1 / math.sqrt(96), 0.10206207633018494),
             (0.3, 0.30000001192092896), (-0.3, -0.30000001192092896), (0.125, 0.125),
             (0.0, 0.0)]
    for x, want in cases:
        assert oracle.scale_as_kernel(x) == want, (x, oracle.scale_as_kernel(x), want)
        assert _f32(x) == want


def pin_scores_use_fp32_scale():
    """End to end: S built here with the scale rounded through its binary32
    encoding (no oracle helper) matches attention's S and LSE to 1e-13, at
    scales whose fp16, bf16 or unrounded values differ from the fp32 one by
    1e-8 .. 1e-3 relative (each far above the tolerance at these logits)."""
    rng = _rng(31)
    q = rng.standard_normal((6, 128)) * 3
    k = rng.standard_normal((9, 128))
    v = rng.standard_normal((9, 4))
    for x in (1 / math.sqrt(128), 1 / math.sqrt(96), 0.3, -0.3):
        s32 = _f32(x)
        O, L, S, P = attention(q, k, v, x, False, return_sp=True)
        S_here = s32 * (q @ k.T)
        assert np.abs(S - S_here).max() <= 1e-13, x
        mx = S_here.max(axis=1)
        L_here = mx + np.log(np.exp(S_here - mx[:, None]).sum(axis=1))
        assert np.abs(L - L_here).max() <= 1e-13, x


def pin_zero_scale_uniform():
    """scale = 0: every visible score is 0, so P is uniform over the visible
    keys, O is their mean and LSE = ln(#visible); empty rows stay O = 0,
    LSE = -inf."""
    rng = _rng(32)
    M, N = 13, 8
    q = rng.standard_normal((M, 5)) * 4
    k = rng.standard_normal((N, 5)) * 4
    v = rng.standard_normal((N, 3))
    for causal in (False, True):
        O, L = attention(q, k, v, 0.0, causal)
        for i in range(M):
            n = N if not causal else max(0, i + N - M + 1)
            if n == 0:
                assert np.all(O[i] == 0.0) and np.isneginf(L[i])
                continue
            assert abs(L[i] - math.log(n)) <= 1e-14
            assert np.abs(O[i] - v[:n].mean(axis=0)).max() <= 1e-14


def pin_negative_scale():
    """A negative scale weights the keys by exp(-|s| q.k): brute force on tiny
    shapes, and the exact identity attention(q, k, v, -s) = attention(-q, k, v, s)
    (negation is exact in binary floating point)."""
    rng = _rng(33)
    for M, N, D, causal in [(5, 7, 3, False), (7, 5, 4, True), (6, 6, 2, True)]:
        q = rng.standard_normal((M, D)) * 2
        k = rng.standard_normal((N, D))
        v = rng.standard_normal((N, 2))
        O, L = attention(q, k, v, -0.7, causal)
        Ob, Lb = _brute(q.tolist(), k.tolist(), v.tolist(), _f32(-0.7), causal)
        Ob, Lb = np.array(Ob), np.array(Lb)
        assert np.array_equal(np.isneginf(L), np.isneginf(Lb))
        fin = np.isfinite(Lb)
        assert np.abs(L[fin] - Lb[fin]).max(initial=0.0) <= 1e-12
        assert np.abs(O - Ob).max() <= 1e-12
        O2, L2 = attention(-q, k, v, 0.7, causal)
        assert np.array_equal(O, O2) and np.array_equal(L, L2)


# ---------------------------------------------------------------- closed forms

def pin_single_key():
    """N = 1: every weight is 1, so O = V_0 and LSE = s * q . k_0."""
    rng = _rng(13)
    q = rng.standard_normal((9, 6))
    k = rng.standard_normal((1, 6))
    v = rng.standard_normal((1, 6))
    for causal in (False, True):
        O, L = attention(q, k, v, 0.3, causal)
        vis_rows = np.arange(9) + (1 - 9) >= 0 if causal else np.ones(9, bool)
        assert np.abs(O[vis_rows] - v[0]).max() <= 1e-15
        assert np.abs(L[vis_rows] - _f32(0.3) * (q @ k[0])[vis_rows]).max() <= 1e-13
        assert np.all(O[~vis_rows] == 0.0) and np.all(np.isneginf(L[~vis_rows]))


def pin_zero_keys_uniform():
    """K = 0: all scores are 0, O is the mean of the visible V rows and LSE = ln(#visible)."""
    rng = _rng(14)
    M, N = 11, 17
    q = rng.standard_normal((M, 4))
    k = np.zeros((N, 4))
    v = rng.standard_normal((N, 4))
    for causal in (False, True):
        O, L = attention(q, k, v, 1.0, causal)
        for i in range(M):
            n = N if not causal else i + N - M + 1
            assert abs(L[i] - math.log(n)) <= 1e-14
            assert np.abs(O[i] - v[:n].mean(axis=0)).max() <= 1e-14


def pin_two_key_ratio_large_logits():
    """Two keys whose scores differ by ln 3 give weights 3/4 and 1/4, even when
    the scores are ~1000 (the stable form subtracts the max first)."""
    q = np.array([[1.0]])
    k = np.array([[1000.0], [1000.0 - math.log(3.0)]])
    v = np.array([[4.0], [8.0]])
    O, L = attention(q, k, v, 1.0)
    assert abs(O[0, 0] - (0.75 * 4 + 0.25 * 8)) <= 1e-12
    assert abs(L[0] - (1000.0 + math.log(4.0 / 3.0))) <= 1e-10


def pin_empty_rows():
    """Causal with M > N: rows i < M - N see no key -> O = 0 exactly, LSE = -inf."""
    rng = _rng(15)
    M, N = 10, 4
    q = rng.standard_normal((M, 3))
    k = rng.standard_normal((N, 3))
    v = rng.standard_normal((N, 3))
    O, L = attention(q, k, v, 1.0, True)
    assert np.all(O[: M - N] == 0.0) and np.all(np.isneginf(L[: M - N]))
    assert np.all(np.isfinite(L[M - N:]))
    # the first non-empty row sees exactly key 0
    assert np.abs(O[M - N] - v[0]).max() <= 1e-15
    # no keys at all: every row is empty, causal or not
    for causal in (False, True):
        O0, L0 = attention(q, np.zeros((0, 3)), np.zeros((0, 3)), 1.0, causal)
        assert np.all(O0 == 0.0) and np.all(np.isneginf(L0))


def pin_shift_feature():
    """Appending a feature Q' = [Q | 1], K' = [K | c] adds s*c to every score:
    O is unchanged, LSE grows by s*c (softmax shift invariance)."""
    rng = _rng(16)
    q = rng.standard_normal((12, 5))
    k = rng.standard_normal((19, 5))
    v = rng.standard_normal((19, 5))
    s, c = 0.4, 4.0
    O, L = attention(q, k, v, s, True)
    O2, L2 = attention(np.hstack([q, np.ones((12, 1))]), np.hstack([k, np.full((19, 1), c)]), v, s, True)
    assert np.abs(O - O2).max() <= 1e-13
    assert np.abs(L2 - L - _f32(s) * c).max() <= 1e-12


def pin_permutation_and_future():
    """Permuting K/V rows jointly (non-causal) changes nothing; changing keys that
    a causal row cannot see leaves that row unchanged; outputs lie in the convex
    hull of the value rows."""
    rng = _rng(17)
    q = rng.standard_normal((15, 6))
    k = rng.standard_normal((23, 6))
    v = rng.standard_normal((23, 6))
    O, L = attention(q, k, v, 0.6, False)
    perm = rng.permutation(23)
    Op, Lp = attention(q, k[perm], v[perm], 0.6, False)
    assert np.abs(O - Op).max() <= 1e-13 and np.abs(L - Lp).max() <= 1e-13
    Oc, Lc = attention(q, k, v, 0.6, True)
    k2, v2 = k.copy(), v.copy()
    k2[-3:] += 5.0
    v2[-3:] -= 7.0
    Oc2, Lc2 = attention(q, k2, v2, 0.6, True)
    off = 23 - 15
    rows_blind = [i for i in range(15) if i + off < 23 - 3]
    assert np.array_equal(Oc[rows_blind], Oc2[rows_blind])
    assert np.array_equal(Lc[rows_blind], Lc2[rows_blind])
    assert not np.allclose(Oc[-1], Oc2[-1])
    assert np.all(O >= v.min(axis=0) - 1e-12) and np.all(O <= v.max(axis=0) + 1e-12)


def pin_sampled_rows_match_full():
    """attention_rows on a row subset equals the same rows of the full result."""
    rng = _rng(18)
    q = rng.standard_normal((3, 40, 8))
    k = rng.standard_normal((3, 50, 8))
    v = rng.standard_normal((3, 50, 8))
    O, L = attention(q, k, v, 0.35, True)
    rows = np.array([[0, 5, 39], [1, 2, 3], [38, 20, 11]])
    Or, Lr = attention_rows(q, k, v, 0.35, True, rows)
    for h in range(3):
        assert np.array_equal(Or[h], O[h, rows[h]]) and np.array_equal(Lr[h], L[h, rows[h]])


def pin_dtype_widening():
    """bf16 / fp16 inputs are widened exactly (values already representable)."""
    import torch

    rng = _rng(19)
    qf = rng.standard_normal((2, 9, 8)).astype(np.float32)
    kf = rng.standard_normal((2, 13, 8)).astype(np.float32)
    vf = rng.standard_normal((2, 13, 8)).astype(np.float32)
    for tdt in (torch.bfloat16, torch.float16):
        qt, kt, vt = (torch.from_numpy(a).to(tdt) for a in (qf, kf, vf))
        O, L = attention(qt, kt, vt, 0.25)
        O2, L2 = attention(qt.double().numpy(), kt.double().numpy(), vt.double().numpy(), 0.25)
        assert np.array_equal(O, O2) and np.array_equal(L, L2)


# ---------------------------------------------------------------- recurrence

def pin_every_split_equals_one_shot():
    """Every composition of a row of length n <= 12 into chunks gives the same
    normalised weights as the one-shot softmax ('softmax of a concatenation can
    be computed from the maxima and sums of its pieces', Module 08)."""
    rng = _rng(20)
    for n in range(1, 13):
        x = rng.standard_normal(n) * 4
        P, _, _ = masked_softmax(x[None, :], np.ones((1, n), dtype=bool))
        for cuts in itertools.product([0, 1], repeat=n - 1):
            sizes, run = [], 1
            for c in cuts:
                if c:
                    sizes.append(run)
                    run = 1
                else:
                    run += 1
            sizes.append(run)
            m, l, _ = online_softmax_trace(x, sizes)
            assert np.abs(np.exp(x - m) / l - P[0]).max() <= 1e-14 * max(1.0, P.max())


def pin_tiled_equals_definition():
    """The tiled recurrence equals the definition for every uniform block size,
    ragged tails, causal (M < N, M = N, M > N) and not, in both bases."""
    rng = _rng(21)
    for M, N, causal in [(37, 53, False), (53, 53, True), (29, 61, True), (61, 29, True)]:
        q = rng.standard_normal((M, 7)) * 3
        k = rng.standard_normal((N, 7))
        v = rng.standard_normal((N, 5))
        O, L = attention(q, k, v, 0.5, causal)
        for bn in list(range(1, 18)) + [N - 1, N, N + 5]:
            for bm, base2 in [(1, True), (16, True), (bn, False), (M, True)]:
                Ot, Lt, _, _ = tiled_attention(q, k, v, 0.5, causal, bm, bn, base2=base2)
                assert np.array_equal(np.isneginf(L), np.isneginf(Lt))
                fin = np.isfinite(L)
                assert np.abs(Ot - O).max() <= 1e-12, (M, N, causal, bm, bn)
                assert np.abs(Lt[fin] - L[fin]).max(initial=0.0) <= 1e-12


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
