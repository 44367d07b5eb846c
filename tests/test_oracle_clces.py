"""Pins of the CLCES / top-k / compaction oracle (CPU only)."""

import os
from fractions import Fraction
import math

import numpy as np
import pytest

from oracle import clces

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "clces_hand_example.txt")


def _golden():
    d = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, rest = line.split(":", 1)
                d[key] = [float(x) for x in rest.split()]
    return d


def _brute_ranks(s):
    n = len(s)
    return np.array([sum(1 for j in range(n) if s[j] < s[i] or (s[j] == s[i] and j < i))
                     for i in range(n)])


def test_ranks_match_brute_force_count_with_ties():
    rng = np.random.default_rng(0)
    for n in (1, 2, 7, 300):
        s = rng.integers(0, 5, size=n).astype(np.float32)  # many ties
        np.testing.assert_array_equal(clces.stable_ranks(s), _brute_ranks(s))
        s = rng.random(n).astype(np.float32)
        np.testing.assert_array_equal(clces.stable_ranks(s), _brute_ranks(s))
    s = np.array([0.0, -0.0, 0.0, 1.0], dtype=np.float32)  # signed zeros compare equal
    np.testing.assert_array_equal(clces.stable_ranks(s), [0, 1, 2, 3])


def test_hand_example():
    g = _golden()
    s = np.array([g["s0"], g["s1"]], dtype=np.float32)
    res = clces.clces(s, 0.5)
    np.testing.assert_array_equal(res["ranks"][0], g["ranks0"])
    np.testing.assert_array_equal(res["ranks"][1], g["ranks1"])
    np.testing.assert_array_equal(res["sigma"], g["sigma"])
    np.testing.assert_array_equal(res["cons"], g["cons"])
    np.testing.assert_array_equal(res["s_hat"], g["s_hat"])
    assert list(np.flatnonzero(clces.topk_keep(res["s_hat"], 1))) == [int(x) for x in g["keep1"]]
    assert list(np.flatnonzero(clces.topk_keep(res["s_hat"], 2))) == [int(x) for x in g["keep2"]]


def test_identical_trajectories_give_cons_one():
    # StreamCacheVGGT 2.1.2: Cons = 1 when the rank is perfectly stable (variance 0).
    rng = np.random.default_rng(1)
    s = rng.random(500).astype(np.float32)
    win = np.stack([s * (l + 1) for l in range(5)])  # same order at every layer
    res = clces.clces(win, 0.5)
    # exact in the rationals; in float64 the mean of five equal values may be off by an ulp
    np.testing.assert_allclose(res["cons"], 1.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(res["s_hat"], 1.5 * win[-1].astype(np.float64), rtol=1e-14)


def test_lambda_zero_is_raw_score():
    # StreamCacheVGGT 2.1.3: lambda = 0 gives back the single-layer score.
    rng = np.random.default_rng(2)
    win = rng.random((5, 400)).astype(np.float32)
    res = clces.clces(win, 0.0)
    np.testing.assert_array_equal(res["s_hat"], win[-1].astype(np.float64))
    keep = clces.topk_keep(res["s_hat"], 123)
    order = sorted(range(400), key=lambda i: (-float(win[-1][i]), i))[:123]
    assert sorted(order) == list(np.flatnonzero(keep))


def test_alternating_extremes_give_cons_zero():
    # ranks alternate 0, N-1, 0, N-1: sigma = 0.5 > 1/sqrt(12) -> Cons = 0
    N = 10
    R = [np.full(N, 0), np.full(N, N - 1), np.full(N, 0), np.full(N, N - 1)]
    mu, sigma, cons = clces.consistency(R, N)
    np.testing.assert_array_equal(mu, 0.5)
    np.testing.assert_array_equal(sigma, 0.5)
    np.testing.assert_array_equal(cons, 0.0)


def test_statistics_match_exact_rational_arithmetic():
    # mean / population variance checked with exact fractions
    rng = np.random.default_rng(3)
    N, n = 37, 5
    R = [rng.permutation(N) for _ in range(n)]
    mu, sigma, cons = clces.consistency(R, N)
    for i in range(N):
        r = [Fraction(int(x[i]), N - 1) for x in R]
        m = sum(r) / n
        var = sum((x - m) ** 2 for x in r) / n
        assert abs(mu[i] - float(m)) <= 1e-15
        assert abs(sigma[i] - math.sqrt(float(var))) <= 1e-15
        c = max(0.0, 1.0 - math.sqrt(float(var)) * math.sqrt(12.0))
        assert abs(cons[i] - c) <= 1e-14


def test_cons_range_and_iid_sanity():
    rng = np.random.default_rng(4)
    win = rng.random((5, 5000)).astype(np.float32)
    res = clces.clces(win, 0.5)
    assert (res["cons"] >= 0).all() and (res["cons"] <= 1).all()
    # iid scores at every layer: ranks are near-uniform, so consistency is low on average
    assert res["cons"].mean() < 0.35
    # s_hat lies between s and (1 + lambda) s
    s = win[-1].astype(np.float64)
    assert (res["s_hat"] >= s).all() and (res["s_hat"] <= 1.5 * s).all()


def test_single_layer_window():
    # layer 0 has a window of one layer: sigma = 0, Cons = 1, s_hat = 1.5 s
    assert clces.window_layers(0, 5) == [0]
    assert clces.window_layers(2, 5) == [0, 1, 2]
    assert clces.window_layers(7, 5) == [3, 4, 5, 6, 7]
    s = np.array([[3.0, 1.0, 2.0]], dtype=np.float32)
    res = clces.clces(s, 0.5)
    np.testing.assert_array_equal(res["cons"], 1.0)
    np.testing.assert_array_equal(res["s_hat"], [4.5, 1.5, 3.0])


def test_one_token():
    res = clces.clces(np.array([[2.0], [5.0]], dtype=np.float32), 0.5)
    np.testing.assert_array_equal(res["ranks"], [[0], [0]])
    np.testing.assert_array_equal(res["cons"], [1.0])


def test_topk_matches_full_sort_with_ties():
    rng = np.random.default_rng(5)
    for n, k in ((50, 0), (50, 50), (200, 77), (1000, 500)):
        s_hat = rng.integers(0, 7, size=n).astype(np.float64) * 0.25  # deliberate ties
        keep = clces.topk_keep(s_hat, k)
        order = sorted(range(n), key=lambda i: (-s_hat[i], i))[:k]
        assert sorted(order) == list(np.flatnonzero(keep))
        assert keep.sum() == k


def test_bad_scores_rejected():
    with pytest.raises(clces.BadScore):
        clces.clces(np.array([[1.0, np.nan]], dtype=np.float32), 0.5)
    with pytest.raises(clces.BadScore):
        clces.clces(np.array([[1.0, -1e-30]], dtype=np.float32), 0.5)


def _hand_cases():
    path = os.path.join(os.path.dirname(__file__), "golden", "compaction_hand_example.txt")
    lines = [ln.rstrip("\n") for ln in open(path) if ln.strip() and not ln.startswith("#")]
    cases = []
    for i in range(0, len(lines), 3):
        keep = [int(x) for x in lines[i].split(":", 1)[1].split()]
        out = [int(x) for x in lines[i + 1].split(":", 1)[1].split()]
        moves = [tuple(int(y) for y in m.split("->")) for m in lines[i + 2].split(":", 1)[1].split()]
        cases.append((keep, out, moves))
    return cases


def test_compaction_hand_examples():
    cases = _hand_cases()
    assert len(cases) == 5
    for keep, out, moves in cases:
        slots = np.arange(len(keep))
        np.testing.assert_array_equal(clces.compact_page(slots, np.array(keep, bool)), out)
        assert clces.compaction_moves(np.array(keep, bool)) == moves


def test_compaction_properties():
    # whatever the placement, compaction to a prefix must move every kept row
    # that lies at or past n; this rule moves exactly those, keeps every other
    # kept row where it is, and loses or duplicates nothing
    rng = np.random.default_rng(6)
    for trial in range(200):
        L = int(rng.integers(1, 130))
        rows = rng.standard_normal((L, 3)).astype(np.float32)
        keep = rng.random(L) < rng.random()
        n = int(keep.sum())
        out = clces.compact_page(rows, keep)
        assert out.shape == (n, 3)
        kept_rows = rows[keep]
        np.testing.assert_array_equal(np.sort(out, axis=0), np.sort(kept_rows, axis=0))
        for j in range(n):
            if keep[j]:
                np.testing.assert_array_equal(out[j], rows[j])
        moves = clces.compaction_moves(keep)
        assert sorted(src for src, _ in moves) == [j for j in range(n, L) if keep[j]]
        assert sorted(dst for _, dst in moves) == [j for j in range(n) if not keep[j]]
        for src, dst in moves:
            np.testing.assert_array_equal(out[dst], rows[src])
    assert clces.compact_page(np.zeros((64, 2)), np.zeros(64, bool)).shape[0] == 0
