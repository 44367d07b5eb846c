"""Pins of the token-budget policy oracle (CPU only).

The paged simulation is checked against a second formulation that keeps one
flat list of token ids (no pages, no compaction), and against the size bound.
"""

import os

import numpy as np

from oracle import budget, clces


def _scores(n_tokens, n_layers, seed):
    rng = np.random.default_rng(seed)
    u = rng.lognormal(0, 0.5, n_tokens)
    return np.sqrt(u[:, None] * rng.chisquare(64, (n_tokens, n_layers))).astype(np.float32)


def test_paged_policy_matches_flat_list():
    # the paged cache keeps the same token set as a flat list that applies the
    # top-k directly; the scores are continuous, so s_hat has no ties and the
    # set does not depend on the order of tokens inside a page
    T, B, frames, L, W = 8, 20, 12, 6, 5
    table = _scores(T * frames, L, seed=1)
    for layer in range(L):
        c = budget.BudgetCache(layer, T, B, num_pages=frames, window=W, lam=0.5)
        flat = np.zeros(0, np.int64)
        for t in range(frames):
            c.append(t)
            flat = np.concatenate([flat, t * T + np.arange(T)])
            ran = c.score_and_compact(table)
            if len(flat) > B:
                assert ran
                lw = clces.window_layers(layer, W)
                res = clces.clces(np.stack([table[flat, l] for l in lw]), 0.5)
                assert len(np.unique(res["s_hat"])) == len(flat)
                flat = flat[clces.topk_keep(res["s_hat"], B)]
                np.testing.assert_array_equal(np.sort(c.last["keep_ids"]), np.sort(flat))
            else:
                assert not ran
            np.testing.assert_array_equal(np.sort(c.all_ids()), np.sort(flat))
            assert len(c.all_ids()) <= max(B, T)
            # bookkeeping: unique ids, no empty page, free + used = pool
            pids = [p for p, _, _ in c.page_table()]
            assert len(set(pids)) == len(pids)
            assert all(n > 0 for _, _, n in c.page_table())
            assert set(pids) | c.free == set(range(frames))
            # page order follows frame order; a page holds only its frame's tokens
            fr = [f for _, f, _ in c.page_table()]
            assert fr == sorted(fr)
            for _, f, ids in c.table:
                assert len(set(ids.tolist())) == len(ids) and (ids // T == f).all()


def test_scale_frames_are_never_scored():
    T, B, frames = 4, 6, 9
    table = _scores(T * frames, 1, seed=2)
    c = budget.BudgetCache(0, T, B, num_pages=frames, window=5, lam=0.5, scale_frames=2)
    for t in range(frames):
        c.append(t)
        c.score_and_compact(table)
        ids = c.all_ids()
        if t >= 1:
            assert list(ids[:2 * T]) == list(range(2 * T))
        assert len(c.candidate_ids()) <= max(B, T)


def test_budget_step_keeps_exactly_budget():
    T, B = 10, 25
    table = _scores(T * 5, 3, seed=3)
    c = budget.BudgetCache(2, T, B, num_pages=5)
    for t in range(5):
        c.append(t)
        c.score_and_compact(table)
        assert len(c.all_ids()) == min((t + 1) * T, B) if (t + 1) * T > B else (t + 1) * T


def _merge_case():
    path = os.path.join(os.path.dirname(__file__), "golden", "merge_hand_example.txt")
    d = {}
    for ln in open(path):
        if ln.strip() and not ln.startswith("#"):
            k, v = ln.split(":", 1)
            d[k.strip()] = [int(x) for x in v.split()]
    return d


def _cache_with_lengths(T, lens, scale_frames=0):
    c = budget.BudgetCache(0, T, 10 ** 9, num_pages=len(lens), scale_frames=scale_frames)
    for t, n in enumerate(lens):
        c.append(t)
        c.table[-1][2] = c.table[-1][2][:n]
    return c


def test_merge_hand_example():
    d = _merge_case()
    c = _cache_with_lengths(d["T"][0], d["lengths"])
    moves = c.merge_pages()
    assert [n for _, _, n in c.page_table()] == d["after"]
    assert sorted(src for src, _, _, _ in moves) == d["released"]
    assert c.free == set(d["released"])


def test_merge_properties():
    # the token sequence is unchanged; greedy leaves every adjacent pair past
    # one page, so fewer than 2N/T + 1 pages remain; scale pages never merge
    rng = np.random.default_rng(8)
    for trial in range(300):
        T = int(rng.integers(4, 200))
        S = int(rng.integers(0, 3))
        lens = [T] * S + [int(x) for x in rng.integers(1, T + 1, size=int(rng.integers(1, 40)))]
        c = _cache_with_lengths(T, lens, scale_frames=S)
        before = c.all_ids().copy()
        pages_before = {p for p, _, _ in c.page_table()}
        moves = c.merge_pages()
        np.testing.assert_array_equal(c.all_ids(), before)
        tab = c.page_table()
        assert [n for _, f, n in tab[:S]] == [T] * S and all(f < S for _, f, _ in tab[:S])
        rest = [n for _, _, n in tab[S:]]
        assert all(n <= T for n in rest)
        assert all(a + b > T for a, b in zip(rest, rest[1:]))
        N = sum(rest)
        assert len(rest) < 2 * N / T + 1
        assert {p for p, _, _ in tab} | {m[0] for m in moves} == pages_before
        assert len(moves) == len(pages_before) - len(tab)
        # every move appends a whole page right after the destination's rows
        for src, dst, slot, n in moves:
            assert 0 < n and slot + n <= T
