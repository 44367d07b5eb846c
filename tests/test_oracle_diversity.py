"""Pins of the diversity oracle (InfiniteVGGT explainer: cosine diversity, per-head top-K, tempered budgets)."""

import math
import os

import numpy as np

from oracle import diversity

HERE = os.path.dirname(__file__)


def test_identical_directions_score_minus_one():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(64)
    keys = rng.uniform(0.1, 5.0, size=(40, 1)) * v[None, :]
    np.testing.assert_allclose(diversity.diversity_scores(keys), -1.0, atol=1e-14)


def test_orthonormal_set_scores_minus_inverse_sqrt_n():
    for n in (1, 2, 7, 64):
        keys = np.eye(64)[:n] * np.arange(1, n + 1)[:, None]  # scaled basis vectors
        np.testing.assert_allclose(diversity.diversity_scores(keys), -1.0 / math.sqrt(n), atol=1e-14)


def test_scale_invariance_and_mean_identity():
    rng = np.random.default_rng(2)
    keys = rng.standard_normal((50, 64))
    s = diversity.diversity_scores(keys)
    scaled = keys * rng.uniform(0.01, 100.0, size=(50, 1))
    np.testing.assert_allclose(diversity.diversity_scores(scaled), s, atol=1e-13)
    # mean over keys of -(khat . m)/|m| is -|m|
    khat = keys / np.linalg.norm(keys, axis=1, keepdims=True)
    m = khat.mean(axis=0)
    np.testing.assert_allclose(s.mean(), -np.linalg.norm(m), atol=1e-14)
    assert np.all(s >= -1 - 1e-12) and np.all(s <= 1 + 1e-12)


def test_brute_force_cosine_small():
    rng = np.random.default_rng(3)
    for trial in range(20):
        n, d = int(rng.integers(1, 9)), int(rng.integers(1, 6))
        keys = rng.standard_normal((n, d))
        if trial % 5 == 0:
            keys[0] = 0.0  # a zero key normalises to zero and scores 0
        unit = []
        for row in keys:
            r = math.sqrt(math.fsum(x * x for x in row))
            unit.append([x / r for x in row] if r > 0 else [0.0] * d)
        mean = [math.fsum(u[j] for u in unit) / n for j in range(d)]
        mnorm = math.sqrt(math.fsum(x * x for x in mean))
        expect = []
        for u, row in zip(unit, keys):
            un = math.sqrt(math.fsum(x * x for x in u))
            expect.append(0.0 if un == 0 or mnorm == 0 else -math.fsum(a * b for a, b in zip(u, mean)) / (un * mnorm))
        np.testing.assert_allclose(diversity.diversity_scores(keys), expect, atol=1e-13)


def test_zero_mean_gives_zero_scores():
    keys = np.array([[1.0, 0.0], [-2.0, 0.0], [0.0, 0.0]])
    np.testing.assert_array_equal(diversity.diversity_scores(keys), [0.0, 0.0, 0.0])


def _example():
    d = {}
    for ln in open(os.path.join(HERE, "golden", "diversity_budget_example.txt")):
        if ln.strip() and not ln.startswith("#"):
            k, v = ln.split(":", 1)
            d[k.strip()] = int(v)
    return d


def test_worked_budget_example():
    d = _example()
    rng = np.random.default_rng(4)
    scores = rng.standard_normal(d["candidates"])
    keep = diversity.topk_desc(scores, d["per_head_budget"])
    assert keep.sum() == d["kept"] and (~keep).sum() == d["dropped"]
    assert scores[keep].min() >= scores[~keep].max()
    assert d["per_head_budget"] * d["heads"] == d["per_layer"]
    assert d["per_layer"] * d["layers"] == d["total"]
    # equal layer diversities split the total evenly
    k = diversity.layer_budgets(np.full(d["layers"], -0.3), 0.1, d["total"], d["heads"])
    np.testing.assert_array_equal(k, d["per_head_budget"])


def test_topk_ties_by_index():
    s = np.array([0.5, 0.7, 0.5, 0.5, 0.9])
    np.testing.assert_array_equal(diversity.topk_desc(s, 3), [True, True, False, False, True])
    np.testing.assert_array_equal(diversity.topk_desc(s, 4), [True, True, True, False, True])


def test_tempered_softmax_limits():
    md = np.array([-0.9, -0.5, -0.7, -0.2])
    cold = diversity.layer_budgets(md, 1e-4, 4096, 16)
    np.testing.assert_array_equal(cold, [0, 0, 0, 256])
    hot = diversity.layer_budgets(md, 1e6, 4096, 16)
    assert np.all(np.abs(hot - 64) <= 1)
    mid = diversity.layer_budgets(md, 0.2, 4096, 16)
    assert list(np.argsort(mid, kind="stable")) == list(np.argsort(md, kind="stable"))  # more diverse, more room
    assert mid.sum() * 16 <= 4096


def test_cache_anchor_and_per_head_topk():
    H, T, D = 3, 8, 4
    rng = np.random.default_rng(5)
    keys = {t: rng.standard_normal((H, T, D)) for t in range(6)}
    key_of = lambda f, h: keys[f][h]
    c = diversity.DiversityCache(H, T, 6)
    for t in range(6):
        c.append(t)
        before = [c.candidates(h).copy() for h in range(H)]
        sc = c.scores(key_of)
        c.prune(key_of, 10)
        for h in range(H):
            kept = c.candidates(h)
            # the anchor frame stays whole; each head keeps its own top 10
            assert list(c.all_ids(h)[:T]) == list(range(T))
            assert len(kept) == min(10, len(before[h]))
            want = before[h][diversity.topk_desc(sc[h], 10)] if len(before[h]) > 10 else before[h]
            assert sorted(kept.tolist()) == sorted(want.tolist())
    tab = c.page_table()
    assert tab[0][1] == 0 and tab[0][2] == (T, T, T)
    assert all(sum(l) > 0 for _, _, l in tab)


def test_prune_decides_on_float64_scores():
    # two candidates whose float64 scores differ by 2^-30 (less than half an
    # fp32 ulp at 0.25): the larger float64 score wins, not the lower index;
    # an exact tie goes to the lower index
    s64 = np.array([0.25, 0.25 + 2.0 ** -30, 0.1])
    assert diversity.topk_desc(s64, 1).tolist() == [False, True, False]
    assert diversity.topk_desc(np.array([0.3, 0.3, 0.1]), 1).tolist() == [True, False, False]
    # through the cache: the prune keeps the top 2 of the float64 scores
    c = diversity.DiversityCache(1, 3, 2)
    c.append(0)
    c.append(1)
    rng = np.random.default_rng(5)
    keys = {0: rng.normal(size=(3, 64)), 1: rng.normal(size=(3, 64))}
    sc = c.scores(lambda f, h: keys[f])[0]
    order = sorted(range(3), key=lambda i: (-sc[i], i))
    m = c.prune(lambda f, h: keys[f], 2)[0]
    assert m.tolist() == [i in order[:2] for i in range(3)]


def _set_table(c, entries):
    c.table = [[pid, f, [np.asarray(x, dtype=np.int64) for x in ids]] for pid, f, ids in entries]
    c.free -= {pid for pid, _, _ in entries}


def test_merge_pages_hand_example():
    # T = 4, two heads.  Page 2 fits after page 1 in both heads (2+1 <= 4, 1+3 <= 4); page 3 does not fit
    # after the merged page in head 0 (3+2 > 4) and starts a new page; page 4 fits after page 3 (2+1, 0+3).
    # The anchor (frame 0) takes no part.
    c = diversity.DiversityCache(2, 4, 6)
    _set_table(c, [(0, 0, ([0, 1, 2, 3], [0, 1, 2, 3])),
                   (1, 1, ([4, 5], [6])),
                   (2, 2, ([9], [8, 10, 11])),
                   (3, 3, ([12, 13], [])),
                   (4, 4, ([17], [16, 18, 19]))])
    before = [c.all_ids(h).tolist() for h in range(2)]
    moves = c.merge_pages()
    assert moves == [(2, 1, (2, 1), (1, 3)), (4, 3, (2, 0), (1, 3))]
    assert c.page_table() == [(0, 0, (4, 4)), (1, 1, (3, 4)), (3, 3, (3, 3))]
    assert [c.all_ids(h).tolist() for h in range(2)] == before
    assert c.table[1][2][0].tolist() == [4, 5, 9] and c.table[2][2][1].tolist() == [16, 18, 19]
    assert c.free == {2, 4, 5}
    assert c.merge_pages() == []  # nothing left to merge


def test_merge_pages_invariants_after_prunes():
    rng = np.random.default_rng(11)
    T, H, F = 20, 3, 12
    keys = {f: rng.standard_normal((H, T, 64)) for f in range(F)}
    c = diversity.DiversityCache(H, T, F + 1)
    total_moves = 0
    for t in range(F):
        c.append(t)
        c.prune(lambda f, h: keys[f][h], 45)
        ids_before = [c.all_ids(h).tolist() for h in range(H)]
        pages_before, free_before = len(c.table), set(c.free)
        moves = c.merge_pages()
        total_moves += len(moves)
        assert [c.all_ids(h).tolist() for h in range(H)] == ids_before
        assert len(c.table) == pages_before - len(moves)
        assert c.free == free_before | {m[0] for m in moves}
        cand = [e for e in c.table if e[1] > 0]
        assert all(len(x) <= T for _, _, ids in cand for x in ids)
        for a, b in zip(cand, cand[1:]):  # the greedy pass leaves no adjacent pair that fits
            assert any(len(a[2][h]) + len(b[2][h]) > T for h in range(H))
        for src, dst, off, cnt in moves:
            assert src not in [e[0] for e in c.table] and len(off) == len(cnt) == H
    assert total_moves > 0
