"""Pins of the window-policy oracle (CPU only).

The oracle's allocator simulation is checked against (a) a page table worked
by hand, (b) an independent closed form of the retained frame set, and (c) the
pages' claims: bounded occupancy and memory growth of about frames / k.
"""

import itertools
import os
import random

import numpy as np
import pytest

from oracle import window

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "config0_page_tables.txt")


def _read_golden():
    rows = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            t, rest = line.split(":", 1)
            rows[int(t)] = [tuple(int(x) for x in e.split(":")) for e in rest.split()]
    return rows


def test_tiny_page_tables_match_hand_worked_table():
    gold = _read_golden()
    c = window.WindowCache(scale_frames=1, window=4, keyframe_interval=1, num_pages=6)
    for t in range(12):
        c.append(t)
        c.evict()
        assert c.table == gold[t], f"frame {t}"
        assert c.attended() == [f for _, f in gold[t]]


@pytest.mark.parametrize("S,W,k", [(1, 4, 1), (8, 64, 1), (8, 64, 4), (0, 3, 2), (2, 0, 3), (4, 5, 2), (3, 1, 5)])
def test_allocator_sim_matches_closed_form(S, W, k):
    frames = 300
    pages = S + (W if W else frames) + 1
    c = window.WindowCache(S, W, k, pages)
    for t in range(frames):
        c.append(t)
        c.evict()
        assert c.persisted() == window.persisted_frames(t, S, W, k)
        att = c.attended()
        assert att == window.attended_frames(t, S, W, k)
        # occupancy bound: scale frames + window (GCTStream explainer, "Sliding Window Eviction")
        if W:
            assert len(c.persisted()) <= S + W
        # page ids unique and disjoint from the free list
        ids = c.page_ids()
        assert len(set(ids)) == len(ids)
        assert set(ids).isdisjoint(c.free)
        assert set(ids) | c.free == set(range(pages))


def test_random_policies_closed_form():
    rng = random.Random(1234)
    for _ in range(40):
        S, W, k = rng.randint(0, 6), rng.randint(0, 9), rng.randint(1, 6)
        frames = rng.randint(1, 120)
        c = window.WindowCache(S, W, k, S + (W if W else frames) + 1)
        for t in range(frames):
            c.append(t)
            c.evict()
            c.attended()
            assert c.persisted() == window.persisted_frames(t, S, W, k)


def test_growth_is_frames_over_k_before_the_window_fills():
    # GCTStream explainer, "Frame-by-Frame Causal Processing": memory grows by
    # about num_frames / keyframe_interval.
    S, k = 8, 4
    for t in range(S, 200):
        n = len(window.persisted_frames(t, S, 0, k))
        assert n == S + (t - S) // k + 1
        assert abs(n - (t + 1) / k) <= S


def test_long_stream_checkpoints():
    # keyframe_interval 4, scale 8, window 64: t = 99 -> 31 frames, t >= 260 -> 72 frames.
    S, W, k = 8, 64, 4
    p99 = window.persisted_frames(99, S, W, k)
    assert p99 == list(range(8)) + list(range(8, 100, 4))
    assert len(p99) == 31
    for t in (260, 999, 9999):
        p = window.persisted_frames(t, S, W, k)
        assert len(p) == 72
    assert window.persisted_frames(999, S, W, k)[8:] == list(range(744, 1000, 4))
    assert window.persisted_frames(9999, S, W, k)[8:] == list(range(9744, 10000, 4))
    assert len(window.persisted_frames(259, S, W, k)) == 71


def test_reset_replay_is_identical():
    def run():
        c = window.WindowCache(8, 64, 4, 73)
        out = []
        for t in range(500):
            c.append(t)
            c.evict()
            c.attended()
            out.append(tuple(c.table))
        return out
    assert run() == run()


def test_pool_exhaustion_raises():
    c = window.WindowCache(1, 4, 1, 5)  # needs S + W + 1 = 6
    with pytest.raises(window.PoolExhausted):
        for t in range(10):
            c.append(t)
            c.evict()


def test_keyframe_rule():
    assert [window.is_keyframe(t, 0, 4) for t in range(9)] == [True, False, False, False, True,
                                                               False, False, False, True]
    assert all(window.is_keyframe(t, 8, 4) for t in range(8))
    for S, k in itertools.product(range(0, 9, 4), (1, 2, 4)):
        for t in range(S, 50):
            assert window.is_keyframe(t, S, k) == ((t - S) % k == 0)


def _special_fixture():
    rows = {}
    for ln in open(os.path.join(os.path.dirname(__file__), "golden", "special_tokens_hand_example.txt")):
        if ln.strip() and not ln.startswith("#"):
            t, rest = ln.split(":", 1)
            tab, ids, free = rest.split("|")
            rows[int(t[1:])] = ([tuple(int(x) for x in e.split(":")) for e in tab.split()],
                                [int(x) for x in ids.split()], {int(x) for x in free.split()})
    return rows


def test_special_tokens_hand_example():
    gold = _special_fixture()
    c = window.SpecialWindowCache(1, 2, 1, 6, special=1, tokens_per_frame=4)
    for t in range(8):
        c.append(t)
        c.evict()
        tab, ids, free = gold[t]
        assert c.page_table() == tab, t
        assert [i for _, toks in c.special_pages for i in toks] == ids, t
        assert c.free == free, t


def test_special_tokens_closed_form_and_fill():
    # the held special ids equal the first slots of every evicted keyframe
    # (an independent closed form); every special page but the last is filled
    # to floor(T / special) frames; the attended set is scale + specials +
    # window + transient; special = 0 is the plain window policy
    rng = np.random.default_rng(12)
    for trial in range(60):
        S, W, k = int(rng.integers(0, 4)), int(rng.integers(1, 6)), int(rng.integers(1, 4))
        T = int(rng.integers(2, 12))
        sp = int(rng.integers(1, T + 1))
        frames = int(rng.integers(5, 80))
        c = window.SpecialWindowCache(S, W, k, S + W + 1 + frames, special=sp, tokens_per_frame=T)
        plain = window.WindowCache(S, W, k, S + W + 1 + frames)
        for t in range(frames):
            c.append(t)
            c.evict()
            plain.append(t)
            plain.evict()
            assert c.persisted() == plain.persisted() == window.persisted_frames(t, S, W, k)
            held = [i for _, toks in c.special_pages for i in toks]
            assert held == window.special_token_ids(t, S, W, k, sp, T)
            per_page = (T // sp) * sp
            lens = [len(toks) for _, toks in c.special_pages]
            assert all(n == per_page for n in lens[:-1]) and (not lens or 0 < lens[-1] <= per_page)
            att = c.attended_tokens()
            fr = window.attended_frames(t, S, W, k) if t >= S else window.persisted_frames(t, S, W, k)
            want = [f * T + j for f in fr if f < S for j in range(T)] + held + \
                [f * T + j for f in fr if f >= S for j in range(T)]
            assert att == want
            pids = [p for p, _, _ in c.page_table()]
            assert len(set(pids)) == len(pids) and not (set(pids) & c.free)
    c = window.SpecialWindowCache(1, 4, 1, 6, special=0, tokens_per_frame=16)
    p = window.WindowCache(1, 4, 1, 6)
    for t in range(12):
        c.append(t), c.evict(), p.append(t), p.evict()
        assert [(a, b) for a, b, _ in c.page_table()] == list(zip(p.page_ids(), p.persisted()))
