"""Pins of the attention oracle (CPU only).

Brute force: dense float64 attention of every frame's queries over the whole
stream with a frame-level mask built from the closed-form retained set,
computed row by row with scipy's logsumexp -- no paging, no gather.  Plus
closed forms and a two-token example worked by hand.
"""

import math

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import attention, window


def _rng(seed):
    return np.random.default_rng(seed)


def _brute_force_stream(S, W, k, T, H, D, frames, tau, seed):
    rng = _rng(seed)
    q = rng.standard_normal((frames, T, H, D))
    kk = rng.standard_normal((frames, T, H, D))
    v = rng.standard_normal((frames, T, H, D))
    results = {}
    for t in range(S, frames):
        vis = set(window.attended_frames(t, S, W, k))
        mask = np.array([f in vis for f in range(frames) for _ in range(T)])
        K = kk.reshape(frames * T, H, D)
        V = v.reshape(frames * T, H, D)
        out = np.zeros((T, H, D))
        lse = np.zeros((T, H))
        for i in range(T):
            for h in range(H):
                z = np.where(mask, tau * (K[:, h, :] @ q[t, i, h, :]), -np.inf)
                lz = logsumexp(z)
                w = np.exp(z - lz)
                out[i, h] = w @ V[:, h, :]
                lse[i, h] = lz
        results[t] = (out, lse)
    return q, kk, v, results


@pytest.mark.parametrize("W", [4, 0])
def test_matches_masked_dense_brute_force(W):
    S, k, T, H, D, frames, tau = 1, 1, 16, 2, 64, 12, 0.125
    q, kk, v, ref = _brute_force_stream(S, W, k, T, H, D, frames, tau, seed=7)
    c = window.WindowCache(S, W, k, 13)
    for t in range(frames):
        c.append(t)
        c.evict()
        att = c.attended()
        if t < S:
            continue
        K = np.concatenate([kk[f] for f in att])
        V = np.concatenate([v[f] for f in att])
        out, lse = attention.attend(q[t], K, V, tau)
        np.testing.assert_allclose(out, ref[t][0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, ref[t][1], rtol=0, atol=1e-12)


def test_keyframe_interval_transient_frame_brute_force():
    S, W, k, T, H, D, frames, tau = 2, 3, 3, 5, 2, 8, 20, 0.3
    q, kk, v, ref = _brute_force_stream(S, W, k, T, H, D, frames, tau, seed=11)
    for t in range(S, frames):
        att = window.attended_frames(t, S, W, k)
        out, lse = attention.attend(q[t], np.concatenate([kk[f] for f in att]),
                                    np.concatenate([v[f] for f in att]), tau)
        np.testing.assert_allclose(out, ref[t][0], rtol=0, atol=1e-12)


def test_scale_phase_block_mask():
    # "Scale-Frame Phase": the first S frames see each other (bidirectional).
    S, T, H, D, tau = 3, 4, 2, 8, 0.5
    rng = _rng(3)
    q = rng.standard_normal((S * T, H, D))
    k = rng.standard_normal((S * T, H, D))
    v = rng.standard_normal((S * T, H, D))
    out, _ = attention.attend(q, k, v, tau)
    for i in range(S * T):
        for h in range(H):
            z = tau * (k[:, h, :] @ q[i, h, :])
            w = np.exp(z - logsumexp(z))
            np.testing.assert_allclose(out[i, h], w @ v[:, h, :], atol=1e-13)


def test_hand_example_two_tokens():
    # z = (0, ln 3) -> weights (1/4, 3/4) -> out = 1/4 * 1 + 3/4 * 5 = 4; lse = ln 4
    q = np.array([[[1.0]]])
    k = np.array([[[0.0]], [[math.log(3.0)]]])
    v = np.array([[[1.0]], [[5.0]]])
    out, lse = attention.attend(q, k, v, 1.0)
    assert abs(out[0, 0, 0] - 4.0) < 1e-14
    assert abs(lse[0, 0] - math.log(4.0)) < 1e-14


def test_closed_forms():
    rng = _rng(5)
    n_q, N, H, D = 7, 33, 3, 16
    q = rng.standard_normal((n_q, H, D))
    k = rng.standard_normal((N, H, D))
    v = rng.standard_normal((N, H, D))
    # V == 1 -> O == 1 (rows of softmax sum to one)
    out, _ = attention.attend(q, k, np.ones_like(v), 0.7)
    np.testing.assert_allclose(out, 1.0, atol=1e-13)
    # Q == 0 -> uniform weights -> mean of V
    out, lse = attention.attend(np.zeros_like(q), k, v, 0.7)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(axis=0), out.shape), atol=1e-13)
    np.testing.assert_allclose(lse, math.log(N), atol=1e-13)
    # all keys equal -> mean of V
    out, _ = attention.attend(q, np.broadcast_to(k[:1], k.shape), v, 0.7)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(axis=0), out.shape), atol=1e-13)
    # a single cached token -> its value
    out, _ = attention.attend(q, k[:1], v[:1], 0.7)
    np.testing.assert_allclose(out, np.broadcast_to(v[0], out.shape), atol=1e-14)
    # invariant under permuting the cache order
    perm = rng.permutation(N)
    a, la = attention.attend(q, k, v, 0.7)
    b, lb = attention.attend(q, k[perm], v[perm], 0.7)
    np.testing.assert_allclose(a, b, atol=1e-13)
    np.testing.assert_allclose(la, lb, atol=1e-13)
    # linear in V
    v2 = rng.standard_normal((N, H, D))
    c, _ = attention.attend(q, k, 2.0 * v - 3.0 * v2, 0.7)
    d, _ = attention.attend(q, k, v2, 0.7)
    np.testing.assert_allclose(c, 2.0 * a - 3.0 * d, atol=1e-12)
    # row chunking does not change anything
    e, le = attention.attend(q, k, v, 0.7, row_chunk=2)
    np.testing.assert_allclose(e, a, rtol=0, atol=1e-14)
    np.testing.assert_allclose(le, la, rtol=0, atol=1e-14)


def test_gather_tokens():
    T, H, D = 4, 2, 3
    frames = {f: np.arange(T * H * D).reshape(T, H, D) + 100 * f for f in range(5)}
    ids = [4 * 3 + 1, 0, 4 * 4 + 3, 4 * 3 + 0]
    rows = attention.gather_tokens(lambda f: frames[f], ids, T)
    for r, i in zip(rows, ids):
        np.testing.assert_array_equal(r, frames[i // T][i % T])
