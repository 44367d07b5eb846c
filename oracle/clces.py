"""Cross-layer rank-consistency score (CLCES), fused score, top-k and compaction.

Oracle (test infrastructure only).  Source: StreamCacheVGGT article
("StreamCacheVGGT：基于跨层一致性评分与混合压缩的流式3D重建缓存管理框架"),
section 2.1 and sub-sections:

* 2.1.1 -- the raw score of token i at layer l is the L2 norm of the FFN
  residual; at every layer of a window of the W most recent layers (W = 5)
  the N tokens are ordered by raw score, giving ranks 0..N-1;
* 2.1.2 -- ranks are normalised to [0, 1]; mean and variance over the window;
  a uniformly random rank has standard deviation 1/sqrt(12), hence
  ``Cons = max(0, 1 - sigma * sqrt(12))`` in [0, 1];
* 2.1.3 -- fused score ``s_hat = s * (1 + lambda * Cons)``, lambda = 0.5;
  lambda = 0 gives back the raw score;
* 2.1.4 -- the rank history lives for one frame only.

Top-k keep and in-place compaction follow the "pure eviction" description in
section 1 of the same article (drop the lowest-scoring tokens to fit the
budget) and the InfiniteVGGT explainer ("Rolling Memory"; step "Prune and roll
the memory": keep the top-K tokens, discard the rest, the cache size stays
fixed).

Readings taken where the pages are silent:

* rank direction ascending, ties by index (a stable sort);
* ``r = R / (N - 1)`` (r = 0 when N = 1);
* window = layers ``max(0, l-W+1) .. l``, so ``n = min(W, l+1)`` entries;
* population variance (divide by n); fixed summation order: oldest window
  layer first; every step in float64 with no fused multiply-add;
* keep order: s_hat descending, then index ascending; K tokens kept;
* compaction is page-local: with n kept rows, kept rows already in slots
  [0, n) stay where they are and the kept rows in slots [n, len) fill the
  dropped slots of [0, n), both taken in ascending slot order; pages left
  empty are released.  (The pages fix no order inside a page and attention
  does not depend on it; this placement moves the fewest rows.)

Pinned by ``tests/test_oracle_clces.py``: ranks against an O(N^2) brute-force
count, the two-token-order hand example in ``tests/golden/clces_hand_example.txt``,
the closed forms Cons = 1 for identical rank trajectories and s_hat = s for
lambda = 0, Cons = 0 for alternating extreme ranks, the range [0, 1], top-k
against a brute-force full sort with deliberate ties, and compaction against
the hand example in ``tests/golden/compaction_hand_example.txt`` and the
properties that fix the placement (the result is a permutation of the kept
rows, kept rows below n are fixed points, and exactly the kept rows at or past
n move, the fewest any compaction to a prefix can move).
"""

from __future__ import annotations

import numpy as np

SQRT12 = float(np.sqrt(12.0))


class BadScore(ValueError):
    """A raw score is NaN or negative (an L2 norm cannot be)."""


def check_scores(s: np.ndarray) -> None:
    s = np.asarray(s)
    if np.isnan(s).any() or (s < 0).any():
        raise BadScore("raw scores must be non-negative and not NaN")


def window_layers(layer: int, window: int) -> list[int]:
    """Layers of the rank window ending at ``layer``, oldest first."""
    return list(range(max(0, layer - window + 1), layer + 1))


def stable_ranks(s: np.ndarray) -> np.ndarray:
    """Rank of each token in the stable ascending order of ``s`` (0..N-1)."""
    s = np.asarray(s)
    order = np.argsort(s, kind="stable")
    ranks = np.empty(len(s), dtype=np.int64)
    ranks[order] = np.arange(len(s), dtype=np.int64)
    return ranks


def consistency(ranks: list[np.ndarray], n_tokens: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Mean, standard deviation and ``Cons`` of the normalised rank trajectories.

    ``ranks`` holds one int array ``[N]`` per window layer, oldest first.
    """
    n = len(ranks)
    if n == 0:
        raise ValueError("empty window")
    if n_tokens > 1:
        r = [np.asarray(R, dtype=np.float64) / float(n_tokens - 1) for R in ranks]
    else:
        r = [np.zeros(len(R), dtype=np.float64) for R in ranks]
    acc = np.zeros(n_tokens, dtype=np.float64)
    for x in r:
        acc = acc + x
    mu = acc / float(n)
    acc2 = np.zeros(n_tokens, dtype=np.float64)
    for x in r:
        d = x - mu
        acc2 = acc2 + d * d
    var = acc2 / float(n)
    sigma = np.sqrt(var)
    cons = np.maximum(0.0, 1.0 - sigma * SQRT12)
    return mu, sigma, cons


def fused_score(s_cur: np.ndarray, cons: np.ndarray, lam: float) -> np.ndarray:
    """``s_hat = s * (1 + lambda * Cons)`` in float64 (-0.0 folded to +0.0)."""
    s = np.asarray(s_cur).astype(np.float64)
    return s * (1.0 + float(lam) * cons) + 0.0


def clces(s_window: np.ndarray, lam: float) -> dict:
    """Full CLCES for one layer.

    ``s_window [n, N]``: raw scores of the candidate tokens at the window
    layers, oldest first; the last row is the current layer.  Returns ranks
    ``[n, N]``, ``mu``, ``sigma``, ``cons`` and ``s_hat`` (all ``[N]``).
    """
    s_window = np.asarray(s_window)
    check_scores(s_window)
    n, N = s_window.shape
    ranks = [stable_ranks(s_window[i]) for i in range(n)]
    mu, sigma, cons = consistency(ranks, N)
    s_hat = fused_score(s_window[-1], cons, lam)
    return {"ranks": np.stack(ranks) if n else np.zeros((0, N), np.int64),
            "mu": mu, "sigma": sigma, "cons": cons, "s_hat": s_hat}


def topk_keep(s_hat: np.ndarray, k: int) -> np.ndarray:
    """Boolean keep mask of the first ``k`` tokens in (s_hat desc, index asc) order."""
    s_hat = np.asarray(s_hat, dtype=np.float64)
    order = np.argsort(-s_hat, kind="stable")
    keep = np.zeros(len(s_hat), dtype=bool)
    keep[order[:k]] = True
    return keep


def compact_page(rows: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """The first n = keep.sum() slots of one page after compaction.

    Slot j < n keeps its own row if that row is kept; otherwise it is a hole,
    and the holes, in ascending order, take the kept rows found at slots >= n,
    in ascending order."""
    rows = np.asarray(rows)
    keep = np.asarray(keep, dtype=bool)
    n = int(keep.sum())
    holes = [j for j in range(n) if not keep[j]]
    fillers = [j for j in range(n, len(keep)) if keep[j]]
    assert len(holes) == len(fillers)
    src = list(range(n))
    for h, f in zip(holes, fillers):
        src[h] = f
    return rows[np.array(src, dtype=np.int64)] if n else rows[:0]


def compaction_moves(keep: np.ndarray) -> list[tuple[int, int]]:
    """(source slot, destination slot) of every row that compaction moves, by destination."""
    keep = np.asarray(keep, dtype=bool)
    n = int(keep.sum())
    holes = [j for j in range(n) if not keep[j]]
    fillers = [j for j in range(n, len(keep)) if keep[j]]
    return list(zip(fillers, holes))
