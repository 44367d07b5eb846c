"""Diversity-scored rolling memory: anchor, cosine diversity, per-head top-K, layer budgets.

Oracle (test infrastructure only).  Source: InfiniteVGGT explainer ("InfiniteVGGT:
Visual Geometry Grounded Transformer for Endless Streams"):

* "Building Blocks" -- the first frame's tokens are an immutable anchor; the
  diversity score of a key is its negative cosine similarity to the mean key
  (higher = more unique); a top-K per layer and head keeps the most diverse
  tokens; layer budgets come from a softmax with a temperature over the
  layers' average diversity;
* "Cosine Similarity" -- vectors are normalised, then compared by direction;
* step-by-step recipe, steps 2-6 -- the candidates of a layer and head are its
  mutable cache plus the new frame's tokens (not the anchor); every key is
  L2-normalised and the mean of the normalised candidate keys is the
  reference; each candidate is scored against it; each layer's average
  diversity gives, through the tempered softmax, its share of the total budget
  and then a per-head top-K; each head keeps the anchor plus its top-K;
* "Concrete mini-example" -- a per-head budget of 512 with 1,200 candidates
  keeps 512 and drops 688.

Readings taken where the pages are silent:

* the anchor is frame 0's page in every layer and head;
* a zero key normalises to the zero vector; when the mean of the normalised
  keys is the zero vector every score is 0;
* score = -(k_hat . m) / |m| with m the mean of the normalised candidate keys,
  in float64 from the stored key values;
* per-head top-K: the K highest scores, ties by candidate index (table order,
  then slot order); K >= the candidate count keeps everything; the recipe's
  step 6 keeps the most diverse tokens and fixes no precision of its own, so
  the decision is taken on the float64 scores themselves;
* layer budgets: p = softmax(mean_diversity / tau) over the layers;
  K_l = floor(floor(p_l * total) / heads) tokens per head of layer l;
  a layer's average diversity is the mean of its scores over heads and
  candidates;
* compaction is per page and head, with the hole-filling rule of
  ``oracle.clces.compact_page``; a page is released once every head of it is
  empty;
* ``merge_pages`` (not on the pages) folds a candidate page into the page
  before it when every head fits, keeping each head's row order.

Pinned by ``tests/test_oracle_diversity.py``: closed forms (identical
directions score -1; an orthonormal set scores -1/sqrt(n); scores are
invariant to positive scaling of a key; the mean of the scores of n keys is
-|m|), a brute-force cosine with exactly rounded component sums on small inputs, the
worked budget example in ``tests/golden/diversity_budget_example.txt``, and the
softmax budgets' limits (equal averages split evenly, a cold temperature gives
everything to the most diverse layer); for ``merge_pages``, a hand-worked
example and invariants after pruning (each head's token order unchanged, no
page over T rows in any head, no adjacent pair of candidate pages left that
fits, the merged pages' ids freed).
"""

from __future__ import annotations

import numpy as np

from . import clces


def diversity_scores(keys: np.ndarray) -> np.ndarray:
    """Negative cosine similarity of each key (rows) to the mean normalised key, float64."""
    k = np.asarray(keys, dtype=np.float64)
    norm = np.sqrt((k * k).sum(axis=1))
    khat = np.zeros_like(k)
    nz = norm > 0
    khat[nz] = k[nz] / norm[nz, None]
    m = khat.mean(axis=0) if len(k) else np.zeros(k.shape[1])
    mn = np.sqrt((m * m).sum())
    if mn == 0:
        return np.zeros(len(k))
    # a fixed-order sum per row (not a BLAS product): identical keys score identically, so exact ties
    # reach the index tie-break of the top-K
    return -((khat * m).sum(axis=1)) / mn


def topk_desc(scores: np.ndarray, k: int) -> np.ndarray:
    """Boolean mask of the k highest scores, ties by index."""
    s = np.asarray(scores, dtype=np.float64)
    keep = np.zeros(len(s), dtype=bool)
    keep[np.argsort(-s, kind="stable")[:k]] = True
    return keep


def layer_budgets(mean_diversity, tau: float, total: int, heads: int) -> np.ndarray:
    """Tokens per head of each layer from the tempered softmax over the layers' average diversity."""
    d = np.asarray(mean_diversity, dtype=np.float64) / tau
    e = np.exp(d - d.max())
    p = e / e.sum()
    return np.floor(np.floor(p * total) / heads).astype(np.int64)


class DiversityCache:
    """One layer: ``table`` = list of [page_id, frame, ids_per_head (list of H int arrays)].

    The anchor is frame 0's page; keys come from ``key_of(frame, head)`` giving a [T, D] array."""

    def __init__(self, heads: int, tokens_per_frame: int, num_pages: int):
        self.H = heads
        self.T = tokens_per_frame
        self.free = set(range(num_pages))
        self.table: list[list] = []

    def append(self, t: int) -> int:
        pid = min(self.free)
        self.free.remove(pid)
        ids = t * self.T + np.arange(self.T, dtype=np.int64)
        self.table.append([pid, t, [ids.copy() for _ in range(self.H)]])
        return pid

    def candidates(self, h: int) -> np.ndarray:
        parts = [ids[h] for _, f, ids in self.table if f > 0]
        return np.concatenate(parts) if parts else np.zeros(0, np.int64)

    def all_ids(self, h: int) -> np.ndarray:
        parts = [ids[h] for _, _, ids in self.table]
        return np.concatenate(parts) if parts else np.zeros(0, np.int64)

    def scores(self, key_of) -> list[np.ndarray]:
        """Per head: the diversity score of every candidate, in candidate order."""
        out = []
        for h in range(self.H):
            cand = self.candidates(h)
            keys = np.stack([key_of(int(i) // self.T, h)[int(i) % self.T] for i in cand]) if len(cand) else \
                np.zeros((0, 64))
            out.append(diversity_scores(keys))
        return out

    def mean_diversity(self, key_of) -> float:
        s = self.scores(key_of)
        n = sum(len(x) for x in s)
        return float(sum(x.sum() for x in s) / n) if n else 0.0

    def prune(self, key_of, k_per_head: int) -> list[np.ndarray]:
        """Keep each head's k_per_head most diverse candidates (float64 scores); return the per-head keep masks."""
        masks = []
        sc = self.scores(key_of)
        for h in range(self.H):
            masks.append(topk_desc(sc[h], k_per_head) if len(sc[h]) > k_per_head else np.ones(len(sc[h]), bool))
        pos = [0] * self.H
        out = []
        for pid, f, ids in self.table:
            if f == 0:
                out.append([pid, f, ids])
                continue
            new_ids = []
            for h in range(self.H):
                m = masks[h][pos[h]:pos[h] + len(ids[h])]
                pos[h] += len(ids[h])
                new_ids.append(clces.compact_page(ids[h], m))
            if all(len(x) == 0 for x in new_ids):
                self.free.add(pid)
            else:
                out.append([pid, f, new_ids])
        self.table = out
        return masks

    def merge_pages(self) -> list[tuple[int, int, tuple, tuple]]:
        """Append each candidate page to the page before it when, in every head, their lengths sum to at most
        T; return the moves ``(src_page, dst_page, per-head dst slots, per-head counts)`` in table order.

        A design step, not on the pages: it bounds the ragged pages that per-head pruning leaves.  Rows keep
        their table-then-slot order in every head, so candidate indices (the top-K tie-break) do not change.
        The anchor page is neither merged nor merged into; a merged page keeps the frame of its first page."""
        moves = []
        out = []
        for pid, f, ids in self.table:
            if f == 0 or not out or out[-1][1] == 0 or \
                    any(len(out[-1][2][h]) + len(ids[h]) > self.T for h in range(self.H)):
                out.append([pid, f, ids])
                continue
            dst = out[-1]
            moves.append((pid, dst[0], tuple(len(x) for x in dst[2]), tuple(len(x) for x in ids)))
            dst[2] = [np.concatenate([dst[2][h], ids[h]]) for h in range(self.H)]
            self.free.add(pid)
        self.table = out
        return moves

    def page_table(self) -> list[tuple[int, int, tuple]]:
        """(page_id, frame, per-head lengths) per entry, in table order."""
        return [(pid, f, tuple(len(x) for x in ids)) for pid, f, ids in self.table]
