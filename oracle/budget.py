"""Per-layer token-budget policy: append a frame, score with CLCES, keep the top K.

Oracle (test infrastructure only).  Sources: InfiniteVGGT explainer ("InfiniteVGGT:
Visual Geometry Grounded Transformer for Endless Streams"), "Rolling Memory"
(candidates = the cache plus the new frame's tokens; score; keep the best;
discard the rest so the size stays bounded) and step "Prune and roll the
memory"; StreamCacheVGGT article, section 2.1 (the score used here is the
fused CLCES score, computed by ``oracle.clces``).

Readings taken where the pages are silent:

* one page per appended frame from a per-layer pool, lowest free id first;
* the candidates of layer ``l`` are the layer's own cached tokens in table
  order (pages of the first ``scale_frames`` frames excluded: they are never
  scored nor dropped); ranks at every window layer are taken over that same
  candidate set, using each token's raw score at that layer, read from a
  table indexed by the global token id ``frame * T + slot``;
* the step runs only when the candidates exceed the budget, and keeps exactly
  ``budget`` of them;
* compaction is page-local (see ``oracle.clces.compact_page``); pages left
  empty are released and leave the table; the table order never changes.

Page merge (``merge_pages``) is not on the pages: it defragments the ragged
pages that compaction leaves.  Walking the table from its first non-scale
page, a page whose length fits after the page before it (sum at most one
frame's tokens) is appended to that page and its id is released; the token
sequence in table order is unchanged.

Pinned by ``tests/test_oracle_budget.py``: the kept set equals a direct top-K
over the flat candidate list (a second formulation without pages), the size
bound after every frame, id bookkeeping invariants, and for the merge the
hand example in ``tests/golden/merge_hand_example.txt``, the unchanged token
sequence, and the greedy properties (every adjacent pair left sums past one
page, so fewer than 2N/T + 1 pages remain).
"""

from __future__ import annotations

import numpy as np

from . import clces


class BudgetCache:
    """One layer's cache under the token budget; ``table`` = list of [page_id, frame, token_ids]."""

    def __init__(self, layer: int, tokens_per_frame: int, budget: int, num_pages: int,
                 window: int = 5, lam: float = 0.5, scale_frames: int = 0):
        self.layer = layer
        self.T = tokens_per_frame
        self.budget = budget
        self.window = window
        self.lam = lam
        self.S = scale_frames
        self.free = set(range(num_pages))
        self.table: list[list] = []
        self.compactions = 0
        self.last = None  # dict of the last CLCES step (ranks, s_hat, keep ...)

    def append(self, t: int) -> int:
        if not self.free:
            raise RuntimeError(f"no free page for frame {t}")
        pid = min(self.free)
        self.free.remove(pid)
        ids = t * self.T + np.arange(self.T, dtype=np.int64)
        self.table.append([pid, t, ids])
        return pid

    def merge_pages(self) -> list[tuple[int, int, int, int]]:
        """Append each page that fits after the page before it; return the moves.

        Moves are ``(src_page, dst_page, dst_slot, count)`` in table order."""
        moves = []
        out = []
        for entry in self.table:
            pid, f, ids = entry
            if f < self.S or not out or out[-1][1] < self.S or len(out[-1][2]) + len(ids) > self.T:
                out.append([pid, f, ids])
                continue
            dst = out[-1]
            moves.append((pid, dst[0], len(dst[2]), len(ids)))
            dst[2] = np.concatenate([dst[2], ids])
            self.free.add(pid)
        self.table = out
        self.merges = getattr(self, "merges", 0) + len(moves)
        return moves

    def candidate_ids(self) -> np.ndarray:
        parts = [ids for _, f, ids in self.table if f >= self.S]
        return np.concatenate(parts) if parts else np.zeros(0, np.int64)

    def all_ids(self) -> np.ndarray:
        parts = [ids for _, _, ids in self.table]
        return np.concatenate(parts) if parts else np.zeros(0, np.int64)

    def score_and_compact(self, score_table: np.ndarray, keep_count: int | None = None) -> bool:
        """Run one CLCES step if the candidates exceed the budget; return whether it ran.

        ``score_table[token_id, layer]`` holds the raw scores.
        """
        k = self.budget if keep_count is None else keep_count
        cand = self.candidate_ids()
        if len(cand) <= k:
            self.last = None
            return False
        layers = clces.window_layers(self.layer, self.window)
        s_win = np.stack([score_table[cand, lw] for lw in layers])
        res = clces.clces(s_win, self.lam)
        keep = clces.topk_keep(res["s_hat"], k)
        res["keep"] = keep
        res["keep_ids"] = cand[keep]
        res["candidate_ids"] = cand
        pos = 0
        new_table = []
        for entry in self.table:
            pid, f, ids = entry
            if f < self.S:
                new_table.append(entry)
                continue
            m = keep[pos:pos + len(ids)]
            pos += len(ids)
            kept = clces.compact_page(ids, m)
            if len(kept) == 0:
                self.free.add(pid)
            else:
                new_table.append([pid, f, kept])
        self.table = new_table
        self.compactions += 1
        self.last = res
        return True

    def page_table(self) -> list[tuple[int, int, int]]:
        """``(page_id, frame, length)`` per entry, in table order."""
        return [(pid, f, len(ids)) for pid, f, ids in self.table]
