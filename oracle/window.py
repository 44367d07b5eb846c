"""Window policy of the bounded KV cache: which frames are kept, in which page.

Oracle (test infrastructure only).  Sources:

* GCTStream explainer ("How GCTStream Implements Streaming 3D Reconstruction
  with KV Cache"), section "Frame-by-Frame Causal Processing": only keyframes
  (every ``keyframe_interval``-th frame) persist their KV; other frames are
  attended and then discarded.  Section "Sliding Window Eviction": once the
  cache is over the window, the oldest blocks go.
* LingBot-Map 20 FPS explainer ("Can LingBot-Map Achieve 20 FPS Streaming 3D
  Reconstruction?"), section "Sliding-Window Eviction Strategy": the window is
  counted in frames (default 64) and the first ``kv_cache_scale_frames``
  (default 8) frames are kept for geometric consistency; FAQ "How does
  LingBot-Map handle sequences longer than 10,000 frames": evicts older
  frames while retaining the scale frames.

Readings taken where the pages are silent:

* the window counts persisted non-scale frames (not stream time);
* keyframe rule ``t < S or (t - S) % k == 0``;
* per frame: append, then evict, then attend; the current frame is part of
  its own attended set, as a transient entry when it is not a keyframe;
* the victim is the oldest persisted non-scale frame, one whole page;
* page ids come from a per-layer pool of ``num_pages`` ids, lowest free id
  first, allocated before the eviction of the same frame; a freed id is free
  at once.  The transient frame lives outside that pool.

Pinned by ``tests/test_oracle_window.py``: the closed form below is checked
against the allocator simulation (two independent formulations), the hand-made
page-table fixture ``tests/golden/config0_page_tables.txt``, the occupancy bound
and the frames/k growth claim.  The special-token variant is pinned by the
hand-worked fixture ``tests/golden/special_tokens_hand_example.txt``, by an
independent closed form of the held special ids on 60 random policies, by the
fill rule of its pages, and by reducing to the plain policy with no special
tokens.
"""

from __future__ import annotations


def is_keyframe(t: int, scale_frames: int, keyframe_interval: int) -> bool:
    """Whether frame ``t`` persists its KV (scale frames always do)."""
    if t < scale_frames:
        return True
    return (t - scale_frames) % keyframe_interval == 0


def persisted_frames(t: int, scale_frames: int, window: int, keyframe_interval: int) -> list[int]:
    """Closed form of the persisted set after frame ``t`` was appended and evicted.

    Scale frames ``0..min(t, S-1)``, then the last ``window`` keyframes among
    ``S..t`` (all of them when ``window == 0``, i.e. the window is off), in
    stream order.
    """
    scale = list(range(min(t + 1, scale_frames)))
    keys = [f for f in range(scale_frames, t + 1) if is_keyframe(f, scale_frames, keyframe_interval)]
    if window > 0:
        keys = keys[-window:]
    return scale + keys


def attended_frames(t: int, scale_frames: int, window: int, keyframe_interval: int) -> list[int]:
    """Frames whose tokens frame ``t`` attends to (t >= S): persisted set plus ``t`` itself."""
    frames = persisted_frames(t, scale_frames, window, keyframe_interval)
    if t not in frames:
        frames.append(t)
    return frames


class PoolExhausted(RuntimeError):
    pass


class WindowCache:
    """Simulation of one layer's page table under the window policy.

    ``table`` is the ordered list of ``(page_id, frame)`` pairs of the
    persisted pages (scale frames first, then window frames oldest to newest);
    ``transient`` is the frame held outside the pool for one attention call.
    """

    def __init__(self, scale_frames: int, window: int, keyframe_interval: int, num_pages: int):
        self.S = scale_frames
        self.W = window
        self.k = keyframe_interval
        self.num_pages = num_pages
        self.free = set(range(num_pages))
        self.table: list[tuple[int, int]] = []
        self.transient: int | None = None
        self.evictions = 0

    def append(self, t: int) -> None:
        if is_keyframe(t, self.S, self.k):
            if not self.free:
                raise PoolExhausted(f"no free page for frame {t}")
            pid = min(self.free)
            self.free.remove(pid)
            self.table.append((pid, t))
        else:
            self.transient = t

    def evict(self) -> int:
        n = 0
        if self.W <= 0:
            return 0
        while sum(1 for _, f in self.table if f >= self.S) > self.W:
            idx = next(i for i, (_, f) in enumerate(self.table) if f >= self.S)
            pid, _ = self.table.pop(idx)
            self.free.add(pid)
            n += 1
        self.evictions += n
        return n

    def attended(self) -> list[int]:
        """Frames of the next attention call, in logical (table) order; consumes the transient."""
        frames = [f for _, f in self.table]
        if self.transient is not None:
            frames.append(self.transient)
            self.transient = None
        return frames

    def persisted(self) -> list[int]:
        return [f for _, f in self.table]

    def page_ids(self) -> list[int]:
        return [p for p, _ in self.table]


class SpecialWindowCache(WindowCache):
    """The window policy with cross-frame special-token persistence.

    GCTStream explainer, "Special Token Persistence": with
    ``kv_cache_cross_frame_special`` the special tokens of a frame survive the
    eviction that discards the rest of its KV.  Readings taken where the page is silent:

    * the special tokens are the first ``special`` slots of every frame;
    * at each eviction (oldest victim first) the victim's special token ids
      go, in slot order, to the end of the layer's last special page; a new
      special page is taken (lowest free id, while the victim still holds its
      own id) when they do not fit in ``tokens_per_frame`` slots; then the
      victim's id is freed;
    * special pages sit after the scale frames, in the order they were
      opened, and are never evicted; they count as no frame of the window.

    ``table`` keeps the ``(page_id, frame)`` pairs of the frame pages;
    ``special_pages`` holds ``[page_id, [token ids]]`` lists.
    """

    def __init__(self, scale_frames: int, window: int, keyframe_interval: int, num_pages: int, special: int,
                 tokens_per_frame: int):
        super().__init__(scale_frames, window, keyframe_interval, num_pages)
        self.special = special
        self.T = tokens_per_frame
        self.special_pages: list[list] = []

    def evict(self) -> int:
        n = 0
        if self.W <= 0:
            return 0
        while sum(1 for _, f in self.table if f >= self.S) > self.W:
            idx = next(i for i, (_, f) in enumerate(self.table) if f >= self.S)
            pid, f = self.table[idx]
            if self.special > 0:
                if not self.special_pages or len(self.special_pages[-1][1]) + self.special > self.T:
                    if not self.free:
                        raise PoolExhausted(f"no free page for the special tokens of frame {f}")
                    sp = min(self.free)
                    self.free.remove(sp)
                    self.special_pages.append([sp, []])
                self.special_pages[-1][1].extend(f * self.T + j for j in range(self.special))
            self.table.pop(idx)
            self.free.add(pid)
            n += 1
        self.evictions += n
        return n

    def attended_tokens(self) -> list[int]:
        """Token ids of the next attention call in table order (scale frames, special pages, window frames,
        then the transient frame, which is consumed)."""
        scale = [f for _, f in self.table if f < self.S]
        rest = [f for _, f in self.table if f >= self.S]
        ids = [f * self.T + j for f in scale for j in range(self.T)]
        for _, toks in self.special_pages:
            ids.extend(toks)
        ids.extend(f * self.T + j for f in rest for j in range(self.T))
        if self.transient is not None:
            ids.extend(self.transient * self.T + j for j in range(self.T))
            self.transient = None
        return ids

    def page_table(self) -> list[tuple[int, int, int]]:
        """``(page_id, frame, length)`` per entry in table order; a special page reports ``-1 - f`` with ``f``
        the first frame whose special tokens it holds."""
        scale = [(p, f, self.T) for p, f in self.table if f < self.S]
        rest = [(p, f, self.T) for p, f in self.table if f >= self.S]
        special = [(p, -1 - toks[0] // self.T, len(toks)) for p, toks in self.special_pages]
        return scale + special + rest


def special_token_ids(t: int, scale_frames: int, window: int, keyframe_interval: int, special: int,
                      tokens_per_frame: int) -> list[int]:
    """Closed form: the special token ids held after frame ``t`` was appended and evicted -- the first
    ``special`` slots of every keyframe past the scale frames that is no longer persisted, oldest first."""
    kept = set(persisted_frames(t, scale_frames, window, keyframe_interval))
    gone = [f for f in range(scale_frames, t + 1)
            if is_keyframe(f, scale_frames, keyframe_interval) and f not in kept]
    return [f * tokens_per_frame + j for f in gone for j in range(special)]
