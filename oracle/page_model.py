"""Exact model of the paged GCA cache: which page holds which row, step by step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages say the cache is paged so that the frequent appends and drops of a
streaming window do not force re-allocation (deep dive §3.4; news article,
inference paragraph), that a frame leaving the window keeps only its S
summary rows ("compressing eviction", paper-to-code map §二 2.3) and that
anchors stay (technical summary §2.2).  They do not give a page policy, so
this model fixes one, and the device cache must reproduce it bit for bit:

* The pool has ``num_pages`` pages of P token slots each.  A page is either
  free or used.  Allocation always takes the lowest-numbered free page.
* A full frame occupies ppf = ceil(F / P) pages of its own; its row r sits in
  page ``pages[r // P]``, slot ``r % P``.  The last page of a frame has
  F - (ppf-1)*P valid slots.
* Anchor initialisation appends frames 0..n-1 in order, each taking ppf
  pages in ascending order.
* Step t appends frame t the same way.  Then, if more than k keyframes after
  the anchors are cached, the oldest of them, e, leaves the window: for
  r = 0..S-1 its summary row r is copied to summary slot g = S*j + r, where j
  counts frames evicted before it; slot g lives in page
  ``summary_pages[g // P]`` at position g % P, and a new summary page (lowest
  free) is appended to that list when g // P reaches its length.  Only after
  the copy are frame e's ppf pages freed.  With keyframe interval 1 the frame
  evicted at step t is t - k, once t - k >= n.
* A step whose frame is not a keyframe (keyframe interval m > 1, deep dive
  §3.2) still attends to its own rows: it takes ppf pages the same way (lowest
  free first) for the duration of the step and frees them at its end, leaving
  the cache as it was.
* Reset frees everything.

Parity status: the policy is this repository's own specification, pinned by
invariants (no page used twice, used + free = pool, resident rows equal the
oracle's cached-token count, the closed form of the technical summary §2.4,
and the computed peak pool size).
"""
from __future__ import annotations

from dataclasses import dataclass, field


def pages_per_frame(F: int, P: int) -> int:
    return -(-F // P)


def pool_pages_needed(n: int, k: int, F: int, S: int, P: int, max_frames: int, m: int = 1) -> int:
    """Peak page count over a stream of max_frames frames (simulated)."""
    pm = PageModel(n=n, k=k, F=F, S=S, P=P, num_pages=10 ** 9, max_frames=max_frames, m=m)
    pm.anchor_init()
    for t in range(n, max_frames):
        pm.step(t)
    return pm.peak_used


@dataclass
class PageModel:
    n: int
    k: int
    F: int
    S: int
    P: int
    num_pages: int
    max_frames: int
    m: int = 1  # keyframe interval
    keyframes: frozenset | None = None  # explicit keyframes >= n (overrides m)
    used: list = field(default_factory=list)  # sorted free-list is derived
    frame_pages: dict = field(default_factory=dict)  # cached frame -> [pages]
    summary_pages: list = field(default_factory=list)
    summary_src: list = field(default_factory=list)  # slot g -> (frame, row)
    n_traj: int = 0
    n_frames: int = 0  # frames processed so far (next frame index)
    peak_used: int = 0
    transient: list = field(default_factory=list)  # pages of a non-keyframe step

    def __post_init__(self):
        self.ppf = pages_per_frame(self.F, self.P)
        self._used = set()
        self._free_hint = 0  # no page below this index is free

    # -- allocator ---------------------------------------------------------
    def _alloc(self) -> int:
        p = self._free_hint
        while p in self._used:
            p += 1
        if p >= self.num_pages:
            raise MemoryError("page pool exhausted")
        self._used.add(p)
        self._free_hint = p + 1
        self.peak_used = max(self.peak_used, len(self._used))
        return p

    def _free(self, p: int) -> None:
        self._used.remove(p)
        self._free_hint = min(self._free_hint, p)

    @property
    def used_pages(self) -> int:
        return len(self._used)

    def used_bitmap(self) -> list:
        return [p in self._used for p in range(self.num_pages)]

    # -- operations --------------------------------------------------------
    def is_keyframe(self, f: int) -> bool:
        if f < self.n:
            return True
        if self.keyframes is not None:
            return f in self.keyframes
        return self.m <= 1 or (f - self.n) % self.m == 0

    def slot_of(self, f: int) -> int:
        """Frame-table slot of cached frame f: anchors, then keyframes in order."""
        return sum(1 for g in range(f) if self.is_keyframe(g))

    @property
    def n_cached(self) -> int:
        """Frames appended to the cache so far (anchors and keyframes)."""
        return sum(1 for g in range(self.n_frames) if self.is_keyframe(g))

    def _append_frame(self, f: int) -> None:
        if f >= self.max_frames:
            raise ValueError("frame index beyond max_frames")
        self.frame_pages[f] = [self._alloc() for _ in range(self.ppf)]
        self.n_frames = f + 1

    def anchor_init(self) -> None:
        if self.n_frames != 0:
            raise RuntimeError("anchor_init on a non-empty cache")
        for f in range(self.n):
            self._append_frame(f)

    def _evict(self, e: int) -> None:
        for r in range(self.S):
            g = self.S * self.n_traj + r
            if g // self.P >= len(self.summary_pages):
                self.summary_pages.append(self._alloc())
            self.summary_src.append((e, r))
        for p in self.frame_pages.pop(e):
            self._free(p)
        self.n_traj += 1

    def begin_step(self, t: int) -> None:
        """Append frame t (or give it transient pages if it is not a
        keyframe); the attention of step t reads the cache after this."""
        if t != self.n_frames or t < self.n:
            raise RuntimeError("steps must follow anchor init in frame order")
        if self.is_keyframe(t):
            self._append_frame(t)
        else:
            if t >= self.max_frames:
                raise ValueError("frame index beyond max_frames")
            self.transient = [self._alloc() for _ in range(self.ppf)]
            self.n_frames = t + 1

    def end_step(self, t: int) -> None:
        """Evict the oldest window keyframe if more than k are cached; free a
        non-keyframe's transient pages."""
        if self.transient:
            for p in self.transient:
                self._free(p)
            self.transient = []
            return
        window = sorted(f for f in self.frame_pages if f >= self.n)
        if len(window) > self.k:
            self._evict(window[0])

    def step(self, t: int) -> None:
        self.begin_step(t)
        self.end_step(t)

    def reset(self) -> None:
        self.transient = []
        self._used.clear()
        self._free_hint = 0
        self.frame_pages.clear()
        self.summary_pages.clear()
        self.summary_src.clear()
        self.n_traj = 0
        self.n_frames = 0

    # -- queries -----------------------------------------------------------
    def frame_row_location(self, f: int, r: int):
        pages = self.frame_pages[f]
        return pages[r // self.P], r % self.P

    def summary_location(self, g: int):
        return self.summary_pages[g // self.P], g % self.P

    def resident_locations(self) -> dict:
        """(frame, row) -> (page, slot) for every cached row."""
        out = {}
        for f, pages in self.frame_pages.items():
            for r in range(self.F):
                out[(f, r)] = (pages[r // self.P], r % self.P)
        for g, (f, r) in enumerate(self.summary_src):
            out[(f, r)] = self.summary_location(g)
        return out

    def visible_page_list(self):
        """Pages a query of the newest frame attends to, with valid counts.

        Meaningful between ``begin_step`` and ``end_step`` (or right after
        ``anchor_init``, where it lists the anchor pages).

        Order: anchor frames, summary pages, window frames (oldest first),
        current frame.  Valid count = number of leading slots holding rows.
        """
        t = self.n_frames - 1
        out = []
        last_valid = self.F - (self.ppf - 1) * self.P
        for f in range(self.n):
            for j, p in enumerate(self.frame_pages[f]):
                out.append((p, self.P if j < self.ppf - 1 else last_valid))
        ns = self.S * self.n_traj
        for j, p in enumerate(self.summary_pages):
            out.append((p, min(self.P, ns - j * self.P)))
        for f in sorted(self.frame_pages):
            if f < self.n:
                continue
            for j, p in enumerate(self.frame_pages[f]):
                out.append((p, self.P if j < self.ppf - 1 else last_valid))
        if self.transient:  # the current frame, not cached
            for j, p in enumerate(self.transient):
                out.append((p, self.P if j < self.ppf - 1 else last_valid))
        else:
            assert t == max(self.frame_pages)
        return out
