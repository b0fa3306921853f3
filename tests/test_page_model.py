"""Invariants of the page-allocator model (the policy the device cache follows)."""
import math

import pytest

from oracle import gca_oracle as go
from oracle.gca_oracle import GcaShape
from oracle.page_model import PageModel, pages_per_frame, pool_pages_needed


def _check_invariants(pm: PageModel):
    owned = []
    for pages in pm.frame_pages.values():
        owned += pages
    owned += pm.summary_pages
    assert len(owned) == len(set(owned)), "a page is owned twice"
    assert set(owned) == {p for p, u in enumerate(pm.used_bitmap()) if u}
    assert pm.used_pages + pm.used_bitmap().count(False) == pm.num_pages


def _closed_pool(n, k, F, S, P, T):
    ppf = pages_per_frame(F, P)
    return (n + min(k, T - 1 - n) + 1) * ppf + math.ceil(S * max(0, T - n - k) / P)


@pytest.mark.parametrize("M,S,n,k,P,T", [(32, 6, 3, 4, 64, 64), (58, 6, 3, 5, 64, 90), (500, 6, 3, 16, 64, 200),
                                         (3, 1, 1, 0, 2, 30), (120, 6, 2, 3, 32, 77), (10, 6, 3, 100, 64, 40)])
def test_stream_invariants_and_resident_rows(M, S, n, k, P, T):
    F = M + S
    shp = GcaShape(M=M, n=n, k=k, S=S)
    npages = _closed_pool(n, k, F, S, P, T)
    pm = PageModel(n=n, k=k, F=F, S=S, P=P, num_pages=npages, max_frames=T)
    pm.anchor_init()
    _check_invariants(pm)
    for t in range(n, T):
        pm.begin_step(t)
        _check_invariants(pm)
        # what the attention reads at step t: exactly the visible keys
        lst = pm.visible_page_list()
        assert sum(c for _, c in lst) == go.visible_key_count(t, shp)
        assert len({p for p, _ in lst}) == len(lst)
        pm.end_step(t)
        _check_invariants(pm)
        loc = pm.resident_locations()
        res = go.resident_rows(t, shp)
        want = {(f, r) for f in range(t + 1) for r in range(F) if res[f, r]}
        assert set(loc) == want
        assert len(set(loc.values())) == len(loc), "two rows share a slot"
    assert pm.peak_used == npages  # the closed-form pool is exactly the peak
    assert pool_pages_needed(n, k, F, S, P, T) == npages


def test_lowest_free_first_trace():
    """Hand-traced allocation: n=1, k=1, F=3 (S=1), P=2, so 2 pages per frame."""
    pm = PageModel(n=1, k=1, F=3, S=1, P=2, num_pages=8, max_frames=10)
    pm.anchor_init()
    assert pm.frame_pages == {0: [0, 1]}
    pm.step(1)  # frame 1 -> [2,3]; 1-1 = 0 < n: no eviction
    assert pm.frame_pages == {0: [0, 1], 1: [2, 3]} and pm.summary_pages == []
    pm.step(2)  # frame 2 -> [4,5]; evict 1: summary page 6 (lowest free), then free 2,3
    assert pm.frame_pages == {0: [0, 1], 2: [4, 5]} and pm.summary_pages == [6]
    pm.step(3)  # frame 3 reuses [2,3]; evict 2 into slot 1 of page 6; free 4,5
    assert pm.frame_pages == {0: [0, 1], 3: [2, 3]} and pm.summary_pages == [6]
    pm.step(4)  # frame 4 -> [4,5]; evict 3: slot 2 needs a new page: 7 (2,3 still used)
    assert pm.frame_pages == {0: [0, 1], 4: [4, 5]} and pm.summary_pages == [6, 7]
    assert pm.summary_location(2) == (7, 0)
    pm.step(5)
    assert pm.frame_pages == {0: [0, 1], 5: [2, 3]} and pm.summary_src == [(1, 0), (2, 0), (3, 0), (4, 0)]
    with pytest.raises(MemoryError):  # 8 pages: the next summary page does not fit
        for t in range(6, 10):
            pm.step(t)


def test_reset_returns_pool_to_empty():
    pm = PageModel(n=3, k=4, F=38, S=6, P=64, num_pages=14, max_frames=64)
    pm.anchor_init()
    for t in range(3, 40):
        pm.step(t)
    pm.reset()
    assert pm.used_pages == 0 and pm.frame_pages == {} and pm.summary_pages == []
    pm.anchor_init()
    assert pm.frame_pages == {0: [0], 1: [1], 2: [2]}


def test_pool_size_at_paper_shapes():
    # M=500 (+6) tokens per frame in pages of 64 -> 8 pages per frame
    assert pages_per_frame(506, 64) == 8 and pages_per_frame(1005, 64) == 16
    assert _closed_pool(3, 64, 506, 6, 64, 10000) == (3 + 64 + 1) * 8 + math.ceil(6 * 9933 / 64)
