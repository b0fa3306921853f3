"""Keyframe interval m > 1: frames attended but not cached (CPU, oracle pins).

The deep dive (§3.2, streaming loop; §3.3) describes the rule: after the n
anchor frames, frame i enters the cache only when (i - n) is a multiple of
the interval; any other frame is still predicted (its queries see the cache
and itself) but its keys and values are never appended, and the window counts
cached keyframes rather than video frames.

The oracle's mask for m > 1 is pinned against things other than itself:

* closed forms for the cached-token and visible-key counts, derived from that
  description (the counts reduce to the pages' M(n+k)+6T at m = 1);
* a structural reduction: since a non-keyframe leaves no trace, the m-stream
  must equal the m = 1 stream run on the anchors and keyframes alone, and a
  non-keyframe's output must equal what the same frame would get as the next
  frame of that dense stream (attention happens before appending);
* brute force over the three frame sets on tiny inputs;
* the page model and the C-ABI planner against the same counts.
"""
import math

import numpy as np
import pytest

from geometric_context_attention_amd import _lib as G
from oracle import gca_oracle as go
from oracle.gca_oracle import GcaShape
from oracle.page_model import PageModel, pages_per_frame, pool_pages_needed


def _keyframes_before(t, n, m):
    return max(0, -(-(t - n) // m))


@pytest.mark.parametrize("M,S,n,k,m", [(7, 6, 3, 4, 2), (5, 1, 1, 0, 3), (9, 6, 2, 3, 5), (4, 2, 3, 100, 4)])
def test_counts_closed_form(M, S, n, k, m):
    shp = GcaShape(M=M, n=n, k=k, S=S, m=m)
    F = M + S
    for t in range(n, 60):
        kb = _keyframes_before(t, n, m)
        assert go.visible_key_count(t, shp) == F * (n + min(k, kb) + 1) + S * max(0, kb - k)
        ka = _keyframes_before(t + 1, n, m)  # keyframes among n..t
        assert go.cached_token_count(t, shp) == F * (n + min(k, ka)) + S * max(0, ka - k)


def test_interval_one_is_the_dense_rule():
    a, b = GcaShape(M=5, n=2, k=3, S=2), GcaShape(M=5, n=2, k=3, S=2, m=1)
    for t in range(2, 30):
        assert np.array_equal(go.step_key_mask(t, a), go.step_key_mask(t, b))


@pytest.mark.parametrize("n,k,m", [(2, 2, 2), (1, 0, 3), (3, 1, 4), (2, 5, 3), (2, 2, "set"), (1, 3, "set")])
def test_stream_reduces_to_dense_stream_of_keyframes(n, k, m):
    T, M, S, H, D = 17, 3, 2, 2, 4
    F = M + S
    rng = np.random.default_rng(100 * n + 10 * k + (7 if m == "set" else m))
    q, kx, v = (rng.standard_normal((T, F, H, D)) for _ in range(3))
    scale = 0.6
    if m == "set":  # an arbitrary caller-chosen keyframe set
        chosen = frozenset(int(f) for f in range(n, T) if rng.random() < 0.45)
        shp = GcaShape(M=M, n=n, k=k, S=S, kf=chosen)
        keyframes = [f for f in range(T) if f < n or f in chosen]
    else:
        shp = GcaShape(M=M, n=n, k=k, S=S, m=m)
        keyframes = [f for f in range(T) if f < n or (f - n) % m == 0]
    o_m, l_m = go.stream_online(q, kx, v, shp, scale)
    dense = GcaShape(M=M, n=n, k=k, S=S)
    # keyframes: the dense stream over the keyframe subsequence
    o_d, l_d = go.stream_online(q[keyframes], kx[keyframes], v[keyframes], dense, scale)
    for j, f in enumerate(keyframes):
        np.testing.assert_allclose(o_m[f], o_d[j], rtol=0, atol=1e-12)
        np.testing.assert_allclose(l_m[f], l_d[j], rtol=0, atol=1e-12)
    # a non-keyframe: the next frame of the dense stream of the keyframes before it
    for i in range(n, T):
        if i in keyframes:
            continue
        seq = [f for f in keyframes if f < i] + [i]
        o_i, l_i = go.stream_online(q[seq], kx[seq], v[seq], dense, scale)
        np.testing.assert_allclose(o_m[i], o_i[-1], rtol=0, atol=1e-12)
        np.testing.assert_allclose(l_m[i], l_i[-1], rtol=0, atol=1e-12)


def _brute_visible(i, n, k, m, F, S):
    """Keys of query frame i, listed from the three frame sets directly."""
    if i < n:
        return [(f, r) for f in range(n) for r in range(F)]
    cached = [f for f in range(n, i) if (f - n) % m == 0]
    window = cached[max(0, len(cached) - k):] if k > 0 else []
    older = cached[: len(cached) - len(window)]
    keys = [(f, r) for f in range(n) for r in range(F)]
    keys += [(f, r) for f in older for r in range(S)]
    keys += [(f, r) for f in window for r in range(F)]
    keys += [(i, r) for r in range(F)]
    return keys


@pytest.mark.parametrize("n,k,m", [(1, 1, 2), (2, 0, 3), (3, 2, 2), (2, 3, 4)])
def test_visibility_brute_force(n, k, m):
    T, M, S = 20, 2, 2
    F = M + S
    shp = GcaShape(M=M, n=n, k=k, S=S, m=m)
    for i in range(T):
        want = set(_brute_visible(i, n, k, m, F, S))
        got = {(f, r) for f in range(T) for r in range(F) if go.is_visible(i, f, r, shp)}
        assert got == want
        if i >= n:
            mask = go.step_key_mask(i, shp).reshape(i + 1, F)
            assert {(f, r) for f in range(i + 1) for r in range(F) if mask[f, r]} == want


@pytest.mark.parametrize("M,S,n,k,P,T,m", [(32, 6, 3, 4, 64, 64, 3), (58, 6, 3, 5, 64, 90, 2),
                                           (3, 1, 1, 0, 2, 30, 4), (120, 6, 2, 3, 32, 77, 5)])
def test_page_model_with_keyframes(M, S, n, k, P, T, m):
    F = M + S
    shp = GcaShape(M=M, n=n, k=k, S=S, m=m)
    npages = pool_pages_needed(n, k, F, S, P, T, m)
    pm = PageModel(n=n, k=k, F=F, S=S, P=P, num_pages=npages, max_frames=T, m=m)
    pm.anchor_init()
    for t in range(n, T):
        before = (dict(pm.frame_pages), list(pm.summary_pages), pm.used_pages)
        pm.begin_step(t)
        lst = pm.visible_page_list()
        assert sum(c for _, c in lst) == go.visible_key_count(t, shp)
        assert len({p for p, _ in lst}) == len(lst)
        pm.end_step(t)
        if not pm.is_keyframe(t):  # the cache is exactly as before the step
            assert (dict(pm.frame_pages), list(pm.summary_pages), pm.used_pages) == before
        loc = pm.resident_locations()
        res = go.resident_rows(t, shp)
        assert set(loc) == {(f, r) for f in range(t + 1) for r in range(F) if res[f, r]}
        assert pm.n_cached == n + _keyframes_before(t + 1, n, m)
    # pool: the last step's frame, the window it sees and the summary pages
    kb_last = _keyframes_before(T - 1, n, m)
    ppf = pages_per_frame(F, P)
    closed = (n + min(k, kb_last) + 1) * ppf + math.ceil(S * max(0, _keyframes_before(T, n, m) - k) / P)
    assert npages == closed


@pytest.mark.parametrize("M,S,n,k,T,m", [(32, 6, 3, 4, 64, 3), (500, 6, 3, 64, 400, 4),
                                         (7, 1, 1, 0, 50, 2), (600, 6, 2, 3, 40, 5)])
def test_planner_matches_oracle_with_keyframes(M, S, n, k, T, m):
    cfg = G.make_config(num_heads=4, image_tokens=M, summary_tokens=S, n_anchor=n, k_window=k,
                        max_frames=T, keyframe_interval=m)
    shp = GcaShape(M=M, n=n, k=k, S=S, m=m)
    F = M + S
    pm = PageModel(n=n, k=k, F=F, S=S, P=64, num_pages=10 ** 6, max_frames=T, m=m)
    pm.anchor_init()
    for t in range(n, T):
        pm.begin_step(t)
        p = G.gca_plan(cfg, t)
        assert p["keys"] == go.visible_key_count(t, shp)
        assert p["pages_visible"] == len(pm.visible_page_list())
        pm.end_step(t)
        assert p["cached_after"] == go.cached_token_count(t, shp)
        assert p["used_pages_after"] == pm.used_pages
    assert p["pool_pages"] == pm.peak_used


def test_explicit_set_equal_to_schedule_is_the_schedule():
    n, m, T = 3, 4, 40
    sched = GcaShape(M=5, n=n, k=3, S=2, m=m)
    chosen = GcaShape(M=5, n=n, k=3, S=2, kf=frozenset(range(n, T, m)))
    for t in range(n, T):
        assert np.array_equal(go.step_key_mask(t, sched), go.step_key_mask(t, chosen))


def test_negative_interval_rejected():
    cfg = G.make_config(num_heads=2, image_tokens=8, n_anchor=1, k_window=1, max_frames=4,
                        keyframe_interval=-1)
    with pytest.raises(G.GcaError, match="keyframe_interval"):
        G.gca_workspace_bytes(cfg)


# ---------------------------------------------------------------------------
# Planted mistakes in the keyframe rule must break the pins above
# ---------------------------------------------------------------------------

def _mutant_mask(kind):
    def step_key_mask(t, shp):
        n, k, S, F = shp.n, shp.k, shp.S, shp.F
        f = np.arange(t + 1)[:, None]
        r = np.arange(F)[None, :]
        if t < n:
            return np.broadcast_to(f < n, (t + 1, F)).reshape(-1).copy()
        kf = (f < n) | ((f - n) % shp.m == 0)
        if kind == "non_keyframes_cached":
            kf = np.ones_like(kf)
        upto = np.cumsum(kf[:, 0])
        later = (upto[t - 1] - upto)[:, None]
        in_window = (f >= t - k) if kind == "window_counts_frames" else (later < k)
        full = (f == t) | (f < n) | (kf & in_window)
        return np.ascontiguousarray(full | (kf & (r < S))).reshape(-1)

    def is_visible(i, f, r, shp):
        if i < shp.n:
            return f < shp.n
        if f > i:
            return False
        return bool(step_key_mask(i, shp).reshape(i + 1, shp.F)[f, r])
    return step_key_mask, is_visible


@pytest.mark.parametrize("kind", ["non_keyframes_cached", "window_counts_frames"])
def test_planted_keyframe_mistakes_are_caught(kind, monkeypatch):
    mask, vis = _mutant_mask(kind)
    monkeypatch.setattr(go, "step_key_mask", mask)
    monkeypatch.setattr(go, "is_visible", vis)
    caught = 0
    for check, args in ((test_stream_reduces_to_dense_stream_of_keyframes, (2, 2, 2)),
                        (test_visibility_brute_force, (3, 2, 2)),
                        (test_counts_closed_form, (7, 6, 3, 4, 2))):
        try:
            check(*args)
        except AssertionError:
            caught += 1
    assert caught >= 1, f"mutation {kind} passed every keyframe pin"
