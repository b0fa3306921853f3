"""Reference semantics of one GCA layer, materialised the slow and obvious way.

TEST INFRASTRUCTURE ONLY (see the package docstring): tests, the smoke check
and the benchmark's CPU-baseline leg are the only callers.

What is computed
----------------
Each frame f carries F = M + S token rows: S summary rows first (camera,
anchor, then registers; the technical summary, §2.3 summary-token table) and
then M image rows.  Row r < S of a frame is a summary row.

Visibility of key row (f, r) to a query row of frame i (rule ``is_visible``):

* Anchor block, i < n: the first n frames attend fully among themselves and
  to nothing later (paper-to-code map §二 2.1; deep dive §3.2, where the
  first frames are processed as one block).
* Streaming frame, i >= n: it sees every row of itself and of the n anchor
  frames, every row of the k window frames i-k .. i-1, and only the S summary
  rows of every older frame n .. i-k-1 (technical summary §2.2 frame-type
  table and §2.5 mask table; paper-to-code map §二 2.3).  Nothing later
  than i is visible.
* Keyframe interval m >= 1 (deep dive §3.2, the streaming loop, and §3.3):
  frame i >= n is a keyframe when (i - n) is a multiple of m; the anchors are
  always cached.  A frame that is not a keyframe is attended like any other
  current frame but never enters the cache, so no later frame sees any of
  its rows.  The window holds the k most recent keyframes before i (it
  counts cached keyframes, not video frames), and older keyframes keep only
  their summary rows.  With m = 1 this is the rule above.  The keyframes may
  also be given as an explicit set (the technical summary §5.1 picks them by
  an optical-flow threshold on the model's own predictions); the rule is the
  same with "keyframe" meaning "in the set".

Readings where the pages leave a step open (each is listed with its reason in
the design notes of the repository):

* the window is the k frames *before* the current one; the current frame is
  always visible to itself, bidirectionally;
* summary rows come first in a frame; within the summary, order does not
  matter to the output;
* the rule does not depend on the query row, and applies to every query
  frame, so a frame that is later in the window saw the same kind of context
  when it was current;
* the softmax scale is 1/sqrt(D) unless given; no position encoding is applied
  inside the step (Q and K arrive already encoded).

Attention is plain masked softmax attention per head in float64:
O = softmax(scale * Q K^T with -inf off the mask) V and
LSE = log sum exp(scale * Q K^T) over the visible keys.

Parity status: every function here is pinned by tests/ (closed-form token
counts from the technical summary §2.4, reduction to frame-block causal
attention for k >= T computed by torch's SDPA, reduction of the anchor block
to unmasked SDPA, scalar brute force on tiny inputs, and the Q = 0 mean
identities).  Values of attention outputs at the full sizes are not printed
on any page, so beyond those pins the oracle itself is the reference.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class GcaShape:
    """Sizes of one GCA stream (names follow the pages' notation)."""

    M: int  # image tokens per frame
    n: int  # anchor frames
    k: int  # pose-reference window frames (keyframes in the cache)
    S: int = 6  # summary tokens per frame (1 camera + 1 anchor + 4 register)
    m: int = 1  # keyframe interval: 1 appends every frame
    kf: frozenset | None = None  # explicit keyframes >= n (overrides m)

    @property
    def F(self) -> int:
        return self.M + self.S


# --------------------------------------------------------------------------
# Mask
# --------------------------------------------------------------------------

def is_keyframe(f: int, shp: GcaShape) -> bool:
    """True if frame f enters the cache (anchors always do)."""
    if f < shp.n:
        return True
    if shp.kf is not None:
        return f in shp.kf
    return shp.m <= 1 or (f - shp.n) % shp.m == 0


def is_visible(i: int, f: int, r: int, shp: GcaShape) -> bool:
    """True if key row r of frame f is visible to query frame i."""
    n, k, S = shp.n, shp.k, shp.S
    if i < n:  # anchor block: bidirectional among the first n frames
        return f < n
    if f > i:
        return False
    if f == i:  # the current frame sees all of itself
        return True
    if f < n:  # anchor context: all rows
        return True
    if not is_keyframe(f, shp):  # never cached
        return False
    later = sum(1 for g in range(f + 1, i) if is_keyframe(g, shp))
    if later < k:  # one of the k latest keyframes before i: all rows
        return True
    return r < S  # trajectory memory: summary rows only


def frame_visibility(i: int, num_frames: int, shp: GcaShape) -> np.ndarray:
    """Boolean [num_frames, F] mask over (frame, row) keys for query frame i."""
    F = shp.F
    out = np.zeros((num_frames, F), dtype=bool)
    for f in range(num_frames):
        for r in range(F):
            out[f, r] = is_visible(i, f, r, shp)
    return out


def step_key_mask(t: int, shp: GcaShape) -> np.ndarray:
    """Per-step key mask over all (t+1)*F tokens of frames 0..t, flattened.

    Same rule as ``is_visible``, evaluated for every (f, r) with numpy so that
    it stays cheap at t ~ 10^4.  Frame-major, row-minor token order.
    """
    n, k, S, F = shp.n, shp.k, shp.S, shp.F
    f = np.arange(t + 1)[:, None]
    r = np.arange(F)[None, :]
    if t < n:
        m = np.broadcast_to(f < n, (t + 1, F))
    else:
        if shp.kf is not None:
            kf = (f < n) | np.isin(f, np.array(sorted(shp.kf), dtype=np.int64))
        else:
            kf = (f < n) | (shp.m <= 1) | ((f - n) % max(shp.m, 1) == 0)
        upto = np.cumsum(kf[:, 0])  # keyframes among frames 0..f
        later = (upto[t - 1] - upto)[:, None]  # keyframes strictly between f and t
        full = (f == t) | (f < n) | (kf & (later < k))
        m = full | (kf & (r < S))
    return np.ascontiguousarray(m).reshape(-1)


def offline_mask(T: int, shp: GcaShape) -> np.ndarray:
    """All-frames 2-D boolean mask [T*F, T*F] (query token, key token)."""
    F = shp.F
    rows = []
    for i in range(T):
        vis = frame_visibility(i, T, shp).reshape(-1)
        rows.append(np.broadcast_to(vis, (F, T * F)))
    return np.concatenate(rows, axis=0)


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                     mask: np.ndarray | None, scale: float):
    """Softmax attention in float64, per head.

    q: [Lq, H, D]; k, v: [Lk, H, D]; mask: [Lq, Lk] bool or None (all True).
    Returns O [Lq, H, D] float64 and LSE [H, Lq] float64 (natural log).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Lq, H, D = q.shape
    out = np.empty((Lq, H, v.shape[2]), dtype=np.float64)
    lse = np.empty((H, Lq), dtype=np.float64)
    for h in range(H):
        s = (q[:, h, :] @ k[:, h, :].T) * scale
        if mask is not None:
            s = np.where(mask, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        l = p.sum(axis=1, keepdims=True)
        out[:, h, :] = (p @ v[:, h, :]) / l
        lse[h] = (m + np.log(l))[:, 0]
    return out, lse


def anchor_init(q, k, v, scale: float):
    """Anchor initialisation: full (unmasked) attention among n*F tokens.

    The first n frames are processed as one block and attend to each other
    without restriction (paper-to-code map §二 2.1; deep dive §3.2).
    """
    return masked_attention(q, k, v, None, scale)


def rotary(x, cos_sin):
    """Rotary position embedding (RoFormer, Su et al.): channels (2i, 2i+1) of
    each row turn by the angle whose (cos, sin) the table gives.

    The model encodes frame time (and optionally patch position) this way
    (technical summary §2.7; deep dive §3.1, the 3D-RoPE switch); the angles
    are inputs because the pages fix no frequency schedule.
    x: [rows, H, D]; cos_sin: [rows, D/2, 2].  Returns float64 [rows, H, D].
    Parity status: pinned against complex multiplication and the rotation
    group laws in tests/test_rotary.py.
    """
    x = np.asarray(x, dtype=np.float64)
    cs = np.asarray(cos_sin, dtype=np.float64)
    c, s = cs[:, None, :, 0], cs[:, None, :, 1]
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def frame_attention(q, k, v, scale: float):
    """Intra-frame attention: each frame's F tokens attend to all of themselves.

    The model alternates frame-attention layers with the GCA layers
    (technical summary §2.1; news article, pipeline figure); a frame-attention
    layer is plain unmasked softmax attention inside one frame.
    q, k, v: [B, F, H, D].  Returns O [B, F, H, D] and LSE [B, H, F].
    """
    B = q.shape[0]
    outs, lses = [], []
    for b in range(B):
        o, l = masked_attention(q[b], k[b], v[b], None, scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def step(t: int, q_t, get_rows, shp: GcaShape, scale: float):
    """GCA output for streaming frame t >= n.

    q_t: [Lq, H', D] queries of frame t (all F rows, or any subset of rows;
    H' may be a subset of the heads as long as get_rows returns the same).
    get_rows(f, rows) -> (k_rows, v_rows), each [len(rows), H', D]: the key
    and value rows of frame f at the given row indices.

    The per-step key mask over all (t+1)*F tokens is materialised and the
    visible columns gathered frame by frame.  The result does not depend on
    which query rows are passed (the rule does not depend on the query row).
    """
    if t < shp.n:
        raise ValueError("step() is for streaming frames t >= n")
    F = shp.F
    mask = step_key_mask(t, shp).reshape(t + 1, F)
    ks, vs = [], []
    for f in range(t + 1):
        rows = np.nonzero(mask[f])[0]
        if rows.size == 0:
            continue
        kf, vf = get_rows(f, rows)
        ks.append(np.asarray(kf, dtype=np.float64))
        vs.append(np.asarray(vf, dtype=np.float64))
    K = np.concatenate(ks, axis=0)
    V = np.concatenate(vs, axis=0)
    return masked_attention(q_t, K, V, None, scale)


def stream_offline(q, k, v, shp: GcaShape, scale: float):
    """Whole stream at once with the explicit 2-D mask over all T*F tokens.

    q, k, v: [T, F, H, D].  Returns O [T, F, H, D] and LSE [H, T*F].
    For tiny inputs only (the mask is (T*F)^2).
    """
    T, F, H, D = q.shape
    mask = offline_mask(T, shp)
    O, L = masked_attention(q.reshape(T * F, H, D), k.reshape(T * F, H, D),
                            v.reshape(T * F, H, D), mask, scale)
    return O.reshape(T, F, H, -1), L


def stream_online(q, k, v, shp: GcaShape, scale: float):
    """Streaming form: anchor init on frames 0..n-1, then one step per frame.

    q, k, v: [T, F, H, D].  Returns O [T, F, H, D] and LSE [T, H, F].
    """
    T, F, H, D = q.shape
    n = shp.n
    O = np.empty((T, F, H, v.shape[3]), dtype=np.float64)
    L = np.empty((T, H, F), dtype=np.float64)
    a_o, a_l = anchor_init(q[:n].reshape(n * F, H, D), k[:n].reshape(n * F, H, D),
                           v[:n].reshape(n * F, H, D), scale)
    O[:n] = a_o.reshape(n, F, H, -1)
    L[:n] = a_l.reshape(H, n, F).transpose(1, 0, 2)

    def get_rows(f, rows):
        return k[f][rows], v[f][rows]

    for t in range(n, T):
        o, l = step(t, q[t], get_rows, shp, scale)
        O[t] = o
        L[t] = l
    return O, L


# --------------------------------------------------------------------------
# Counts, obtained by counting the mask (not by formula)
# --------------------------------------------------------------------------

def visible_key_count(t: int, shp: GcaShape) -> int:
    """Number of keys a query of frame t attends to (count of the mask)."""
    return int(step_key_mask(t, shp).sum())


def resident_rows(t: int, shp: GcaShape) -> np.ndarray:
    """Rows that must stay cached after step t: those frame t+1 can see.

    Returns a boolean [(t+1), F] array over frames 0..t.
    """
    nxt = t + 1
    m = step_key_mask(nxt, shp).reshape(nxt + 1, shp.F)
    return m[: t + 1]


def cached_token_count(t: int, shp: GcaShape) -> int:
    """Cached tokens after frames 0..t have been processed (count of rows)."""
    return int(resident_rows(t, shp).sum())
