"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these checks re-types the oracle's own code: each compares it with a
value printed on the pages, a closed form, a library routine on a special case
the method reduces to, or a scalar brute force written from the pages' prose.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import gca_oracle as go
from oracle.gca_oracle import GcaShape

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "token_counts.json")


def _golden():
    with open(GOLDEN) as fh:
        return {c["what"]: c for c in json.load(fh)["cases"]}


# ---------------------------------------------------------------------------
# (1) Cached-token count: printed values and the closed form M(n+k)+6T
#     (gitcode technical summary, §2.4 Total Tokens equation and table)
# ---------------------------------------------------------------------------

def test_cached_tokens_match_printed_values():
    g = _golden()
    c = g["gca_cached_tokens"]
    shp = GcaShape(M=c["M"], n=c["n"], k=c["k"], S=c["S"])
    gca = go.cached_token_count(c["T"] - 1, shp)
    assert gca == c["value"]
    # the affine part 9500 is M(n+k)
    a = g["gca_cached_tokens_affine_part"]
    assert gca - 6 * c["T"] == a["value"]
    cz = g["causal_cached_tokens"]
    causal = go.cached_token_count(cz["T"] - 1, GcaShape(M=cz["M"], n=cz["n"], k=cz["T"], S=cz["S"]))
    assert causal == cz["value"]
    r = g["compression_ratio"]
    assert abs(causal / gca - r["value"]) <= r["tolerance"]
    pf = g["per_frame_growth"]
    # growth per appended frame once the window is full: 6 summary rows
    a1 = go.cached_token_count(5000, shp)
    a0 = go.cached_token_count(4999, shp)
    assert a1 - a0 == pf["value_gca"]
    c1 = go.cached_token_count(5000, GcaShape(M=500, n=3, k=10 ** 6))
    c0 = go.cached_token_count(4999, GcaShape(M=500, n=3, k=10 ** 6))
    assert c1 - c0 == pf["value_causal"]


@pytest.mark.parametrize("M,n,k,S", [(32, 3, 4, 6), (500, 3, 64, 6), (7, 1, 0, 6), (5, 2, 2, 1),
                                     (999, 3, 64, 6), (3, 3, 1, 6)])
def test_cached_tokens_closed_form(M, n, k, S):
    shp = GcaShape(M=M, n=n, k=k, S=S)
    for T in list(range(n, n + k + 6)) + [n + k + 50, 300]:
        got = go.cached_token_count(T - 1, shp)
        if T >= n + k:
            assert got == M * (n + k) + S * T, (T, got)
        else:  # nothing has left the window yet: every row is cached
            assert got == (M + S) * T


# ---------------------------------------------------------------------------
# (2) k >= T reduces to frame-block causal attention (library SDPA)
#     (news article, attention-mask comparison figure: (b) causal vs (d) GCA;
#      technical summary §2.5 complexity table)
# ---------------------------------------------------------------------------

def _block_causal_mask(T, F, n):
    fr = torch.arange(T * F) // F
    qf = torch.clamp(fr, min=n - 1)[:, None]
    return fr[None, :] <= qf  # True = attend


def _sdpa(q, k, v, mask, scale):
    # [L, H, D] -> [H, L, D]
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).permute(1, 0, 2)
    vt = torch.from_numpy(v).permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("M,n,H,D,T", [(4, 3, 2, 8, 9), (5, 1, 1, 4, 7), (3, 2, 3, 16, 10)])
def test_large_window_is_block_causal(M, n, H, D, T):
    rng = np.random.default_rng(1)
    S = 6
    F = M + S
    shp = GcaShape(M=M, n=n, k=T, S=S)
    q, k, v = (rng.standard_normal((T, F, H, D)) for _ in range(3))
    scale = 1 / math.sqrt(D)
    ref = _sdpa(q.reshape(T * F, H, D), k.reshape(T * F, H, D), v.reshape(T * F, H, D),
                _block_causal_mask(T, F, n), scale).reshape(T, F, H, D)
    o_off, _ = go.stream_offline(q, k, v, shp, scale)
    o_on, _ = go.stream_online(q, k, v, shp, scale)
    np.testing.assert_allclose(o_off, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o_on, ref, rtol=0, atol=1e-12)


def test_anchor_block_is_unmasked_attention():
    rng = np.random.default_rng(2)
    n, F, H, D = 3, 11, 2, 8
    q, k, v = (rng.standard_normal((n * F, H, D)) for _ in range(3))
    scale = 0.3
    o, lse = go.anchor_init(q, k, v, scale)
    ref = _sdpa(q, k, v, None, scale)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    # LSE by its definition with the library's logsumexp
    s = torch.einsum("qhd,khd->hqk", torch.from_numpy(q), torch.from_numpy(k)) * scale
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# (3) Scalar brute force on tiny inputs.  The visible set is written here from
#     the pages' prose as three explicit frame sets (technical summary §2.2
#     frame-type table; paper-to-code map §二 2.1-2.3), not from the oracle's
#     rule function.
# ---------------------------------------------------------------------------

def _brute_visible(t, n, k, F, S):
    if t < n:
        return [(f, r) for f in range(n) for r in range(F)]
    anchors = list(range(n))
    window = [f for f in range(t - k, t) if f >= n]
    older = [f for f in range(n, t) if f not in window]
    keys = []
    for f in anchors + window + [t]:
        keys += [(f, r) for r in range(F)]
    for f in older:
        keys += [(f, r) for r in range(S)]
    return keys


def _brute_attend(qrow, keys, k, v, scale):
    H, D = qrow.shape
    out = np.zeros((H, v.shape[-1]))
    lse = np.zeros(H)
    for h in range(H):
        sc = []
        for (f, r) in keys:
            s = 0.0
            for d in range(D):
                s += qrow[h, d] * k[f, r, h, d]
            sc.append(s * scale)
        m = max(sc)
        w = [math.exp(x - m) for x in sc]
        den = sum(w)
        for j, (f, r) in enumerate(keys):
            for d in range(v.shape[-1]):
                out[h, d] += w[j] * v[f, r, h, d]
        out[h] /= den
        lse[h] = m + math.log(den)
    return out, lse


@pytest.mark.parametrize("n", [1, 2, 3])
@pytest.mark.parametrize("k", [0, 1, 2, "T"])
def test_brute_force_tiny(n, k):
    T, M, S, H, D = 9, 3, 6, 1, 5
    F = M + S
    kk = T if k == "T" else k
    shp = GcaShape(M=M, n=n, k=kk, S=S)
    rng = np.random.default_rng(10 * n + (kk if k != "T" else 99))
    q, kx, v = (rng.standard_normal((T, F, H, D)) for _ in range(3))
    scale = 0.7
    o_on, l_on = go.stream_online(q, kx, v, shp, scale)
    o_off, _ = go.stream_offline(q, kx, v, shp, scale)
    for t in range(T):
        keys = _brute_visible(t, n, kk, F, S)
        for r in (0, S - 1, S, F - 1):
            ob, lb = _brute_attend(q[t, r], keys, kx, v, scale)
            np.testing.assert_allclose(o_on[t, r], ob, rtol=0, atol=1e-12)
            np.testing.assert_allclose(o_off[t, r], ob, rtol=0, atol=1e-12)
            np.testing.assert_allclose(l_on[t, :, r], lb, rtol=0, atol=1e-12)


def test_mask_figure_n2_k2():
    """The news article's GCA mask figure uses n=2 anchors and k=2 window frames.

    Row pattern for query frame 6 of 7: anchors 0,1 full; frames 2,3 summary
    only; window 4,5 full; itself full.
    """
    shp = GcaShape(M=3, n=2, k=2, S=1)
    vis = go.frame_visibility(6, 7, shp)
    full = [True] * 4
    summ = [True, False, False, False]
    assert vis.tolist() == [full, full, summ, summ, full, full, full]
    # anchor frames see only the anchor block, both ways
    assert go.frame_visibility(0, 7, shp).tolist() == [full, full] + [[False] * 4] * 5


# ---------------------------------------------------------------------------
# (4) Closed forms: Q = 0 averages the visible V rows
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,k", [(3, 4), (1, 0), (2, 7)])
def test_zero_query_gives_mean_of_visible_values(n, k):
    M, S, H, D, T = 10, 6, 2, 4, 20
    F = M + S
    shp = GcaShape(M=M, n=n, k=k, S=S)
    q = np.zeros((T, F, H, D))
    kx = np.random.default_rng(3).standard_normal((T, F, H, D))
    v = np.zeros((T, F, H, D))
    v[:, :S, :, 0] = 1.0  # indicator of summary rows
    v[:, :, :, 1] = 2.5  # constant
    o, lse = go.stream_online(q, kx, v, shp, 0.5)
    for t in range(n, T):
        w = min(k, t - n)
        Lk = (n + w + 1) * F + S * (t - n - w)
        n_sum = S * (t + 1)
        np.testing.assert_allclose(o[t, :, :, 0], n_sum / Lk, rtol=0, atol=1e-14)
        np.testing.assert_allclose(o[t, :, :, 1], 2.5, rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[t], math.log(Lk), rtol=0, atol=1e-12)
    # anchor block: Lk = n*F
    np.testing.assert_allclose(o[:n, :, :, 0], S / F, rtol=0, atol=1e-14)


def test_visible_key_count_formula():
    """Keys seen at step t: full rows of anchors, window and current frame plus
    summaries of the older frames; for t >= n+k it is M(n+k+1) + 6(t+1)."""
    shp = GcaShape(M=500, n=3, k=64)
    for t in (3, 4, 66, 67, 68, 1000, 9999):
        w = min(shp.k, t - shp.n)
        exp = (shp.n + w + 1) * shp.F + 6 * (t - shp.n - w)
        assert go.visible_key_count(t, shp) == exp
        if t >= shp.n + shp.k:
            assert exp == 500 * (3 + 64 + 1) + 6 * (t + 1)
    assert go.visible_key_count(9999, shp) == 94000
    assert go.visible_key_count(9999, GcaShape(M=500, n=3, k=16)) == 70000


def test_streaming_equals_offline_random():
    rng = np.random.default_rng(4)
    shp = GcaShape(M=6, n=3, k=4, S=6)
    T, H, D = 14, 2, 8
    q, k, v = (rng.standard_normal((T, shp.F, H, D)) for _ in range(3))
    o_on, l_on = go.stream_online(q, k, v, shp, 0.35)
    o_off, l_off = go.stream_offline(q, k, v, shp, 0.35)
    np.testing.assert_allclose(o_on, o_off, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_on.transpose(1, 0, 2).reshape(H, -1), l_off, rtol=0, atol=1e-12)
