"""Plant plausible mistakes in the oracle (on the CPU) and require a pin to fail.

This shows the pins are strong enough: a dropped term, an off-by-one window,
a wrong row order, a wrong scale or a swapped operand each break at least one
of the checks in test_oracle_pins.py.
"""
import numpy as np
import pytest

from oracle import gca_oracle as go
import tests.test_oracle_pins as pins

_orig_vis = go.is_visible
_orig_mask = go.step_key_mask
_orig_attn = go.masked_attention


def _rule(window_lo, summary_first=True, self_full=True, anchors_full=True):
    def is_visible(i, f, r, shp):
        n, k, S, F = shp.n, shp.k, shp.S, shp.F
        summ = (r < S) if summary_first else (r >= F - S)
        if i < n:
            return f < n
        if f > i:
            return False
        if f == i:
            return True if self_full else summ
        if f < n:
            return True if anchors_full else summ
        if f >= window_lo(i, k):
            return True
        return summ

    def step_key_mask(t, shp):
        n, k, S, F = shp.n, shp.k, shp.S, shp.F
        f = np.arange(t + 1)[:, None]
        r = np.arange(F)[None, :]
        if t < n:
            return np.broadcast_to(f < n, (t + 1, F)).reshape(-1)
        summ = (r < S) if summary_first else (r >= F - S)
        m = np.where(f == t, True if self_full else summ,
                     np.where(f < n, True if anchors_full else summ,
                              np.where(f >= window_lo(t, k), True, summ)))
        return np.broadcast_to(m, (t + 1, F)).reshape(-1)

    return is_visible, step_key_mask


def _attn(kind):
    def masked_attention(q, k, v, mask, scale):
        if kind == "inverted_scale":
            return _orig_attn(q, k, v, mask, 1.0 / scale)
        if kind == "values_are_keys":
            return _orig_attn(q, k, k, mask, scale)
        if kind == "lse_without_max":
            o, l = _orig_attn(q, k, v, mask, scale)
            qq = np.asarray(q, dtype=np.float64)
            kk = np.asarray(k, dtype=np.float64)
            for h in range(qq.shape[1]):
                s = qq[:, h] @ kk[:, h].T * scale
                if mask is not None:
                    s = np.where(mask, s, -np.inf)
                l[h] -= s.max(axis=1)
            return o, l
        raise KeyError(kind)
    return masked_attention


MUTATIONS = {
    "window_k_plus_1": ("rule", dict(window_lo=lambda i, k: i - k - 1)),
    "window_k_minus_1": ("rule", dict(window_lo=lambda i, k: i - k + 1)),
    "summary_rows_last": ("rule", dict(window_lo=lambda i, k: i - k, summary_first=False)),
    "current_frame_summary_only": ("rule", dict(window_lo=lambda i, k: i - k, self_full=False)),
    "anchors_summary_only": ("rule", dict(window_lo=lambda i, k: i - k, anchors_full=False)),
    "inverted_scale": ("attn", "inverted_scale"),
    "values_are_keys": ("attn", "values_are_keys"),
    "lse_without_max": ("attn", "lse_without_max"),
}


def _run_pins():
    checks = [
        pins.test_cached_tokens_match_printed_values,
        lambda: pins.test_cached_tokens_closed_form(32, 3, 4, 6),
        lambda: pins.test_large_window_is_block_causal(4, 3, 2, 8, 9),
        pins.test_anchor_block_is_unmasked_attention,
        lambda: pins.test_brute_force_tiny(2, 1),
        lambda: pins.test_brute_force_tiny(3, "T"),
        pins.test_mask_figure_n2_k2,
        lambda: pins.test_zero_query_gives_mean_of_visible_values(3, 4),
    ]
    failed = 0
    for c in checks:
        try:
            c()
        except AssertionError:
            failed += 1
    return failed


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    kind, arg = MUTATIONS[name]
    if kind == "rule":
        vis, mask = _rule(**arg)
        monkeypatch.setattr(go, "is_visible", vis)
        monkeypatch.setattr(go, "step_key_mask", mask)
    else:
        monkeypatch.setattr(go, "masked_attention", _attn(arg))
    assert _run_pins() >= 1, f"no pin caught mutation {name}"


def test_unmutated_oracle_passes_all():
    assert _run_pins() == 0
