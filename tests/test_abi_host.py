"""Host-side checks of the C ABI (no GPU): symbols, config validation, planner."""
import ctypes
import os
import re

import pytest

from geometric_context_attention_amd import _lib as G
from oracle import gca_oracle as go
from oracle.gca_oracle import GcaShape
from oracle.page_model import PageModel

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "gca.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gca_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = G.lib()
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert sorted(G.exported_symbols()) == names


def _cfg(**kw):
    base = dict(num_layers=1, num_heads=2, head_dim=64, image_tokens=32, summary_tokens=6,
                n_anchor=3, k_window=4, max_frames=64, dtype=G.GCA_FP32)
    base.update(kw)
    return G.make_config(**base)


@pytest.mark.parametrize("bad,code", [
    (dict(head_dim=128), G.GCA_E_UNSUPPORTED), (dict(page_tokens=32), G.GCA_E_UNSUPPORTED),
    (dict(num_heads=0), G.GCA_E_INVALID_ARG), (dict(summary_tokens=0), G.GCA_E_INVALID_ARG),
    (dict(summary_tokens=65), G.GCA_E_INVALID_ARG), (dict(n_anchor=0), G.GCA_E_INVALID_ARG),
    (dict(k_window=-1), G.GCA_E_INVALID_ARG), (dict(max_frames=2), G.GCA_E_INVALID_ARG),
    (dict(dtype=7), G.GCA_E_INVALID_ARG), (dict(scale=-1.0), G.GCA_E_INVALID_ARG),
    (dict(num_layers=0), G.GCA_E_INVALID_ARG),
])
def test_invalid_configs_are_rejected(bad, code):
    cfg = _cfg(**bad)
    assert G.lib().gca_workspace_bytes(ctypes.byref(cfg)) == 0
    with pytest.raises(G.GcaError) as ei:
        G.gca_plan(cfg, 5)
    assert ei.value.code == code


def test_pool_smaller_than_the_anchor_block_is_rejected():
    """An explicit pool must hold the n anchor frames (3 frames x 2 pages here);
    a smaller one is refused before any workspace is sized."""
    cfg = _cfg(image_tokens=100, pool_pages=5)
    assert G.lib().gca_workspace_bytes(ctypes.byref(cfg)) == 0
    with pytest.raises(G.GcaError) as ei:
        G.gca_plan(cfg, 5)
    assert ei.value.code == G.GCA_E_INVALID_ARG
    assert G.gca_workspace_bytes(_cfg(image_tokens=100, pool_pages=6)) > 0


def test_workspace_grows_with_layers_and_pool():
    a = G.gca_workspace_bytes(_cfg())
    b = G.gca_workspace_bytes(_cfg(num_layers=3))
    c = G.gca_workspace_bytes(_cfg(max_frames=640))
    assert b > a and c > a
    assert a % 256 == 0


@pytest.mark.parametrize("M,S,n,k,T,dtype", [
    (32, 6, 3, 4, 64, G.GCA_FP32),
    (100, 6, 3, 5, 40, G.GCA_BF16),
    (500, 6, 3, 64, 400, G.GCA_BF16),
    (999, 6, 3, 64, 128, G.GCA_BF16),
    (7, 1, 1, 0, 50, G.GCA_BF16),
    (600, 6, 2, 3, 12, G.GCA_FP32),
])
def test_planner_matches_oracle(M, S, n, k, T, dtype):
    cfg = _cfg(image_tokens=M, summary_tokens=S, n_anchor=n, k_window=k, max_frames=T,
               num_heads=4, dtype=dtype)
    shp = GcaShape(M=M, n=n, k=k, S=S)
    F = M + S
    pm = PageModel(n=n, k=k, F=F, S=S, P=64, num_pages=10 ** 6, max_frames=T)
    pm.anchor_init()
    p = G.gca_plan(cfg, 0)
    assert p["keys"] == n * F and p["cached_after"] == n * F
    assert p["pages_visible"] == len(pm.visible_page_list())
    assert p["used_pages_after"] == pm.used_pages
    for t in range(n, T):
        pm.begin_step(t)
        p = G.gca_plan(cfg, t)
        assert p["keys"] == go.visible_key_count(t, shp)
        assert p["pages_visible"] == len(pm.visible_page_list())
        pm.end_step(t)
        assert p["cached_after"] == go.cached_token_count(t, shp)
        assert p["used_pages_after"] == pm.used_pages
        assert p["flop"] == 4.0 * F * p["keys"] * 64 * 4
        assert 1 <= p["splits"] <= p["pages_visible"]
    assert p["pool_pages"] == pm.peak_used


def test_planner_at_paper_shape():
    cfg = G.make_config(num_layers=12, num_heads=16, image_tokens=500, n_anchor=3, k_window=64,
                        max_frames=10000)
    p = G.gca_plan(cfg, 9999)
    assert p["keys"] == 94000
    assert p["cached_after"] == 500 * (3 + 64) + 6 * 10000
    assert p["pages_visible"] == 24 + -(-6 * 9932 // 64) + 65 * 8
    assert p["splits"] == 16 and p["qblocks"] == 1
    assert p["flop"] == pytest.approx(4 * 506 * 94000 * 64 * 16)
