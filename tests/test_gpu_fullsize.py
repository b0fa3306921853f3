"""GPU parity at the paper's token shape (M = 500 or 999 image tokens + 6
summary tokens, 16 heads, head_dim 64, bf16), over whole streams in the
launch configuration the benchmark uses, checked at sampled steps.

The stream is drawn chunk by chunk on the GPU (synth recipe); the summary
rows of every frame are kept on the host, the recent chunks and the current
anchors in full, which is everything the oracle needs at a sampled step.
"""
import math

import numpy as np
import pytest
import torch

from geometric_context_attention_amd import _lib as G
from geometric_context_attention_amd.synth import StreamSpec, draw_chunk, rotary_table
from oracle import gca_oracle as go
from oracle.gca_oracle import GcaShape
from oracle.page_model import PageModel
from tests.gpu_util import check_outputs, check_state, rotate_as_cached, say, to64

pytestmark = pytest.mark.gpu

D, C = 64, 32


def _fullsize(M, n, k, T, H, layer, samples, state_at=(), window_len=None, key_offset_std=0.0,
              heads=None, row_stride=1, bytes_at=(), interval=1, rotary=False, S=6):
    F = M + S
    Tw = window_len or T
    spec = StreamSpec(H=H, D=D, M=M, S=S, dtype=torch.bfloat16, seed=0, chunk=C,
                      key_offset_std=key_offset_std)
    cfg = G.make_config(num_heads=H, image_tokens=M, summary_tokens=S, n_anchor=n, k_window=k,
                        max_frames=Tw, dtype=G.GCA_BF16, keyframe_interval=interval)
    stack = G.GcaStack(cfg)
    pool = G.gca_plan(cfg, 0)["pool_pages"]
    pm = PageModel(n=n, k=k, F=F, S=S, P=64, num_pages=pool, max_frames=Tw, m=interval)
    shp = GcaShape(M=M, n=n, k=k, S=S, m=interval)
    scale = 1 / math.sqrt(D)
    hs = list(range(H)) if heads is None else list(heads)
    keep_chunks = (min(k * interval, Tw) + 1) // C + 2  # the window spans k keyframes
    keep = {}
    sum_k = torch.empty((T, S, H, D), dtype=torch.bfloat16)
    sum_v = torch.empty((T, S, H, D), dtype=torch.bfloat16)
    # Rotary angles use the frame index as time (synth recipe); summary rows
    # sit at patch (0, 0), so their angles depend on the frame alone.
    tab_sum = rotary_table(0, T, S, S) if rotary else None  # [T, S, D/2, 2]
    tab_sum_d = tab_sum.cuda() if rotary else None
    anc = None  # (q, k, v, angles) of the current window's anchor frames, device
    checked = 0

    def frame(g):
        q, kk, v, tab = keep[g // C]
        i = g % C
        return q[i], kk[i], v[i], (tab[i] if rotary else None)

    def rot64(x, tab):
        """fp64 rows [len, H, D], rotated by the given angles when rotary is on."""
        x = to64(x)
        return go.rotary(x, to64(tab)) if rotary else x

    def provider(w0, t):
        def get_rows(f, rows):
            rows = np.asarray(rows)
            g = w0 + f
            ri = torch.as_tensor(rows)
            if rows.max() >= S:  # a full frame: anchor, window keyframe or the current frame
                if f < n:
                    kk, v, tab = anc[1][f], anc[2][f], (anc[3][f] if rotary else None)
                else:
                    assert g // C in keep, f"frame {g} left the kept chunks"
                    _, kk, v, tab = frame(g)
                rd = ri.to(kk.device)
                kr = rot64(kk[rd], tab[rd] if rotary else None)
                return kr[:, hs], to64(v[rd])[:, hs]
            kr = rot64(sum_k[g, ri], tab_sum[g, ri] if rotary else None)
            return kr[:, hs], to64(sum_v[g, ri])[:, hs]
        return get_rows

    def rows_batch(w0):
        def fn(fr, rw):
            out_k = torch.empty((len(fr), H, D), dtype=torch.bfloat16, device="cuda")
            out_v = torch.empty_like(out_k)
            out_t = torch.empty((len(fr), D // 2, 2), dtype=torch.float32, device="cuda")
            summ = rw < S
            idx = np.nonzero(summ)[0]
            gi = torch.as_tensor(w0 + fr[idx])
            ri = torch.as_tensor(rw[idx])
            di = torch.as_tensor(idx, device="cuda")
            out_k[di] = sum_k[gi, ri].cuda()
            out_v[di] = sum_v[gi, ri].cuda()
            if rotary:
                out_t[di] = tab_sum_d[gi.cuda(), ri.cuda()]
            for f in np.unique(fr[~summ]):
                sel = np.nonzero((fr == f) & ~summ)[0]
                if f < n:
                    kk, v, tab = anc[1][f], anc[2][f], (anc[3][f] if rotary else None)
                else:
                    _, kk, v, tab = frame(w0 + f)
                r = torch.as_tensor(rw[sel], device="cuda")
                ds = torch.as_tensor(sel, device="cuda")
                out_k[ds] = kk[r]
                out_v[ds] = v[r]
                if rotary:
                    out_t[ds] = tab[r]
            if rotary:
                out_k = rotate_as_cached(out_k, out_t)
            return out_k, out_v
        return fn

    for g in range(T):
        if g % C == 0:
            c = g // C
            q_c, k_c, v_c = draw_chunk(spec, layer, c, device="cuda")
            tab_c = rotary_table(c * C, C, F, S).cuda() if rotary else None  # [C, F, D/2, 2]
            keep[c] = (q_c, k_c, v_c, tab_c)
            hi = min(C, T - g)
            sum_k[g:g + hi] = k_c[:hi, :S].cpu()
            sum_v[g:g + hi] = v_c[:hi, :S].cpu()
            for old in [x for x in keep if x < c - keep_chunks]:
                del keep[old]
        t = g % Tw
        w0 = g - t
        if t == 0 and g > 0:
            stack.reset()
            pm.reset()
        if t < n - 1:
            continue
        if t == n - 1:
            fa = [frame(w0 + f) for f in range(n)]
            qa = torch.stack([x[0] for x in fa]).reshape(n * F, H, D)
            ka = torch.stack([x[1] for x in fa])
            va = torch.stack([x[2] for x in fa])
            ta = torch.stack([x[3] for x in fa]) if rotary else None  # kept alive with anc
            anc = (qa, ka, va, ta)
            if rotary:
                G.gca_set_rotary(stack.ctx, ta.reshape(n * F, D // 2, 2))
            out, lse = stack.anchor_init(0, qa, ka.reshape(n * F, H, D), va.reshape(n * F, H, D))
            pm.anchor_init()
            if g in samples:
                tq = ta.reshape(n * F, D // 2, 2) if rotary else None
                ref, lref = go.anchor_init(rot64(qa, tq)[:, hs], rot64(ka.reshape(n * F, H, D), tq)[:, hs],
                                           to64(va.reshape(n * F, H, D))[:, hs], scale)
                check_outputs(out[:, hs], ref, lse[hs], lref, "bf16", f"anchor init at frame {g}")
                checked += 1
        else:
            q, kk, v, tab = frame(g)
            if rotary:
                G.gca_set_rotary(stack.ctx, tab)
            out, lse = stack.step(0, q, kk, v)
            pm.step(t)
            if g in samples:
                rows = np.arange(0, F, row_stride)
                rd = torch.as_tensor(rows, device="cuda")
                qr = rot64(q[rd], tab[rd] if rotary else None)
                ref, lref = go.step(t, qr[:, hs], provider(w0, t), shp, scale)
                ma, rel = check_outputs(out[rd][:, hs], ref, lse[hs][:, rd], lref,
                                        "bf16", f"frame {g} (step {t})")
                say(f"  frame {g}: keys {go.visible_key_count(t, shp)}, max-abs {ma:.2e}, rel {rel:.2e}")
                checked += 1
        if g in state_at:
            check_state(stack, 0, pm, rows_of_batch=rows_batch(w0) if g in bytes_at else None)
    if rotary:
        G.gca_set_rotary(stack.ctx, None)
    assert checked == len(samples)
    stack.close()

def test_paper_shape_one_layer_k16_correlated_keys():
    """M=500+6, 16 heads, n=3, k=16, T=10000, per-frame key offsets N(0, 0.5^2);
    ends at 69,500 cached tokens."""
    T = 10000
    _fullsize(500, 3, 16, T, 16, layer=0, samples={2, 3, 4, 18, 19, 20, 1000, T - 1},
              state_at={2, 3, 19, 20, 1000, T - 1}, bytes_at={20, T - 1}, key_offset_std=0.5)


def test_direct_mode_layer_k64():
    """The benchmark's stack shape (k=64), layer index 11's seeds, T=10000."""
    T = 10000
    _fullsize(500, 3, 64, T, 16, layer=11, samples={3, 66, 67, 68, 5000, T - 1},
              state_at={67, 68, T - 1}, bytes_at={T - 1})


def test_dense_grid_with_window_resets():
    """M=999+6 (two 512-row query blocks), k=64, reset every 128 frames."""
    T = 10000
    _fullsize(999, 3, 64, T, 16, layer=0, window_len=128,
              samples={2, 3, 67, 68, 127, 130, 131, 5000, 9986, T - 1},
              state_at={127, 131, T - 1}, bytes_at={127, T - 1})


def test_full_causal_cache():
    """k >= T (every frame keeps all 506 tokens), T=2000: 1,012,000 keys at the
    last step; sampled heads and rows there."""
    T = 2000
    _fullsize(500, 3, T, T, 16, layer=0, samples={3, 1000, T - 1}, heads=(0, 7, 15), row_stride=4,
              state_at={1000, T - 1}, bytes_at={1000})


@pytest.mark.parametrize("interval,rotary", [(4, True), (4, False), (1, True)])
def test_keyframe_interval_and_rotary(interval, rotary):
    """The benchmark's variants at the paper's shape: keyframe interval 4
    (k=64 keyframes span 256 frames) and rotary angles on Q and cached K,
    M=500+6, 16 heads, T=3000."""
    T = 3000
    # keyframe 3 keeps only its summary rows once 64 later keyframes are cached:
    # from step 3 + 64 * interval + 1 on (68 for interval 1, 260 for interval 4)
    first_old = 3 + 64 * interval + 1
    _fullsize(500, 3, 64, T, 16, layer=3, interval=interval, rotary=rotary,
              samples={2, 3, 4, 5, first_old - 1, first_old, first_old + 1, 1501, T - 1},
              state_at={3, 4, first_old - 1, first_old, T - 1}, bytes_at={first_old, T - 1})


def test_one_summary_token():
    """S = 1 (camera token only): M=500+1, 16 heads, k=64, T=3000; 64 old
    frames share a summary page."""
    T = 3000
    _fullsize(500, 3, 64, T, 16, layer=5, S=1, samples={2, 3, 67, 68, 69, 131, 132, 1501, T - 1},
              state_at={68, 131, 132, T - 1}, bytes_at={132, T - 1})
