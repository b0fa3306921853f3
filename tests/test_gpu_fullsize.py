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
from geometric_context_attention_amd.synth import StreamSpec, draw_chunk
from oracle import gca_oracle as go
from oracle.gca_oracle import GcaShape
from oracle.page_model import PageModel
from tests.gpu_util import check_outputs, check_state, say, to64

pytestmark = pytest.mark.gpu

S, D, C = 6, 64, 32


def _fullsize(M, n, k, T, H, layer, samples, state_at=(), window_len=None, key_offset_std=0.0,
              heads=None, row_stride=1, bytes_at=()):
    F = M + S
    Tw = window_len or T
    spec = StreamSpec(H=H, D=D, M=M, S=S, dtype=torch.bfloat16, seed=0, chunk=C,
                      key_offset_std=key_offset_std)
    cfg = G.make_config(num_heads=H, image_tokens=M, summary_tokens=S, n_anchor=n, k_window=k,
                        max_frames=Tw, dtype=G.GCA_BF16)
    stack = G.GcaStack(cfg)
    pool = G.gca_plan(cfg, 0)["pool_pages"]
    pm = PageModel(n=n, k=k, F=F, S=S, P=64, num_pages=pool, max_frames=Tw)
    shp = GcaShape(M=M, n=n, k=k, S=S)
    scale = 1 / math.sqrt(D)
    hs = list(range(H)) if heads is None else list(heads)
    keep_chunks = (min(k, Tw) + 1) // C + 2
    keep = {}
    sum_k = torch.empty((T, S, H, D), dtype=torch.bfloat16)
    sum_v = torch.empty((T, S, H, D), dtype=torch.bfloat16)
    anc = None  # (q, k, v) of the current window's anchor frames, device
    checked = 0

    def frame(g):
        q, kk, v = keep[g // C]
        i = g % C
        return q[i], kk[i], v[i]

    def provider(w0, t):
        def get_rows(f, rows):
            rows = np.asarray(rows)
            g = w0 + f
            if f < n or f >= t - k:
                _, kk, v = frame(g) if f >= n else (None, anc[1][f], anc[2][f])
                kr = kk[torch.as_tensor(rows, device=kk.device)][:, hs]
                vr = v[torch.as_tensor(rows, device=v.device)][:, hs]
                return to64(kr), to64(vr)
            assert rows.max() < S, "trajectory frame asked for image rows"
            return to64(sum_k[g, rows][:, hs]), to64(sum_v[g, rows][:, hs])
        return get_rows

    def rows_batch(w0):
        def fn(fr, rw):
            out_k = torch.empty((len(fr), H, D), dtype=torch.bfloat16, device="cuda")
            out_v = torch.empty_like(out_k)
            summ = rw < S
            idx = np.nonzero(summ)[0]
            gi = torch.as_tensor(w0 + fr[idx])
            ri = torch.as_tensor(rw[idx])
            out_k[torch.as_tensor(idx, device="cuda")] = sum_k[gi, ri].cuda()
            out_v[torch.as_tensor(idx, device="cuda")] = sum_v[gi, ri].cuda()
            for f in np.unique(fr[~summ]):
                sel = np.nonzero((fr == f) & ~summ)[0]
                if f < n:
                    kk, v = anc[1][f], anc[2][f]
                else:
                    _, kk, v = frame(w0 + f)
                r = torch.as_tensor(rw[sel], device="cuda")
                out_k[torch.as_tensor(sel, device="cuda")] = kk[r]
                out_v[torch.as_tensor(sel, device="cuda")] = v[r]
            return out_k, out_v
        return fn

    for g in range(T):
        if g % C == 0:
            c = g // C
            keep[c] = draw_chunk(spec, layer, c, device="cuda")
            hi = min(C, T - g)
            sum_k[g:g + hi] = keep[c][1][:hi, :S].cpu()
            sum_v[g:g + hi] = keep[c][2][:hi, :S].cpu()
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
            qa = torch.stack([frame(w0 + f)[0] for f in range(n)]).reshape(n * F, H, D)
            ka = torch.stack([frame(w0 + f)[1] for f in range(n)])
            va = torch.stack([frame(w0 + f)[2] for f in range(n)])
            anc = (qa, ka, va)
            out, lse = stack.anchor_init(0, qa, ka.reshape(n * F, H, D), va.reshape(n * F, H, D))
            pm.anchor_init()
            if g in samples:
                ref, lref = go.anchor_init(to64(qa)[:, hs], to64(ka.reshape(n * F, H, D))[:, hs],
                                           to64(va.reshape(n * F, H, D))[:, hs], scale)
                check_outputs(out[:, hs], ref, lse[hs], lref, "bf16", f"anchor init at frame {g}")
                checked += 1
        else:
            q, kk, v = frame(g)
            out, lse = stack.step(0, q, kk, v)
            pm.step(t)
            if g in samples:
                rows = np.arange(0, F, row_stride)
                ref, lref = go.step(t, to64(q)[rows][:, hs], provider(w0, t), shp, scale)
                ma, rel = check_outputs(out[torch.as_tensor(rows, device="cuda")][:, hs], ref,
                                        lse[hs][:, torch.as_tensor(rows, device="cuda")], lref,
                                        "bf16", f"frame {g} (step {t})")
                say(f"  frame {g}: keys {go.visible_key_count(t, shp)}, max-abs {ma:.2e}, rel {rel:.2e}")
                checked += 1
        if g in state_at:
            check_state(stack, 0, pm, rows_of_batch=rows_batch(w0) if g in bytes_at else None)
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
