"""Helpers of the GPU parity tests: tolerance gates and bit-exact cache checks."""
from __future__ import annotations

import sys

import numpy as np
import torch

from geometric_context_attention_amd import _lib as G
from oracle.page_model import PageModel

# Tolerances.  max-abs gates: 2e-2 (bf16 in, fp32 accumulate) and 1e-4 (fp32).
# The extra relative gates catch an output that is small everywhere (at
# ~10^5 keys, |O| is ~0.02, so max-abs alone barely separates a wrong kernel
# from zeros).  LSE gates are absolute on natural-log values.
GATES = {
    "bf16": dict(max_abs=2e-2, rel_fro=1e-2, lse=1e-2),
    "fp32": dict(max_abs=1e-4, rel_fro=1e-5, lse=1e-4),
}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def check_outputs(o_gpu, o_ref, lse_gpu, lse_ref, mode, what=""):
    g = GATES[mode]
    o = to64(o_gpu)
    err = np.abs(o - o_ref)
    max_abs = float(err.max())
    rel = float(np.linalg.norm(o - o_ref) / max(np.linalg.norm(o_ref), 1e-300))
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    assert max_abs <= g["max_abs"], f"{what}: max-abs {max_abs:.3e} > {g['max_abs']}"
    assert rel <= g["rel_fro"], f"{what}: rel-Frobenius {rel:.3e} > {g['rel_fro']}"
    if lse_gpu is not None:
        le = float(np.abs(to64(lse_gpu) - lse_ref).max())
        assert le <= g["lse"], f"{what}: LSE error {le:.3e} > {g['lse']}"
    return max_abs, rel


def rotate_as_cached(x, tab):
    """Rotary rotation the way the cache stores it: x [..., H, D] (device),
    tab [..., D/2, 2] fp32; each product and the sum rounded separately in
    fp32 (no fused multiply-add), then rounded to x's dtype."""
    x0, x1 = x[..., 0::2].float(), x[..., 1::2].float()
    c, s = tab[..., None, :, 0], tab[..., None, :, 1]
    y = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y.to(x.dtype)


def swap23(s):
    s = np.asarray(s)
    return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1)


def check_state(stack: G.GcaStack, layer: int, pm: PageModel, rows_of=None, rows_of_batch=None):
    """Device page-table state equals the page model bit for bit; optionally
    the cached K/V bytes equal the input rows.

    rows_of(f, rows) -> (k [len, H, D], v [len, H, D]) device tensors holding
    the input bits of frame f; or rows_of_batch(frames, rows) -> (k, v)
    [N, H, D] for arrays of (frame, row) pairs.
    """
    st = stack.export_state(layer)
    assert st["device_error"] == 0, f"device error flag {st['device_error']}"
    assert st["frames_appended"] == pm.n_cached
    assert st["n_traj"] == pm.n_traj
    assert st["n_summary_pages"] == len(pm.summary_pages)
    assert st["used_pages"] == pm.used_pages
    assert st["pool_pages"] == pm.num_pages
    bits = np.unpackbits(st["used_bitmap"].view(np.uint8), bitorder="little")[: pm.num_pages]
    assert bits.astype(bool).tolist() == pm.used_bitmap()
    ft = st["frame_table"]
    exp = np.full_like(ft, -1)
    for f, pages in pm.frame_pages.items():
        exp[pm.slot_of(f)] = pages
    assert np.array_equal(ft, exp), "frame table differs"
    sp = st["summary_pages"]
    ns = len(pm.summary_pages)
    assert sp[:ns].tolist() == pm.summary_pages
    assert (sp[ns:] == -1).all()
    if rows_of is None and rows_of_batch is None:
        return
    kpool, vpool = stack.pools(layer)
    loc = pm.resident_locations()
    items = sorted(loc.items())
    fr = np.array([f for (f, _), _ in items])
    rw = np.array([r for (_, r), _ in items])
    pg = torch.tensor([p for _, (p, _) in items], device=kpool.device)
    sl = np.array([s for _, (_, s) in items])
    slots = torch.tensor(sl, device=kpool.device)
    vcols = torch.tensor(swap23(sl), device=kpool.device)
    if rows_of_batch is not None:
        k_in, v_in = rows_of_batch(fr, rw)
    else:
        ks, vs = [], []
        for f in np.unique(fr):
            sel = fr == f
            a, b = rows_of(int(f), rw[sel].tolist())
            ks.append(a); vs.append(b)
        k_in, v_in = torch.cat(ks), torch.cat(vs)
    iv = torch.int16 if stack.dtype == torch.bfloat16 else torch.int32
    k_got = kpool[pg, :, slots, :]              # [N, H, D]
    v_got = vpool[pg, :, :, vcols]              # [N, H, D]
    assert torch.equal(k_got.view(iv), k_in.to(kpool.device).contiguous().view(iv)), "cached K bytes differ"
    assert torch.equal(v_got.view(iv), v_in.to(kpool.device).contiguous().view(iv)), "cached V bytes differ"
