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


def swap23(s):
    s = np.asarray(s)
    return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1)


def check_state(stack: G.GcaStack, layer: int, pm: PageModel, rows_of=None):
    """Device page-table state equals the page model bit for bit; optionally
    the cached K/V bytes equal the input rows.

    rows_of(f, rows) -> (k [len, H, D], v [len, H, D]) device tensors of the
    input bits of frame f.
    """
    st = stack.export_state(layer)
    assert st["device_error"] == 0, f"device error flag {st['device_error']}"
    assert st["frames_appended"] == pm.n_frames
    assert st["n_traj"] == pm.n_traj
    assert st["n_summary_pages"] == len(pm.summary_pages)
    assert st["used_pages"] == pm.used_pages
    assert st["pool_pages"] == pm.num_pages
    bits = np.unpackbits(st["used_bitmap"].view(np.uint8), bitorder="little")[: pm.num_pages]
    assert bits.astype(bool).tolist() == pm.used_bitmap()
    ft = st["frame_table"]
    exp = np.full_like(ft, -1)
    for f, pages in pm.frame_pages.items():
        exp[f] = pages
    assert np.array_equal(ft, exp), "frame table differs"
    sp = st["summary_pages"]
    ns = len(pm.summary_pages)
    assert sp[:ns].tolist() == pm.summary_pages
    assert (sp[ns:] == -1).all()
    if rows_of is None:
        return
    kpool, vpool = stack.pools(layer)
    loc = pm.resident_locations()
    by_frame = {}
    for (f, r), (p, s) in loc.items():
        by_frame.setdefault(f, []).append((r, p, s))
    iv = torch.int16 if stack.dtype == torch.bfloat16 else torch.int32
    for f, lst in by_frame.items():
        lst.sort()
        rows = [r for r, _, _ in lst]
        pages = torch.tensor([p for _, p, _ in lst], device=kpool.device)
        slots = torch.tensor([s for _, _, s in lst], device=kpool.device)
        vcols = torch.tensor(swap23(np.array([s for _, _, s in lst])), device=kpool.device)
        k_in, v_in = rows_of(f, rows)
        k_got = kpool[pages, :, slots, :]              # [N, H, D]
        v_got = vpool[pages, :, :, vcols]              # [N, H, D]
        assert torch.equal(k_got.view(iv), k_in.contiguous().view(iv)), f"K bytes of frame {f}"
        assert torch.equal(v_got.view(iv), v_in.contiguous().view(iv)), f"V bytes of frame {f}"
