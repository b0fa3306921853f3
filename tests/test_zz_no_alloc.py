"""gca_step_noalloc (split partials in the library's static device array)
against gca_step (partials in the workspace), through the C ABI: the same
kernels run with the same split counts, so the outputs must agree bit for
bit, and both must meet the oracle's tolerance.  Two streams in a row, the
second with smaller frames and fewer heads, then a step whose partials do not
fit the array, which is refused with the state unchanged."""
import math

import numpy as np
import pytest
import torch

from geometric_context_attention_amd import _lib as G
from geometric_context_attention_amd.synth import StreamSpec, draw_frames
from oracle import gca_oracle as go
from oracle.gca_oracle import GcaShape
from oracle.page_model import PageModel
from tests.gpu_util import check_outputs, check_state, say, to64

pytestmark = pytest.mark.gpu

STATIC_BYTES = 32 << 20


def _pair(mode, M, n, k, T, H, seed):
    gdt, tdt = {"bf16": (G.GCA_BF16, torch.bfloat16), "fp32": (G.GCA_FP32, torch.float32)}[mode]
    F = M + 6
    cfg = G.make_config(num_heads=H, image_tokens=M, n_anchor=n, k_window=k, max_frames=T, dtype=gdt)
    a, b = G.GcaStack(cfg), G.GcaStack(cfg)
    spec = StreamSpec(H=H, D=64, M=M, dtype=tdt, seed=seed, chunk=16)
    q, kx, v = draw_frames(spec, 0, 0, T)
    shp = GcaShape(M=M, n=n, k=k)
    o_ref, l_ref = go.stream_online(to64(q), to64(kx), to64(v), shp, 1 / math.sqrt(64))
    qd, kd, vd = q.cuda(), kx.cuda(), v.cuda()
    rows = n * F
    for st in (a, b):
        st.anchor_init(0, qd[:n].reshape(rows, H, 64), kd[:n].reshape(rows, H, 64), vd[:n].reshape(rows, H, 64))
    return cfg, a, b, (qd, kd, vd), (o_ref, l_ref), tdt


def _noalloc_step(st, t, qd, kd, vd):
    out = torch.empty_like(qd[t])
    lse = torch.empty((st.cfg.num_heads, st.F), dtype=torch.float32, device="cuda")
    G.gca_step_noalloc(st.ctx, 0, qd[t], kd[t], vd[t], out, lse)
    return out, lse


@pytest.mark.parametrize("mode,M,n,k,T,H", [
    ("bf16", 500, 3, 8, 24, 16),   # the benchmark's frame shape: 16 key splits per head
    ("bf16", 100, 2, 3, 20, 4),    # then smaller frames and fewer heads on the same array
])
def test_noalloc_matches_step(mode, M, n, k, T, H):
    cfg, a, b, (qd, kd, vd), (o_ref, l_ref), _ = _pair(mode, M, n, k, T, H, seed=11)
    splits = [G.gca_plan(cfg, t)["splits"] for t in range(n, T)]
    assert max(splits) > 1, "the case must use split partials"
    for t in range(n, T):
        oa, la = a.step(0, qd[t], kd[t], vd[t])
        ob, lb = _noalloc_step(b, t, qd, kd, vd)
        assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)), f"step {t}: outputs differ"
        assert torch.equal(la, lb), f"step {t}: LSE differs"
        check_outputs(ob, o_ref[t], lb, l_ref[t], mode, f"noalloc step {t}")
    sa, sb = a.export_state(0), b.export_state(0)
    assert sb["device_error"] == 0
    assert np.array_equal(sa["frame_table"], sb["frame_table"])
    assert np.array_equal(sa["used_bitmap"], sb["used_bitmap"])
    say(f"  noalloc {mode} M={M} H={H}: {T - n} steps bit-identical to gca_step, splits up to {max(splits)}")
    a.close()
    b.close()


def test_noalloc_refuses_partials_beyond_the_array():
    """fp32 frames of 106 rows (one 256-row query block, padded to 512 rows of
    partials) with 4 heads: once 64 pages are visible the step uses 64 splits,
    4 * 64 * 512 * 64 * 4 bytes of O plus the (m, l) pairs > 32 MiB."""
    M, n, k, T, H = 100, 3, 40, 48, 4
    F = M + 6
    cfg, a, b, (qd, kd, vd), (o_ref, l_ref), _ = _pair("fp32", M, n, k, T, H, seed=12)

    def need(t):
        s = G.gca_plan(cfg, t)["splits"]
        return (H * s * 512 * 64 * 4 + H * s * 512 * 8) if s > 1 else 0

    t_big = next(t for t in range(n, T) if need(t) > STATIC_BYTES)
    pm = PageModel(n=n, k=k, F=F, S=6, P=64, num_pages=G.gca_plan(cfg, 0)["pool_pages"], max_frames=T)
    pm.anchor_init()
    for t in range(n, t_big):
        oa, _ = a.step(0, qd[t], kd[t], vd[t])
        ob, _ = _noalloc_step(b, t, qd, kd, vd)
        assert torch.equal(oa, ob), f"step {t}: outputs differ"
        pm.step(t)
    with pytest.raises(G.GcaError) as e:
        _noalloc_step(b, t_big, qd, kd, vd)
    assert e.value.code == G.GCA_E_INVALID_ARG
    check_state(b, 0, pm)  # nothing changed
    ob, lb = b.step(0, qd[t_big], kd[t_big], vd[t_big])  # gca_step serves it
    check_outputs(ob, o_ref[t_big], lb, l_ref[t_big], "fp32", f"step {t_big} after the refusal")
    say(f"  noalloc fp32: refused step {t_big} ({need(t_big)} bytes), served by gca_step")
    a.close()
    b.close()
