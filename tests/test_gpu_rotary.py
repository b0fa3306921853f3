"""GPU parity with rotary position embedding (gca_set_rotary) against the oracle.

Every frame gets its rows' rotary angles (a synthetic 3-axis table); the
oracle rotates Q and K in fp64 and attends as usual.  The cache must hold the
rotated keys: each product and the sum rounded separately in fp32, then
rounded to the stream dtype, which torch's eager fp32 arithmetic reproduces
bit for bit, so the cached bytes are compared exactly.
"""
import math

import pytest
import torch

from geometric_context_attention_amd import _lib as G
from geometric_context_attention_amd.synth import StreamSpec, draw_frames, rotary_table
from oracle import gca_oracle as go
from oracle.gca_oracle import GcaShape
from oracle.page_model import PageModel
from tests.gpu_util import check_outputs, check_state, rotate_as_cached, say, to64

pytestmark = pytest.mark.gpu

DT = {"bf16": (G.GCA_BF16, torch.bfloat16), "fp32": (G.GCA_FP32, torch.float32)}


@pytest.mark.parametrize("mode,M,H,k,T", [("fp32", 32, 2, 4, 30), ("bf16", 181, 4, 3, 24),
                                          ("fp32", 500, 4, 3, 10)])
def test_stream_with_rotary(mode, M, H, k, T):
    gdt, tdt = DT[mode]
    S, n = 6, 3
    F = M + S
    cfg = G.make_config(num_heads=H, image_tokens=M, summary_tokens=S, n_anchor=n, k_window=k,
                        max_frames=T, dtype=gdt)
    stack = G.GcaStack(cfg)
    spec = StreamSpec(H=H, D=64, M=M, S=S, dtype=tdt, seed=4, chunk=16)
    q, kx, v = draw_frames(spec, 0, 0, T)
    tab = rotary_table(0, T, F, S)  # [T, F, 32, 2]
    qr = go.rotary(to64(q).reshape(T * F, H, 64), tab.double().numpy().reshape(T * F, 32, 2))
    kr = go.rotary(to64(kx).reshape(T * F, H, 64), tab.double().numpy().reshape(T * F, 32, 2))
    shp = GcaShape(M=M, n=n, k=k, S=S)
    o_ref, l_ref = go.stream_online(qr.reshape(T, F, H, 64), kr.reshape(T, F, H, 64), to64(v), shp,
                                    1 / math.sqrt(64))
    qd, kd, vd, td = q.cuda(), kx.cuda(), v.cuda(), tab.cuda()
    k_cached = rotate_as_cached(kd, td)  # what the cache must hold
    pm = PageModel(n=n, k=k, F=F, S=S, P=64, num_pages=G.gca_plan(cfg, 0)["pool_pages"], max_frames=T)

    def rows_of(f, rows):
        return k_cached[f, rows], vd[f, rows]

    tab_a = td[:n].reshape(n * F, 32, 2).contiguous()  # must outlive the launches that read it
    G.gca_set_rotary(stack.ctx, tab_a)
    out, lse = stack.anchor_init(0, qd[:n].reshape(n * F, H, 64), kd[:n].reshape(n * F, H, 64),
                                 vd[:n].reshape(n * F, H, 64))
    torch.cuda.synchronize()
    pm.anchor_init()
    check_outputs(out.reshape(n, F, H, 64), o_ref[:n], lse.reshape(H, n, F).permute(1, 0, 2), l_ref[:n],
                  mode, "anchor init")
    check_state(stack, 0, pm, rows_of)
    worst = 0.0
    for t in range(n, T):
        G.gca_set_rotary(stack.ctx, td[t])
        out, lse = stack.step(0, qd[t], kd[t], vd[t])
        pm.step(t)
        ma, _ = check_outputs(out, o_ref[t], lse, l_ref[t], mode, f"step {t}")
        worst = max(worst, ma)
        check_state(stack, 0, pm, rows_of)
    G.gca_set_rotary(stack.ctx, None)
    say(f"  rotary {mode} M={M} H={H} k={k} T={T}: worst max-abs {worst:.2e}")
    stack.close()


@pytest.mark.parametrize("mode,B,M", [("bf16", 3, 250), ("bf16", 6, 250), ("bf16", 70, 250), ("fp32", 3, 250),
                                      ("bf16", 1, 181), ("bf16", 4, 447), ("bf16", 7, 181), ("bf16", 5, 500),
                                      ("bf16", 2, 40), ("bf16", 6, 40)])
def test_frame_attention_with_rotary(mode, B, M):
    """1-4 bf16 frames: one page per wave; 5 and more (70: a full launch of 64
    frames, then 6): each frame held in LDS; fp32: scratch pages.  M = 250
    fills 4 whole pages; 181 and 447 end in a partial page (3 and 8 pages),
    500 fills 8 pages with a partial last one, 40 a single partial page."""
    gdt, tdt = DT[mode]
    S, H = 6, 4
    F = M + S
    cfg = G.make_config(num_heads=H, image_tokens=M, summary_tokens=S, n_anchor=3, k_window=2,
                        max_frames=8, dtype=gdt)
    stack = G.GcaStack(cfg)
    q, kx, v = draw_frames(StreamSpec(H=H, D=64, M=M, S=S, dtype=tdt, seed=9, chunk=8), 0, 0, B)
    tab = rotary_table(5, B, F, S)
    qr = go.rotary(to64(q).reshape(B * F, H, 64), tab.double().numpy().reshape(B * F, 32, 2))
    kr = go.rotary(to64(kx).reshape(B * F, H, 64), tab.double().numpy().reshape(B * F, 32, 2))
    o_ref, l_ref = go.frame_attention(qr.reshape(B, F, H, 64), kr.reshape(B, F, H, 64), to64(v),
                                      1 / math.sqrt(64))
    tab_d = tab.cuda().reshape(B * F, 32, 2).contiguous()  # must outlive the launches that read it
    G.gca_set_rotary(stack.ctx, tab_d)
    out, lse = stack.frame_attention(q.cuda(), kx.cuda(), v.cuda())
    torch.cuda.synchronize()
    check_outputs(out, o_ref, lse, l_ref, mode, f"frame attention with rotary ({mode})")
    stack.close()
