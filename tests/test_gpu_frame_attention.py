"""GPU parity of intra-frame attention (gca_frame_attention) against the oracle.

Frames of the stream shapes (M = 500 and a ragged M), bf16 and fp32, are
attended within themselves through the C ABI and compared with the fp64
oracle: bf16 calls of up to 4 frames of up to 8 pages (one page per wave
of a workgroup, combined in LDS: a lone frame, ragged and full last pages,
frames with fewer pages than waves, a 7-row frame); longer bf16 calls of up
to 8 pages per frame (the pipelined page loop, each workgroup walking one or
more (frame, head) items in turn; with rotary angles the kernel that holds a
frame in LDS, 64 frames per launch, so 70 frames make a partial second batch); longer bf16 frames (M = 700: 12 pages, through
scratch pages, 8 frames per launch at H = 16; the largest frame, 2048 rows); fp32 (64 frames per launch
at H = 4); and the benchmark's launch, 64 frames of M = 500 at H = 16; the call must leave every layer's cache untouched, so a stream
interleaving frame attention with GCA steps still matches the oracle and its
page state stays bit-exact.
"""
import math

import pytest
import torch

from geometric_context_attention_amd import _lib as G
from geometric_context_attention_amd.synth import StreamSpec, draw_frames
from oracle import gca_oracle as go
from oracle.gca_oracle import GcaShape
from oracle.page_model import PageModel
from tests.gpu_util import check_outputs, check_state, say, to64

pytestmark = pytest.mark.gpu

DT = {"bf16": (G.GCA_BF16, torch.bfloat16), "fp32": (G.GCA_FP32, torch.float32)}


@pytest.mark.parametrize("mode,M,H,B", [("bf16", 500, 16, 3), ("bf16", 181, 4, 5), ("fp32", 58, 2, 4),
                                         ("bf16", 500, 16, 1), ("bf16", 500, 16, 21), ("fp32", 120, 4, 70),
                                         ("bf16", 120, 4, 70), ("bf16", 700, 16, 10), ("bf16", 500, 16, 64),
                                         ("bf16", 181, 4, 2), ("bf16", 58, 2, 4), ("bf16", 506, 16, 1),
                                         ("bf16", 1, 2, 3), ("bf16", 250, 8, 4), ("bf16", 500, 16, 5),
                                         ("bf16", 2042, 2, 3), ("fp32", 2042, 1, 2),
                                         # the pipelined frame loop at one page: 7 rows, a full page
                                         ("bf16", 1, 2, 9), ("bf16", 58, 2, 6), ("bf16", 122, 4, 8),
                                         # several (frame, head) items per workgroup: two full pages,
                                         # three with a ragged last one
                                         ("bf16", 122, 16, 64), ("bf16", 181, 8, 100),
                                         # head counts that do not divide the 256 workgroups, so that
                                         # stepping to a workgroup's next item carries into the frame
                                         ("bf16", 122, 12, 30), ("bf16", 122, 3, 100), ("bf16", 500, 12, 64),
                                         # frames of exactly 8 full pages, walked by persistent workgroups
                                         ("bf16", 506, 4, 70)])
def test_frame_attention_matches_oracle(mode, M, H, B):
    gdt, tdt = DT[mode]
    S = 6
    cfg = G.make_config(num_heads=H, image_tokens=M, summary_tokens=S, n_anchor=3, k_window=4,
                        max_frames=16, dtype=gdt)
    stack = G.GcaStack(cfg)
    spec = StreamSpec(H=H, D=64, M=M, S=S, dtype=tdt, seed=11, chunk=16)
    q, k, v = draw_frames(spec, 0, 0, B)  # [B, F, H, D]
    out, lse = stack.frame_attention(q.cuda(), k.cuda(), v.cuda())
    o_ref, l_ref = go.frame_attention(to64(q), to64(k), to64(v), 1 / math.sqrt(64))
    ma, rel = check_outputs(out, o_ref, lse, l_ref, mode, f"frame attention {mode} M={M} B={B}")
    say(f"  frame attention {mode} M={M} H={H} B={B}: max-abs {ma:.2e} rel {rel:.2e}")
    stack.close()


@pytest.mark.parametrize("M,H,B", [(500, 16, 64), (500, 16, 16), (500, 16, 2), (181, 4, 70)])
def test_frame_attention_without_lse(M, H, B):
    """No LSE buffer (as the benchmark calls it): the outputs are the same
    bits as with one, on every kernel that serves bf16 calls."""
    S = 6
    cfg = G.make_config(num_heads=H, image_tokens=M, summary_tokens=S, n_anchor=3, k_window=4,
                        max_frames=16, dtype=G.GCA_BF16)
    stack = G.GcaStack(cfg)
    spec = StreamSpec(H=H, D=64, M=M, S=S, dtype=torch.bfloat16, seed=13, chunk=16)
    q, k, v = (t.cuda() for t in draw_frames(spec, 0, 0, B))
    with_lse, _ = stack.frame_attention(q, k, v)
    without, lse = stack.frame_attention(q, k, v, want_lse=False)
    assert lse is None
    assert torch.equal(with_lse.view(torch.int16), without.view(torch.int16))
    say(f"  frame attention without LSE M={M} H={H} B={B}: bit-identical")
    stack.close()


def test_frame_attention_between_steps_leaves_the_cache_alone():
    """GCA steps with intra-frame attention calls in between, bf16."""
    M, S, n, k, T, H = 120, 6, 3, 4, 20, 4
    F = M + S
    cfg = G.make_config(num_heads=H, image_tokens=M, summary_tokens=S, n_anchor=n, k_window=k,
                        max_frames=T, dtype=G.GCA_BF16)
    stack = G.GcaStack(cfg)
    spec = StreamSpec(H=H, D=64, M=M, S=S, dtype=torch.bfloat16, seed=2, chunk=16)
    q, kx, v = draw_frames(spec, 0, 0, T)
    shp = GcaShape(M=M, n=n, k=k, S=S)
    scale = 1 / math.sqrt(64)
    o_ref, l_ref = go.stream_online(to64(q), to64(kx), to64(v), shp, scale)
    f_ref, fl_ref = go.frame_attention(to64(q), to64(kx), to64(v), scale)
    qd, kd, vd = q.cuda(), kx.cuda(), v.cuda()
    pm = PageModel(n=n, k=k, F=F, S=S, P=64, num_pages=G.gca_plan(cfg, 0)["pool_pages"], max_frames=T)

    def rows_of(f, rows):
        return kd[f, rows], vd[f, rows]

    stack.anchor_init(0, qd[:n].reshape(n * F, H, 64), kd[:n].reshape(n * F, H, 64),
                      vd[:n].reshape(n * F, H, 64))
    pm.anchor_init()
    for t in range(n, T):
        fo, fl = stack.frame_attention(qd[t:t + 1], kd[t:t + 1], vd[t:t + 1])
        check_outputs(fo[0], f_ref[t], fl[0], fl_ref[t], "bf16", f"frame attention of frame {t}")
        out, lse = stack.step(0, qd[t], kd[t], vd[t])
        pm.step(t)
        check_outputs(out, o_ref[t], lse, l_ref[t], "bf16", f"step {t}")
        check_state(stack, 0, pm, rows_of)
    stack.close()
