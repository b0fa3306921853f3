"""The profiling hooks (gca_profile_enable / gca_profile_read) on the GPU.

With an interval N, exactly the launches 0, N, 2N, ... after enabling are
timed: the launch count and the summed algorithmic flop must equal what the
planner gives for those steps, the summed time must be positive, and the
clock the sampled workgroups measure must be a plausible shader clock.
"""
import pytest
import torch

from geometric_context_attention_amd import _lib as G
from geometric_context_attention_amd.synth import StreamSpec, draw_frames

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("every", [1, 3, 7])
def test_sampled_launches_and_flop(every):
    M, S, H, n, k, T = 120, 6, 4, 3, 4, 30
    F = M + S
    cfg = G.make_config(num_heads=H, image_tokens=M, summary_tokens=S, n_anchor=n, k_window=k,
                        max_frames=T, dtype=G.GCA_BF16)
    stack = G.GcaStack(cfg)
    q, kx, v = (t.cuda() for t in draw_frames(StreamSpec(H=H, D=64, M=M, S=S, dtype=torch.bfloat16,
                                                         seed=3, chunk=16), 0, 0, T))
    stack.anchor_init(0, q[:n].reshape(n * F, H, 64), kx[:n].reshape(n * F, H, 64),
                      v[:n].reshape(n * F, H, 64))
    G.gca_profile_enable(stack.ctx, True, every=every)
    want_flop = 0.0
    for i, t in enumerate(range(n, T)):
        stack.step(0, q[t], kx[t], v[t])
        if i % every == 0:
            want_flop += 4.0 * F * G.gca_plan(cfg, t)["keys"] * 64 * H
    torch.cuda.synchronize()
    p = G.gca_profile_read(stack.ctx)
    G.gca_profile_enable(stack.ctx, False)
    launches = T - n
    assert p["attn_launches"] == (launches + every - 1) // every
    assert p["attn_flop"] == pytest.approx(want_flop, rel=1e-12)
    assert p["attn_ms"] > 0.0
    assert 0.5 < p["attn_clock_ghz"] < 4.0
    stack.close()


def test_negative_interval_rejected():
    cfg = G.make_config(num_heads=2, image_tokens=32, n_anchor=3, k_window=4, max_frames=8,
                        dtype=G.GCA_BF16)
    stack = G.GcaStack(cfg)
    with pytest.raises(G.GcaError, match="interval"):
        G.gca_profile_enable(stack.ctx, True, every=-2)
    stack.close()
