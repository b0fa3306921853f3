"""Intra-frame attention (frame-attention layers): oracle pin on the CPU.

Each frame's tokens attend to all tokens of the same frame and nothing else,
so the oracle must equal torch's scaled-dot-product attention run frame by
frame (a library routine), and frames must not see each other.
"""
import numpy as np
import torch

from oracle import gca_oracle as go


def test_frame_attention_is_per_frame_sdpa():
    rng = np.random.default_rng(3)
    B, F, H, D = 3, 19, 2, 8
    q, k, v = (rng.standard_normal((B, F, H, D)) for _ in range(3))
    scale = 0.41
    o, l = go.frame_attention(q, k, v, scale)
    for b in range(B):
        qt, kt, vt = (torch.from_numpy(x[b]).permute(1, 0, 2) for x in (q, k, v))  # [H, F, D]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
        np.testing.assert_allclose(o[b], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
        lref = torch.logsumexp(qt @ kt.transpose(1, 2) * scale, dim=-1)
        np.testing.assert_allclose(l[b], lref.numpy(), rtol=0, atol=1e-12)


def test_frames_do_not_see_each_other():
    rng = np.random.default_rng(4)
    B, F, H, D = 2, 7, 1, 4
    q, k, v = (rng.standard_normal((B, F, H, D)) for _ in range(3))
    o, _ = go.frame_attention(q, k, v, 0.5)
    k2, v2 = k.copy(), v.copy()
    k2[1] += 5.0
    v2[1] *= -3.0
    o2, _ = go.frame_attention(q, k2, v2, 0.5)
    np.testing.assert_array_equal(o[0], o2[0])
