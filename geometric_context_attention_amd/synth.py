"""Seeded synthetic Q/K/V streams for the GCA step.

This module only draws random numbers.  It holds none of the method's
arithmetic and is shared by the parity tests (which hand the same tensors to
the CPU oracle and to the HIP library) and by the benchmark.

Recipe (one stream = one GCA layer):

* Frame f of layer l has F = M + S rows per head; rows 0..S-1 are the
  summary rows, rows S..F-1 the image rows.  Q, K and V are iid N(0, 1).
* Frames are drawn in chunks of ``chunk`` consecutive frames.  Chunk c of
  layer l uses a ``torch.Generator`` on the requested device seeded with
  ``seed * 1000003 + l * 7919 + c``; within a chunk the draws are one
  [chunk, 3, F, H, D] normal tensor (q, then k, then v).
* With ``key_offset_std`` > 0, one offset vector per (frame, head) with
  entries N(0, key_offset_std^2) is added to all F key rows of that frame
  (drawn after q/k/v from the same generator), so scores are correlated
  within a frame.
* Values are drawn in float32 and then rounded to the stream dtype (bf16
  rounds to nearest even).  The oracle receives exact float64 upcasts of the
  rounded tensors.

The CPU and CUDA generators produce different numbers for the same seed;
every parity test draws once and hands the same tensors to both sides.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class StreamSpec:
    H: int
    D: int
    M: int
    S: int = 6
    dtype: torch.dtype = torch.bfloat16
    key_offset_std: float = 0.0
    seed: int = 0
    chunk: int = 32

    @property
    def F(self) -> int:
        return self.M + self.S


def chunk_seed(spec: StreamSpec, layer: int, chunk: int) -> int:
    return spec.seed * 1000003 + layer * 7919 + chunk


def draw_chunk(spec: StreamSpec, layer: int, chunk: int, device="cpu"):
    """Q, K, V for frames [chunk*C, (chunk+1)*C), each [C, F, H, D] in spec.dtype."""
    g = torch.Generator(device=device)
    g.manual_seed(chunk_seed(spec, layer, chunk))
    C, F, H, D = spec.chunk, spec.F, spec.H, spec.D
    x = torch.randn((C, 3, F, H, D), generator=g, device=device, dtype=torch.float32)
    q, k, v = x[:, 0], x[:, 1], x[:, 2]
    if spec.key_offset_std > 0:
        off = torch.randn((C, 1, H, D), generator=g, device=device, dtype=torch.float32)
        k = k + spec.key_offset_std * off
    return (q.to(spec.dtype).contiguous(), k.to(spec.dtype).contiguous(),
            v.to(spec.dtype).contiguous())


def draw_frames(spec: StreamSpec, layer: int, first: int, count: int, device="cpu"):
    """Q, K, V for frames [first, first+count), each [count, F, H, D]."""
    qs, ks, vs = [], [], []
    C = spec.chunk
    c0, c1 = first // C, (first + count - 1) // C
    for c in range(c0, c1 + 1):
        q, k, v = draw_chunk(spec, layer, c, device)
        lo = max(first, c * C) - c * C
        hi = min(first + count, (c + 1) * C) - c * C
        qs.append(q[lo:hi]); ks.append(k[lo:hi]); vs.append(v[lo:hi])
    return torch.cat(qs), torch.cat(ks), torch.cat(vs)


def rotary_table(first: int, count: int, F: int, S: int, D: int = 64, grid_w: int = 37,
                 base: float = 10000.0) -> torch.Tensor:
    """Synthetic rotary angles for frames [first, first+count): fp32 [count, F, D/2, 2].

    The pages fix no frequency schedule, so this stand-in for a video (3-axis)
    schedule is an input like the others: channel pair i uses axis i % 3
    (frame time, patch row, patch column) with frequency base^(-(i // 3) / (D/6));
    summary rows sit at patch (0, 0), image row S + p at patch (p // grid_w,
    p % grid_w).  Entry [f, r, i] = (cos, sin) of position * frequency.
    """
    half = D // 2
    i = torch.arange(half, dtype=torch.float64)
    axis = (i % 3).long()
    freq = base ** (-(torch.div(i, 3, rounding_mode="floor")) / (D / 6))
    t = torch.arange(first, first + count, dtype=torch.float64)[:, None].expand(count, F)
    p = torch.clamp(torch.arange(F, dtype=torch.float64) - S, min=-1)
    y = torch.where(p < 0, torch.zeros_like(p), torch.div(p, grid_w, rounding_mode="floor"))
    x = torch.where(p < 0, torch.zeros_like(p), p - y * grid_w)
    pos = torch.stack([t, y[None].expand(count, F), x[None].expand(count, F)], dim=-1)  # [count, F, 3]
    ang = pos[..., axis] * freq  # [count, F, half]
    return torch.stack([torch.cos(ang), torch.sin(ang)], dim=-1).to(torch.float32).contiguous()
