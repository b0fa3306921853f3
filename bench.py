"""Benchmark of the GCA step on one MI355X.

One bench step = one whole stream of the direct-mode stack: reset, anchor
initialisation of the 12 layers, then frames n..T-1 streamed one per step
through all 12 layers (M = 500 image + 6 summary tokens, 16 heads, head_dim
64, n = 3 anchors, window k = 64, T = 10000 frames, bf16 in / fp32
accumulate).  Reported value: frames per second of the whole stream.

Inputs are synthetic (seeded N(0,1)) and resident in HBM before timing: each
layer draws a pool of 64 distinct frames and frame t uses entry
(t + 17*layer) mod 64.  The kernels do the same work whatever the values.

The JSON line also carries:
* roofline: the attention kernel (the dominant one) against the dense bf16
  MFMA peak, from HIP events around every 13th attention launch of the timed
  region (algorithmic flop 4 * (M+6) * keys * D * H per launch);
* cpu_baseline: the fp64 CPU oracle timed on a bounded sample of the same
  workload (one layer, a few sampled steps, linear in the key count) and
  extrapolated to the whole stream.

The other stream configurations the step is quoted on, each one line with
its own cpu_baseline (--config N sets the flags):
  1  tiny fp32 stream: 1 layer, 2 heads, M=32+6, n=3, k=4, T=64
  2  one layer at the paper's token shape, k=16, per-frame key offsets
     N(0, 0.5^2), T=10000 (69.5k cached tokens at the end)
  3  the default line above
  4  full causal cache: k >= T, T=2000, 12 layers (1.01M keys at the end)
  5  dense grid: M=999+6, reset and anchor init every 128 frames, 12 layers

Variants of the stream (no cpu_baseline): --keyframe-interval m (frames
between keyframes), --summary-tokens S, --rotary (rotary angles applied to Q
and to K as it is cached), and --workload frame-attention (the intra-frame
layers through gca_frame_attention, --frames-per-call frames per call).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_CLOCK_GHZ = 2.4   # the clock the published peak is quoted at
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3   # MI355X dense fp32 (matrix cores and vector units alike)
PEAK_HBM_GBS = 8000.0
PROFILE_EVERY = 13     # attention launches per timed sample
METRIC = "GCA frames/s (12 layers, M=500,n=3,k=64,T=10k) + % of bf16 MFMA peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1, help="timed streams")
    ap.add_argument("--warmup", type=int, default=1, help="untimed streams before timing")
    ap.add_argument("--config", type=int, choices=[1, 2, 3, 4, 5], default=0,
                    help="preset of one of the five stream configurations (sets the flags below)")
    ap.add_argument("--frames", type=int, default=10000, help="T (frames per stream)")
    ap.add_argument("--layers", type=int, default=12)
    ap.add_argument("--window", type=int, default=64)
    ap.add_argument("--image-tokens", type=int, default=500)
    ap.add_argument("--heads", type=int, default=16)
    ap.add_argument("--dtype", choices=["bf16", "fp32"], default="bf16")
    ap.add_argument("--key-offset-std", type=float, default=0.0,
                    help="std of the per-frame offset added to every key row of a frame")
    ap.add_argument("--pool", type=int, default=64, help="resident input frames per layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (x4) for counter calibration")
    # variants of the stream and the intra-frame layer (not the default line)
    ap.add_argument("--workload", choices=["stream", "frame-attention"], default="stream")
    ap.add_argument("--keyframe-interval", type=int, default=1)
    ap.add_argument("--summary-tokens", type=int, default=6)
    ap.add_argument("--rotary", action="store_true", help="rotary angles on Q and cached K")
    ap.add_argument("--reset-every", type=int, default=0, metavar="R",
                    help="windows of R frames: reset and anchor init at the start of each")
    ap.add_argument("--frames-per-call", type=int, default=16,
                    help="frames per gca_frame_attention call (frame-attention workload)")
    args = ap.parse_args()
    presets = {
        1: dict(layers=1, heads=2, image_tokens=32, window=4, frames=64, dtype="fp32", pool=64),
        2: dict(layers=1, window=16, key_offset_std=0.5),
        3: {},
        4: dict(window=2000, frames=2000),
        5: dict(image_tokens=999, reset_every=128),
    }
    for key, val in presets.get(args.config, {}).items():
        setattr(args, key, val)
    return args


def default_workload(args):
    return (args.workload == "stream" and args.keyframe_interval == 1 and args.summary_tokens == 6
            and not args.rotary and args.reset_every == 0 and args.layers == 12 and args.window == 64
            and args.frames == 10000 and args.image_tokens == 500 and args.heads == 16
            and args.dtype == "bf16" and args.key_offset_std == 0.0)


def config_workload(args):
    """The numbered stream configuration these flags are, or 0."""
    if (args.workload != "stream" or args.keyframe_interval != 1 or args.summary_tokens != 6
            or args.rotary):
        return 0
    shape = (args.layers, args.heads, args.image_tokens, args.window, args.frames, args.dtype,
             args.key_offset_std, args.reset_every)
    return {(1, 2, 32, 4, 64, "fp32", 0.0, 0): 1, (1, 16, 500, 16, 10000, "bf16", 0.5, 0): 2,
            (12, 16, 500, 64, 10000, "bf16", 0.0, 0): 3, (12, 16, 500, 2000, 2000, "bf16", 0.0, 0): 4,
            (12, 16, 999, 64, 10000, "bf16", 0.0, 128): 5}.get(shape, 0)


def copy_calibration(mib):
    """A plain elementwise copy of known size (fp32 x*1): each launch reads
    and writes exactly mib MiB; used to scale FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(4):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read_per_launch": n * 4,
                      "copy_calibration_bytes_written_per_launch": n * 4, "launches": 4}))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the GCA step is built and timed on a single MI355X; "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch
    from geometric_context_attention_amd import _lib as G
    from geometric_context_attention_amd.profiling import read_traffic
    from geometric_context_attention_amd.synth import StreamSpec, draw_frames

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    H, D, M, S, n = args.heads, 64, args.image_tokens, args.summary_tokens, 3
    k, T, Ly = args.window, args.frames, args.layers
    F = M + S
    f32 = args.dtype == "fp32"
    tdt = torch.float32 if f32 else torch.bfloat16
    esz = 4 if f32 else 2
    W = args.reset_every if args.reset_every > 0 else T  # frames per window (state reset between)
    if W <= n or 0 < T % W <= n:
        print("--reset-every: every window must hold more than the 3 anchor frames", file=sys.stderr)
        sys.exit(2)
    cfg = G.make_config(num_layers=Ly, num_heads=H, head_dim=D, image_tokens=M, summary_tokens=S,
                        n_anchor=n, k_window=k, max_frames=W, dtype=G.GCA_FP32 if f32 else G.GCA_BF16,
                        keyframe_interval=args.keyframe_interval)
    if args.workload == "frame-attention":
        return frame_attention_bench(args, cfg, G, torch, dev)
    stack = G.GcaStack(cfg, device=dev)
    L = G.lib()
    ctx = stack.ctx
    log(f"workspace {stack.workspace.numel() / 2**30:.2f} GiB, pool "
        f"{G.gca_plan(cfg, 0)['pool_pages']} pages per layer")

    # resident inputs
    R = args.pool
    pools = []
    for layer in range(Ly):
        spec = StreamSpec(H=H, D=D, M=M, S=S, dtype=tdt, seed=0, chunk=32,
                          key_offset_std=args.key_offset_std)
        q, kk, v = draw_frames(spec, layer, 0, max(R, n), device=dev)
        pools.append((q, kk, v))
    outs = [torch.empty((F, H, D), dtype=tdt, device=dev) for _ in range(Ly)]
    anc_out = torch.empty((n * F, H, D), dtype=tdt, device=dev)
    # per layer, per pool entry: device addresses
    ptrs = []
    for layer in range(Ly):
        q, kk, v = pools[layer]
        fb = F * H * D * esz
        ptrs.append([(ctypes.c_void_p(q.data_ptr() + i * fb), ctypes.c_void_p(kk.data_ptr() + i * fb),
                      ctypes.c_void_p(v.data_ptr() + i * fb)) for i in range(R)])
    optr = [ctypes.c_void_p(o.data_ptr()) for o in outs]
    # rotary angles: a resident table per pool entry (the rotation costs the
    # same whatever the angles) and one for the anchor block
    rot_set = L.gca_set_rotary
    if args.rotary:
        from geometric_context_attention_amd.synth import rotary_table
        tabs = rotary_table(0, R, F, S, D).to(dev)
        tab_anchor = rotary_table(0, n, F, S, D).to(dev).reshape(n * F, D // 2, 2).contiguous()
        tptr = [ctypes.c_void_p(tabs[i].data_ptr()) for i in range(R)]
        aptr = ctypes.c_void_p(tab_anchor.data_ptr())
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    step_fn = L.gca_step
    anchor_fn = L.gca_anchor_init

    def run_stream():
        for w0 in range(0, T, W):
            run_window(w0)

    def run_window(w0):
        rc = L.gca_reset(ctx, sp)
        if rc:
            raise G.GcaError(rc, L.gca_last_error().decode())
        for layer in range(Ly):
            q, kk, v = pools[layer]
            if args.rotary:
                rot_set(ctx, aptr)
            rc = anchor_fn(ctx, layer, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kk.data_ptr()),
                           ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(anc_out.data_ptr()), None, sp)
            if rc:
                raise G.GcaError(rc, L.gca_last_error().decode())
        for t in range(w0 + n, min(w0 + W, T)):
            for layer in range(Ly):
                e = (t + 17 * layer) % R
                qp, kp, vp = ptrs[layer][e]
                if args.rotary:
                    rot_set(ctx, tptr[e])
                rc = step_fn(ctx, layer, qp, kp, vp, optr[layer], None, sp)
                if rc:
                    raise G.GcaError(rc, L.gca_last_error().decode())
            if t % 2000 == 0:
                log(f"  frame {t}")

    for w in range(args.warmup):
        log(f"warmup stream {w + 1}/{args.warmup}")
        run_stream()
    torch.cuda.synchronize()
    # HIP events around every 13th attention launch (13 is prime to the 12
    # layers, so every layer is sampled): events around every launch would
    # slow the stream by about 3 %
    G.gca_profile_enable(ctx, True, every=PROFILE_EVERY)
    log(f"timed: {args.steps} stream(s) of {T} frames x {Ly} layers")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_stream()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    prof = G.gca_profile_read(ctx)
    G.gca_profile_enable(ctx, False)
    frames = args.steps * T
    fps = frames / elapsed
    attn_avg_ms = prof["attn_ms"] / max(prof["attn_launches"], 1)
    # attention launches of the timed steps
    timed_launches = args.steps * Ly * sum(min(W, T - w0) - n for w0 in range(0, T, W))
    achieved = prof["attn_flop"] / (prof["attn_ms"] * 1e-3) / 1e12 if prof["attn_ms"] > 0 else 0.0
    clock = prof["attn_clock_ghz"]
    log(f"{fps:.1f} frames/s; attention {prof['attn_launches']} sampled launches, avg {attn_avg_ms * 1e3:.1f} us, "
        f"{achieved:.1f} TFLOP/s; attention share of wall {attn_avg_ms * timed_launches / 1e3 / elapsed:.2%}; "
        f"shader clock {clock:.2f} GHz")

    phases = phase_summary(prof)
    if phases:
        log(f"phase cycles (workgroup 0 of the sampled launches): {json.dumps(phases)}")

    variant = [f"keyframe interval {args.keyframe_interval}"] if args.keyframe_interval != 1 else []
    variant += [f"S={S}"] if S != 6 else []
    variant += ["rotary Q/K"] if args.rotary else []
    variant += [f"reset every {W} frames"] if W != T else []
    variant += [f"key offset N(0, {args.key_offset_std}^2)"] if args.key_offset_std else []
    variant = [f"{Ly} layers, H={H}, M={M}, k={k}, T={T}, {args.dtype}"] + variant
    cfg_no = config_workload(args)
    peak = PEAK_FP32_TFLOPS if f32 else PEAK_BF16_TFLOPS
    result = {
        "metric": METRIC if default_workload(args) else f"GCA frames/s ({', '.join(variant)})",
        "value": round(fps, 2),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": (f"synthetic (seeded N(0,1)"
                 + (f", per-frame key offset N(0, {args.key_offset_std}^2)" if args.key_offset_std else "")
                 + f", resident pool of {R} frames per layer)"),
        "config": {"workload": f"GCA direct-mode stream: {Ly} layers, H={H}, D={D}, M={M}+{S}, "
                               f"n={n}, k={k}, T={T}, keyframe interval {args.keyframe_interval}, {args.dtype}"
                               + (", rotary Q/K" if args.rotary else "")
                               + (f", per-frame key offset std {args.key_offset_std}" if args.key_offset_std else "")
                               + (f", reset and anchor init every {W} frames" if W != T else ""),
                   "config_number": cfg_no or None,
                   "layers": Ly, "heads": H, "head_dim": D, "image_tokens": M,
                   "summary_tokens": S, "n_anchor": n, "k_window": k, "frames": T},
        "roofline": {
            "bound": "mfma",
            "kernel": "k_attn_f32" if f32 else "k_attn_bf16",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": read_traffic() if (T, Ly, k, M) == (10000, 12, 64, 500) and default_workload(args) else None,
            "avg_launch_us": round(attn_avg_ms * 1e3, 2),
            "launches": timed_launches,
            "sampled_launches": prof["attn_launches"],
            "algorithmic_flop_per_launch": prof["attn_flop"] / max(prof["attn_launches"], 1),
            "algorithmic_kv_bytes_per_launch": prof["attn_kv_bytes"] / max(prof["attn_launches"], 1),
            # the peak assumes 2.4 GHz; the same peak at the clock measured
            # inside the timed launches
            "clock_ghz": round(clock, 3),
            "frac_at_clock": round(achieved / (peak * clock / PEAK_CLOCK_GHZ), 4) if clock > 0 else None,
        },
    }
    if phases:
        result["phase_cycles"] = phases
    stack.close()
    del pools
    torch.cuda.empty_cache()

    if not args.no_cpu_baseline and cfg_no:
        result["cpu_baseline"] = cpu_baseline(args, H, D, M, S, n, k, T, Ly, W, tdt)
    print(json.dumps(result), flush=True)


PHASES = ["args_and_split", "page_list", "first_pages", "mfma_phases", "softmax_phases",
          "barrier_and_copy_waits", "epilogue"]


def phase_summary(prof):
    """Per-launch and per-page phase cycles of a GCA_PHASE_TIMING build (None
    for the default build, whose phase counters stay zero)."""
    pc = prof.get("phase_cycles") or []
    if not any(pc) or prof["attn_launches"] == 0:
        return None
    out = {}
    for g, wave in ((0, "wave0_group_a"), (1, "wave4_group_b")):
        c = pc[8 * g: 8 * g + 8]
        pages = c[7]
        n = prof["attn_launches"]
        out[wave] = {
            "per_launch": {name: round(c[i] / n, 1) for i, name in enumerate(PHASES)},
            "per_page_in_loop": {name: round(c[i] / pages, 1) for i, name in enumerate(PHASES) if 3 <= i <= 5},
            "pages_per_launch": round(pages / n, 2),
        }
    return out


def frame_attention_bench(args, cfg, G, torch, dev):
    """The intra-frame layers: every frame's M+S tokens attend among
    themselves, in each of the layers, gca_frame_attention taking
    --frames-per-call frames per call (1 = streaming, one frame per step)."""
    from geometric_context_attention_amd.profiling import FRAME_TRAFFIC_FILE, read_traffic
    from geometric_context_attention_amd.synth import StreamSpec, draw_frames

    H, D, M, S, Ly, T = cfg.num_heads, cfg.head_dim, cfg.image_tokens, cfg.summary_tokens, cfg.num_layers, args.frames
    F = M + S
    B = args.frames_per_call
    stack = G.GcaStack(cfg, device=dev)
    L = G.lib()
    ctx = stack.ctx
    R = max(args.pool, B)
    f32 = args.dtype == "fp32"
    tdt = torch.float32 if f32 else torch.bfloat16
    pools = []
    for layer in range(Ly):
        spec = StreamSpec(H=H, D=D, M=M, S=S, dtype=tdt, seed=0, chunk=32)
        pools.append(draw_frames(spec, layer, 0, R, device=dev))
    out = torch.empty((B, F, H, D), dtype=tdt, device=dev)
    fb = F * H * D * (4 if f32 else 2)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    fa = L.gca_frame_attention
    calls = [(t, min(B, T - t)) for t in range(0, T, B)]
    if args.rotary:  # one call's frames of angles, resident for the whole run
        from geometric_context_attention_amd.synth import rotary_table
        tab = rotary_table(0, B, F, S, D).to(dev).reshape(B * F, D // 2, 2).contiguous()
        G.gca_set_rotary(ctx, tab)
    # the kernel that runs the calls (see gca_frame_attention): up to 4 bf16
    # frames of <= 8 pages one page per wave, more of them through the
    # pipelined page loop's frame mode (k_attn_bf16<8, true>) or, with rotary
    # angles, k_frame_attn_bf16; longer frames and fp32 over scratch pages
    ppf = -(-F // 64)
    if f32:
        frame_kernel = "k_attn_f32"
    elif ppf > 8:
        frame_kernel = "k_attn_bf16"
    elif B <= 4:
        frame_kernel = "k_frame_wsplit_bf16"
    else:
        frame_kernel = "k_frame_attn_bf16" if args.rotary else "k_attn_bf16 frame mode"
    peak = PEAK_FP32_TFLOPS if f32 else PEAK_BF16_TFLOPS

    def run():
        for t, nb in calls:
            for layer in range(Ly):
                q, kk, v = pools[layer]
                e = (t + 17 * layer) % (R - nb + 1)  # nb consecutive resident frames
                rc = fa(ctx, ctypes.c_void_p(q.data_ptr() + e * fb), ctypes.c_void_p(kk.data_ptr() + e * fb),
                        ctypes.c_void_p(v.data_ptr() + e * fb), ctypes.c_void_p(out.data_ptr()), None, nb, sp)
                if rc:
                    raise G.GcaError(rc, L.gca_last_error().decode())

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    G.gca_profile_enable(ctx, True, every=PROFILE_EVERY)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    prof = G.gca_profile_read(ctx)
    G.gca_profile_enable(ctx, False)
    fps = args.steps * T / elapsed
    achieved = prof["attn_flop"] / (prof["attn_ms"] * 1e-3) / 1e12 if prof["attn_ms"] > 0 else 0.0
    avg_ms = prof["attn_ms"] / max(prof["attn_launches"], 1)
    clock = prof["attn_clock_ghz"]
    log(f"{fps:.1f} frames/s; attention {prof['attn_launches']} sampled launches, avg {avg_ms * 1e3:.1f} us, "
        f"{achieved:.1f} TFLOP/s; shader clock {clock:.2f} GHz")
    phases = phase_summary(prof)
    if phases:
        log(f"phase cycles (workgroup 0 of the sampled launches): {json.dumps(phases)}")
    # Algorithmic bytes: every frame's Q, K and V read once and O written once
    # (no LSE here), i.e. twice the K/V bytes the profile counts.  At
    # head_dim 64 and M+S = 506 that is 253 flop/byte, below the ridge of the
    # bf16 peak over HBM (312.5 flop/byte): the roofline that bounds these
    # layers is HBM, and the MFMA fraction is reported beside it.  (Longer
    # frames, and the fp32 peak, whose ridge is 19.7 flop/byte, are bound by
    # the matrix cores.)
    launches = max(prof["attn_launches"], 1)
    io_bytes = 2.0 * prof["attn_kv_bytes"]
    intensity = prof["attn_flop"] / io_bytes if io_bytes > 0 else 0.0
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    gbs = io_bytes / (prof["attn_ms"] * 1e-3) / 1e9 if prof["attn_ms"] > 0 else 0.0
    hbm_bound = intensity < ridge
    attainable = min(peak, PEAK_HBM_GBS * intensity / 1e3)
    result = {
        "metric": f"intra-frame attention frames/s ({Ly} layers, M={M}+{S}, H={H}) + % of the roofline",
        "value": round(fps, 2),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic (seeded N(0,1), resident pool of frames per layer)",
        "config": {"workload": f"intra-frame attention: {Ly} layers, H={H}, D={D}, M={M}+{S}, T={T} frames, "
                               f"{B} frames per call, {args.dtype}" + (", rotary Q/K" if args.rotary else ""),
                   "frames_per_call": B},
        "roofline": {
            "bound": "hbm" if hbm_bound else "mfma",
            "kernel": frame_kernel,
            "achieved": round(gbs, 1) if hbm_bound else round(achieved, 2),
            "peak": PEAK_HBM_GBS if hbm_bound else peak,
            "unit": "GB/s" if hbm_bound else "TFLOP/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4) if hbm_bound else round(achieved / peak, 4),
            "traffic": (read_traffic(FRAME_TRAFFIC_FILE)
                        if (B, T, Ly, H, M, S) == (64, 2048, 12, 16, 500, 6) and not args.rotary and not f32
                        else None),
            "avg_launch_us": round(avg_ms * 1e3, 2),
            "sampled_launches": prof["attn_launches"],
            "algorithmic_flop_per_launch": prof["attn_flop"] / launches,
            "algorithmic_bytes_per_launch": io_bytes / launches,
            "arithmetic_intensity_flop_per_byte": round(intensity, 1),
            "tflops": round(achieved, 2),
            "frac_of_mfma_peak": round(achieved / peak, 4),
            "frac_of_attainable": round(achieved / attainable, 4) if attainable > 0 else None,
            "clock_ghz": round(clock, 3),
            "frac_at_clock": round(achieved / (peak * clock / PEAK_CLOCK_GHZ), 4) if clock > 0 else None,
        },
    }
    stack.close()
    print(json.dumps(result), flush=True)


def cpu_baseline(args, H, D, M, S, n, k, T, Ly, W, tdt):
    """Time the fp64 oracle on a bounded sample of the workload; extrapolate.

    A stream short enough (the tiny configuration) is timed whole.  Otherwise
    one layer is timed at sampled steps, smallest key count first, until the
    budget is spent; the oracle's step cost is linear in the key count, so
    time(t) = a + b*keys(t) is fitted to the samples and summed over every
    step of the stream (windows of W frames with an anchor block each), times
    the layers.
    """
    import numpy as np
    import torch

    from geometric_context_attention_amd.synth import StreamSpec, draw_frames
    from oracle import gca_oracle as go

    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        pools = threadpool_info()
        threads = max([i.get("num_threads", 1) for i in pools] or [1])
        blas = ", ".join(sorted({f"{i.get('internal_api', '?')} {i.get('version') or ''}".strip()
                                 for i in pools if i.get("user_api") == "blas"})) or blas
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), cpu)
    except OSError:  # pragma: no cover
        pass
    shp = go.GcaShape(M=M, n=n, k=k, S=S)
    F = M + S
    scale = 1 / math.sqrt(D)
    base = {"unit": "frames/s", "cores": int(threads), "kind": "oracle", "cpu": cpu, "blas": blas}
    if T * Ly <= 256:  # the whole stream, every layer
        t0 = time.perf_counter()
        for layer in range(Ly):
            spec = StreamSpec(H=H, D=D, M=M, S=S, dtype=tdt, seed=0, chunk=16,
                              key_offset_std=args.key_offset_std)
            q, kk, v = (x.double().numpy() for x in draw_frames(spec, layer, 0, T))
            go.stream_online(q, kk, v, shp, scale)
        secs = time.perf_counter() - t0
        return dict(base, value=round(T / secs, 6),
                    sample=f"fp64 numpy oracle over the whole stream ({T} frames x {Ly} layer(s), {secs:.2f} s)")
    R = 16
    spec = StreamSpec(H=H, D=D, M=M, S=S, dtype=tdt, seed=0, chunk=16, key_offset_std=args.key_offset_std)
    q, kk, v = (x.double().numpy() for x in draw_frames(spec, 0, 0, R))

    def get_rows(f, rows):
        return kk[f % R][rows], v[f % R][rows]

    samples = []
    budget = args.cpu_seconds
    spent = 0.0
    t_a = time.perf_counter()
    go.anchor_init(q[:n].reshape(n * F, H, D), kk[:n].reshape(n * F, H, D), v[:n].reshape(n * F, H, D), scale)
    anchor_s = time.perf_counter() - t_a
    spent += anchor_s
    def keys_at(t):  # keys visible at step t: anchors, window, itself, older summaries
        w = min(k, t - n)
        return (n + w + 1) * F + S * (t - n - w)

    cand = sorted({min(max(t, n), W - 1) for t in (n + 1, n + k, W // 8, W // 4, W // 2, W - 1)},
                  key=keys_at)
    for t in cand:
        if spent > budget and len(samples) >= 2:
            break
        t0 = time.perf_counter()
        go.step(t, q[t % R], get_rows, shp, scale)
        dt = time.perf_counter() - t0
        spent += dt
        samples.append((keys_at(t), dt, t))
        log(f"cpu oracle step t={t}: {dt:.2f} s")
    keys = np.array([s[0] for s in samples], dtype=float)
    secs = np.array([s[1] for s in samples])
    b, a = np.polyfit(keys, secs, 1) if len(samples) >= 2 else (secs[0] / keys[0], 0.0)
    steps = [t - w0 for w0 in range(0, T, W) for t in range(w0 + n, min(w0 + W, T))]
    windows = len(range(0, T, W))
    all_keys = np.array([keys_at(t) for t in sorted(set(steps))], dtype=float)
    per_t = dict(zip(sorted(set(steps)), a + b * all_keys))
    stream_s = Ly * (windows * anchor_s + float(sum(per_t[t] for t in steps)))
    return dict(base, value=round(T / stream_s, 6),
                sample=(f"fp64 numpy oracle, one layer: anchor init + steps t={[s[2] for s in samples]} "
                        f"({spent:.1f} s); time linear in keys fitted and summed over every step of the "
                        f"stream ({windows} window(s) of {W} frames), x{Ly} layers (extrapolated)"))


if __name__ == "__main__":
    main()
