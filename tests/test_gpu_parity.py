"""GPU parity of the HIP library against the CPU oracle, small and medium shapes.

Every case draws seeded inputs once (geometric_context_attention_amd.synth),
hands the same bits to libgca.so (through the C ABI) and to the fp64 oracle,
and compares outputs element by element and cache state bit for bit.
"""
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

DT = {"bf16": (G.GCA_BF16, torch.bfloat16), "fp32": (G.GCA_FP32, torch.float32)}


def _run_stream(mode, M, n, k, T, H, S=6, seed=0, layers=1, max_splits=0, q_scale=1.0,
                state_every=1, check_bytes=True, key_offset_std=0.0, interval=1, chosen=None,
                pool_pages=0, k_boost=()):
    """Stream T frames through every layer; compare each step with the oracle."""
    gdt, tdt = DT[mode]
    F = M + S
    cfg = G.make_config(num_layers=layers, num_heads=H, image_tokens=M, summary_tokens=S,
                        n_anchor=n, k_window=k, max_frames=T, dtype=gdt, max_splits=max_splits,
                        keyframe_interval=interval, pool_pages=pool_pages)
    stack = G.GcaStack(cfg)
    shp = GcaShape(M=M, n=n, k=k, S=S, m=interval, kf=chosen)
    scale = 1 / math.sqrt(64)
    results = []
    for layer in range(layers):
        spec = StreamSpec(H=H, D=64, M=M, S=S, dtype=tdt, seed=seed, chunk=16,
                          key_offset_std=key_offset_std)
        q, kx, v = draw_frames(spec, layer, 0, T)  # CPU generator: [T, F, H, D]
        if q_scale != 1.0:
            q = (q.float() * q_scale).to(tdt)
        for f, r, h, fac in k_boost:  # powers of two: exact in either dtype
            kx[f, r, h] = (kx[f, r, h].float() * fac).to(tdt)
        o_ref, l_ref = go.stream_online(to64(q), to64(kx), to64(v), shp, scale)
        qd, kd, vd = q.cuda(), kx.cuda(), v.cuda()
        pm = PageModel(n=n, k=k, F=F, S=S, P=64, num_pages=G.gca_plan(cfg, 0)["pool_pages"],
                       max_frames=T, m=interval, keyframes=chosen)

        def rows_of(f, rows):
            return kd[f, rows], vd[f, rows]

        out, lse = stack.anchor_init(layer, qd[:n].reshape(n * F, H, 64), kd[:n].reshape(n * F, H, 64),
                                     vd[:n].reshape(n * F, H, 64))
        pm.anchor_init()
        check_outputs(out.reshape(n, F, H, 64), o_ref[:n], lse.reshape(H, n, F).permute(1, 0, 2),
                      l_ref[:n], mode, f"anchor init layer {layer}")
        check_state(stack, layer, pm, rows_of if check_bytes else None)
        worst = 0.0
        for t in range(n, T):
            out, lse = stack.step(layer, qd[t], kd[t], vd[t],
                                  append=None if chosen is None else t in chosen)
            pm.step(t)
            ma, _ = check_outputs(out, o_ref[t], lse, l_ref[t], mode, f"layer {layer} step {t}")
            worst = max(worst, ma)
            if (t - n) % state_every == 0 or t == T - 1:
                check_state(stack, layer, pm, rows_of if check_bytes else None)
        results.append(worst)
        say(f"  {mode} M={M} n={n} k={k} T={T} H={H} m={interval} layer {layer}: worst max-abs {worst:.2e}")
    stack.close()
    return results


def test_tiny_fp32_stream_full_state():
    """1 layer, 2 heads, D=64, fp32, M=32 (+6), n=3, k=4, T=64: every step."""
    _run_stream("fp32", M=32, n=3, k=4, T=64, H=2)


def test_fp32_paper_frame_shape():
    """fp32 on the matrix cores at M = 500 + 6: two 256-row query blocks per
    step, six in the anchor block, a ragged last page (58 rows), 16 heads."""
    _run_stream("fp32", M=500, n=3, k=4, T=14, H=16, state_every=3)


def test_tiny_fp32_single_split():
    _run_stream("fp32", M=32, n=3, k=4, T=40, H=2, max_splits=1, state_every=8)


def test_bf16_ragged_pages_multi_split():
    """F = 106: two pages per frame, the second holding 42 rows."""
    _run_stream("bf16", M=100, n=3, k=5, T=40, H=4, state_every=3)


def test_bf16_two_query_blocks_and_two_layers():
    """F = 606: two 512-row query blocks, 10 pages per frame; two layers."""
    _run_stream("bf16", M=600, n=2, k=3, T=12, H=2, layers=2, state_every=2)


def test_bf16_no_window_and_camera_token_only():
    """k = 0 (every frame is evicted right after its step) and S = 1."""
    _run_stream("bf16", M=40, n=1, k=0, T=30, H=3, S=1, state_every=5)


def test_bf16_window_covers_stream():
    """k >= T: no eviction, frame-block causal attention."""
    _run_stream("bf16", M=70, n=2, k=50, T=25, H=2, state_every=6)


@pytest.mark.parametrize("M,n,k,T,H", [
    (2042, 1, 2, 6, 2),    # the largest frame: 2048 rows, 32 pages, four 512-row query blocks
    (122, 2, 3, 16, 2),    # frames end on a page boundary (two full pages)
    (1, 3, 2, 12, 2),      # 7-row frames
    (100, 2, 3, 12, 32),   # 32 heads: fewer key splits per head
])
def test_bf16_edge_shapes(M, n, k, T, H):
    """Frame sizes and head counts at the edges of what the library accepts."""
    _run_stream("bf16", M=M, n=n, k=k, T=T, H=H, state_every=1)


def test_bf16_sharpened_queries():
    """Q scaled by 4 makes the softmax peaked (|O| ~ 1), so the max-abs gate bites."""
    _run_stream("bf16", M=120, n=3, k=4, T=24, H=2, q_scale=4.0, state_every=8, check_bytes=False)


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
def test_outlier_keys_raise_the_max(mode):
    """A few key rows scaled by 64 score up to ~200 (natural units) above
    the rest: on the pages that hold them the exponentials at the running
    max overflow, and the max has to be raised mid-split.  One of them is a
    summary row, so it stays in trajectory memory after its frame leaves
    the window."""
    boost = ((4, 2, 0, 64.0), (9, 70, 1, 64.0), (15, 33, 0, 64.0), (19, 5, 1, 64.0))
    _run_stream(mode, M=120, n=3, k=4, T=24, H=2, k_boost=boost, state_every=8, check_bytes=False)


def test_fp32_correlated_keys():
    """Per-frame key offsets N(0, 0.5^2) correlate the scores within a frame."""
    _run_stream("fp32", M=60, n=3, k=2, T=20, H=2, key_offset_std=0.5, state_every=5)


def test_split_count_invariance():
    """One key split against the automatic count: same result to fp32 rounding."""
    H, M, n, k, T = 2, 120, 3, 4, 30
    F = M + 6
    spec = StreamSpec(H=H, D=64, M=M, dtype=torch.float32, seed=5, chunk=16)
    q, kx, v = (t.cuda() for t in draw_frames(spec, 0, 0, T))
    outs = []
    for ms in (1, 0):
        cfg = G.make_config(num_heads=H, image_tokens=M, n_anchor=n, k_window=k, max_frames=T,
                            dtype=G.GCA_FP32, max_splits=ms)
        st = G.GcaStack(cfg)
        o, _ = st.anchor_init(0, q[:n].reshape(n * F, H, 64), kx[:n].reshape(n * F, H, 64),
                              v[:n].reshape(n * F, H, 64))
        res = [o]
        for t in range(n, T):
            o, _ = st.step(0, q[t], kx[t], v[t])
            res.append(o)
        outs.append(torch.cat([r.reshape(-1) for r in res]))
        st.close()
    assert G.gca_plan(G.make_config(num_heads=H, image_tokens=M, n_anchor=n, k_window=k,
                                    max_frames=T, dtype=G.GCA_FP32), T - 1)["splits"] > 1
    assert (outs[0] - outs[1]).abs().max().item() <= 2e-6


def test_reset_midstream_then_reanchor():
    """Reset in the middle of a stream; the second stream matches the oracle."""
    H, M, n, k, T = 2, 50, 3, 3, 20
    F = M + 6
    cfg = G.make_config(num_heads=H, image_tokens=M, n_anchor=n, k_window=k, max_frames=T,
                        dtype=G.GCA_FP32)
    st = G.GcaStack(cfg)
    spec = StreamSpec(H=H, D=64, M=M, dtype=torch.float32, seed=9, chunk=16)
    q, kx, v = draw_frames(spec, 0, 0, T)
    qd, kd, vd = q.cuda(), kx.cuda(), v.cuda()
    st.anchor_init(0, qd[:n].reshape(n * F, H, 64), kd[:n].reshape(n * F, H, 64), vd[:n].reshape(n * F, H, 64))
    for t in range(n, 11):
        st.step(0, qd[t], kd[t], vd[t])
    st.reset()
    pm = PageModel(n=n, k=k, F=F, S=6, P=64, num_pages=G.gca_plan(cfg, 0)["pool_pages"], max_frames=T)
    check_state(st, 0, pm)
    # second stream: frames 5.. of the same draw, re-indexed from 0
    q2, k2, v2 = qd[5:], kd[5:], vd[5:]
    T2 = T - 5
    o_ref, l_ref = go.stream_online(to64(q[5:]), to64(kx[5:]), to64(v[5:]), GcaShape(M=M, n=n, k=k), 0.125)
    o, l = st.anchor_init(0, q2[:n].reshape(n * F, H, 64), k2[:n].reshape(n * F, H, 64), v2[:n].reshape(n * F, H, 64))
    pm.anchor_init()
    check_outputs(o.reshape(n, F, H, 64), o_ref[:n], None, None, "fp32", "re-anchor")
    for t in range(n, T2):
        o, l = st.step(0, q2[t], k2[t], v2[t])
        pm.step(t)
        check_outputs(o, o_ref[t], l, l_ref[t], "fp32", f"restream step {t}")
    check_state(st, 0, pm, lambda f, rows: (k2[f, rows], v2[f, rows]))
    st.close()


def test_error_paths():
    H, M = 2, 32
    F = M + 6
    cfg = G.make_config(num_heads=H, image_tokens=M, n_anchor=3, k_window=4, max_frames=6,
                        dtype=G.GCA_FP32)
    st = G.GcaStack(cfg)
    x = torch.randn(3 * F, H, 64, device="cuda")
    f1 = torch.randn(F, H, 64, device="cuda")
    out = torch.empty_like(f1)
    with pytest.raises(G.GcaError) as e:
        G.gca_step(st.ctx, 0, f1, f1, f1, out)
    assert e.value.code == G.GCA_E_BAD_STATE
    with pytest.raises(G.GcaError) as e:
        G.gca_step(st.ctx, 1, f1, f1, f1, out)
    assert e.value.code == G.GCA_E_INVALID_ARG
    with pytest.raises(G.GcaError) as e:
        G._check(G.lib().gca_step(st.ctx, 0, None, None, None, None, None, None))
    assert e.value.code == G.GCA_E_INVALID_ARG
    st.anchor_init(0, x, x, x)
    with pytest.raises(G.GcaError) as e:
        st.anchor_init(0, x, x, x)
    assert e.value.code == G.GCA_E_BAD_STATE
    for _ in range(3):
        st.step(0, f1, f1, f1)
    with pytest.raises(G.GcaError) as e:  # frame 6 == max_frames
        st.step(0, f1, f1, f1)
    assert e.value.code == G.GCA_E_OUT_OF_PAGES
    st.close()
    # a pool too small for the stream: refused on the host, state unchanged
    cfg = G.make_config(num_heads=H, image_tokens=M, n_anchor=3, k_window=4, max_frames=40,
                        dtype=G.GCA_FP32, pool_pages=5)
    st = G.GcaStack(cfg)
    st.anchor_init(0, x, x, x)
    st.step(0, f1, f1, f1)
    st.step(0, f1, f1, f1)
    pm = PageModel(n=3, k=4, F=F, S=6, P=64, num_pages=5, max_frames=40)
    pm.anchor_init(); pm.step(3); pm.step(4)
    with pytest.raises(G.GcaError) as e:
        st.step(0, f1, f1, f1)
    assert e.value.code == G.GCA_E_OUT_OF_PAGES
    check_state(st, 0, pm)
    st.close()
    # wrong shapes / dtypes are refused by the binding before any call
    cfg = G.make_config(num_heads=H, image_tokens=M, n_anchor=3, k_window=4, max_frames=10,
                        dtype=G.GCA_BF16)
    st = G.GcaStack(cfg)
    with pytest.raises(ValueError):
        st.anchor_init(0, x, x, x)  # fp32 tensors for a bf16 context
    st.close()


def test_fp32_keyframe_interval_full_state():
    """Keyframe interval 3 (non-keyframes attended, not cached), fp32, state every step."""
    _run_stream("fp32", M=32, n=3, k=4, T=48, H=2, interval=3)


def test_bf16_keyframe_interval_ragged():
    """Keyframe interval 2 with ragged frames and several splits, bf16."""
    _run_stream("bf16", M=181, n=2, k=3, T=40, H=4, interval=2, state_every=5)


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
def test_variants_combined(mode):
    """Keyframe interval 2, two summary tokens and a single anchor frame
    together, with ragged frames (M + S = 83), state every step."""
    _run_stream(mode, M=81, n=1, k=3, T=30, H=3, S=2, interval=2, state_every=1)


def test_bf16_many_heads():
    """96 heads: fewer key splits per head than pages, one split for some
    steps, the grid still filling the chip."""
    _run_stream("bf16", M=40, n=2, k=3, T=14, H=96, state_every=4)


def test_bf16_caller_chosen_keyframes():
    """Keyframes chosen per step by the caller (gca_step_keyframe), bf16, state checks."""
    rng = np.random.default_rng(5)
    chosen = frozenset(int(t) for t in range(3, 60) if rng.random() < 0.4)
    _run_stream("bf16", M=120, n=3, k=4, T=60, H=4, chosen=chosen, state_every=3)


def test_caller_caches_more_frames_than_the_schedule():
    """Keyframe interval 4 sizes the pool for one frame in four; with a pool
    large enough the caller may still cache every frame (gca_step_keyframe),
    and the summary list holds them all: state bit-exact, outputs green."""
    chosen = frozenset(range(3, 60))
    _run_stream("bf16", M=40, n=3, k=4, T=60, H=2, interval=4, chosen=chosen, pool_pages=64,
                state_every=4)


def test_corrupted_tables_are_flagged():
    """Failure injection: a frame-table entry overwritten with another in-pool
    page is reported by gca_export_state (the device tables no longer match
    the host's record); an entry outside the pool is masked by attention,
    which flags it on the device.  gca_reset clears both."""
    H, M, n, k, T = 2, 100, 3, 4, 12
    F = M + 6
    cfg = G.make_config(num_heads=H, image_tokens=M, n_anchor=n, k_window=k, max_frames=T,
                        dtype=G.GCA_BF16, max_splits=1)
    st = G.GcaStack(cfg)
    spec = StreamSpec(H=H, D=64, M=M, dtype=torch.bfloat16, seed=3, chunk=16)
    q, kx, v = (t.cuda() for t in draw_frames(spec, 0, 0, T))
    rows = n * F
    st.anchor_init(0, q[:n].reshape(rows, H, 64), kx[:n].reshape(rows, H, 64), v[:n].reshape(rows, H, 64))
    for t in range(n, 6):
        st.step(0, q[t], kx[t], v[t])
    s0 = st.export_state(0)
    assert s0["device_error"] == 0
    ft = s0["frame_table"]
    ppf = s0["pages_per_frame"]
    pool = s0["pool_pages"]
    # entry 1 of anchor frame 1 (not the first page of the split) -> another in-pool page
    idx = ppf + 1
    true_pg = int(ft.reshape(-1)[idx])
    other = (true_pg + 1) % pool
    G.gca_debug_set_table_entry(st.ctx, 0, 0, idx, other)
    s1 = st.export_state(0)
    assert s1["device_error"] == G.GCA_ERR_TABLE_MISMATCH
    assert int(s1["frame_table"].reshape(-1)[idx]) == other
    G.gca_debug_set_table_entry(st.ctx, 0, 0, idx, true_pg)  # restored: consistent again
    assert st.export_state(0)["device_error"] == 0
    # an id outside the pool: the next step masks that page and flags it
    G.gca_debug_set_table_entry(st.ctx, 0, 0, idx, pool + 7)
    out, _ = st.step(0, q[6], kx[6], v[6])
    torch.cuda.synchronize()
    s2 = st.export_state(0)
    assert s2["device_error"] & G.GCA_ERR_PAGE_OUT_OF_POOL
    assert s2["device_error"] & G.GCA_ERR_TABLE_MISMATCH
    # out-of-range indices and unknown tables are refused on the host
    for table, index in ((0, -1), (0, T * ppf), (1, 10 ** 6), (2, 0)):
        with pytest.raises(G.GcaError) as e:
            G.gca_debug_set_table_entry(st.ctx, 0, table, index, 0)
        assert e.value.code == G.GCA_E_INVALID_ARG
    st.reset()
    assert st.export_state(0)["device_error"] == 0
    st.close()


def _swap23(s):
    return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1)


def test_poisoned_padding_slots_change_nothing():
    """The empty slots of partial pages (a frame's last page, the summary tail
    page) are masked: filled with huge finite values before every step, they
    leave every output bit unchanged (their scores are masked before the max,
    and their probability is exactly 0)."""
    H, M, n, k, T = 4, 100, 3, 4, 24
    F = M + 6
    cfg = G.make_config(num_heads=H, image_tokens=M, n_anchor=n, k_window=k, max_frames=T, dtype=G.GCA_BF16)
    clean, dirty = G.GcaStack(cfg), G.GcaStack(cfg)
    spec = StreamSpec(H=H, D=64, M=M, dtype=torch.bfloat16, seed=9, chunk=16)
    q, kx, v = (t.cuda() for t in draw_frames(spec, 0, 0, T))
    rows = n * F
    poison = torch.tensor(1e30, dtype=torch.bfloat16)
    ppf, last_valid = 2, F - 64

    def poison_padding(st):
        kp, vp = st.pools(0)
        s = st.export_state(0)
        pages = [int(p) for p in s["frame_table"][:, ppf - 1] if p >= 0]
        spans = [(p, last_valid) for p in pages]
        ns = s["n_summary_pages"]
        if ns:
            tail_valid = 6 * s["n_traj"] - 64 * (ns - 1)
            spans.append((int(s["summary_pages"][ns - 1]), tail_valid))
        for p, valid in spans:
            if valid >= 64:
                continue
            kp[p, :, valid:, :] = poison
            cols = torch.as_tensor(_swap23(np.arange(valid, 64)), device="cuda")
            vp[p, :, :, cols] = poison
        torch.cuda.synchronize()

    outs = []
    for st in (clean, dirty):
        st.anchor_init(0, q[:n].reshape(rows, H, 64), kx[:n].reshape(rows, H, 64), v[:n].reshape(rows, H, 64))
    for t in range(n, T):
        poison_padding(dirty)
        oc, lc = clean.step(0, q[t], kx[t], v[t])
        od, ld = dirty.step(0, q[t], kx[t], v[t])
        assert torch.equal(oc.view(torch.int16), od.view(torch.int16)), f"step {t}: outputs differ"
        assert torch.equal(lc, ld), f"step {t}: LSE differs"
        outs.append(t)
    assert dirty.export_state(0)["device_error"] == 0
    clean.close()
    dirty.close()


def test_page_order_does_not_change_the_result():
    """Attention over a page list does not depend on the order of its pages:
    two window frames' page-table entries swapped on the device (the same keys,
    walked in another order and cut into other splits) give the output of the
    unshuffled twin to fp32 rounding; swapped back, the stream goes on with
    consistent state."""
    H, M, n, k, T = 2, 100, 3, 6, 16
    F = M + 6
    cfg = G.make_config(num_heads=H, image_tokens=M, n_anchor=n, k_window=k, max_frames=T, dtype=G.GCA_FP32)
    a, b = G.GcaStack(cfg), G.GcaStack(cfg)
    spec = StreamSpec(H=H, D=64, M=M, dtype=torch.float32, seed=10, chunk=16)
    q, kx, v = (t.cuda() for t in draw_frames(spec, 0, 0, T))
    rows = n * F
    for st in (a, b):
        st.anchor_init(0, q[:n].reshape(rows, H, 64), kx[:n].reshape(rows, H, 64), v[:n].reshape(rows, H, 64))
    swapped_steps = 0
    for t in range(n, T):
        s = b.export_state(0)
        ft = s["frame_table"]
        ppf = s["pages_per_frame"]
        # two cached frames in the middle of the window (neither leaves the cache at this step),
        # plus anchor frames 0 and 2
        pairs = [(0, 2)]
        if t - n >= 4:
            pairs.append((t - 3, t - 2))
        for f1, f2 in pairs:
            for j in range(ppf):
                G.gca_debug_set_table_entry(b.ctx, 0, 0, f1 * ppf + j, int(ft[f2, j]))
                G.gca_debug_set_table_entry(b.ctx, 0, 0, f2 * ppf + j, int(ft[f1, j]))
        assert b.export_state(0)["device_error"] == G.GCA_ERR_TABLE_MISMATCH
        oa, la = a.step(0, q[t], kx[t], v[t])
        ob, lb = b.step(0, q[t], kx[t], v[t])
        err = float((oa - ob).abs().max())
        assert err <= 2e-6, f"step {t}: shuffled pages change the output by {err}"
        assert float((la - lb).abs().max()) <= 2e-6
        for f1, f2 in pairs:  # restore the true entries
            for j in range(ppf):
                G.gca_debug_set_table_entry(b.ctx, 0, 0, f1 * ppf + j, int(ft[f1, j]))
                G.gca_debug_set_table_entry(b.ctx, 0, 0, f2 * ppf + j, int(ft[f2, j]))
        assert b.export_state(0)["device_error"] == 0
        swapped_steps += 1
    assert swapped_steps == T - n
    a.close()
    b.close()
