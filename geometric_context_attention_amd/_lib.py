"""ctypes binding of libgca.so: argument marshalling only.

Every function here has the name of the C entry point it calls (include/gca.h)
and does nothing but check tensor arguments, take their device addresses and
the current HIP stream, and translate error codes into exceptions.  All of the
GCA step runs in the library's kernels; if the library is missing this module
raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

# GCA_LIBRARY names another build of the library in the package directory
# (a compile-time variant of the kernels, see build.py); default libgca.so.
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        os.path.basename(os.environ.get("GCA_LIBRARY", "libgca.so")))

GCA_BF16, GCA_FP32 = 0, 1
GCA_OK = 0
GCA_E_INVALID_ARG = -1
GCA_E_BAD_STATE = -2
GCA_E_OUT_OF_PAGES = -3
GCA_E_HIP = -4
GCA_E_UNSUPPORTED = -5
GCA_ERR_PAGE_OUT_OF_POOL = 1
GCA_ERR_TABLE_MISMATCH = 2

_DTYPES = {GCA_BF16: torch.bfloat16, GCA_FP32: torch.float32}


class gca_config(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("image_tokens", ctypes.c_int32),
                ("summary_tokens", ctypes.c_int32), ("n_anchor", ctypes.c_int32),
                ("k_window", ctypes.c_int32), ("max_frames", ctypes.c_int32),
                ("page_tokens", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("pool_pages", ctypes.c_int32),
                ("max_splits", ctypes.c_int32), ("keyframe_interval", ctypes.c_int32)]


class gca_plan_info(ctypes.Structure):
    _fields_ = [("keys", ctypes.c_int64), ("cached_after", ctypes.c_int64),
                ("pages_visible", ctypes.c_int32), ("used_pages_after", ctypes.c_int32),
                ("pool_pages", ctypes.c_int32), ("pages_per_frame", ctypes.c_int32),
                ("splits", ctypes.c_int32), ("qblocks", ctypes.c_int32),
                ("flop", ctypes.c_double)]


class gca_state_host(ctypes.Structure):
    _fields_ = [("frames_appended", ctypes.c_int32), ("n_traj", ctypes.c_int32),
                ("n_summary_pages", ctypes.c_int32), ("used_pages", ctypes.c_int32),
                ("pool_pages", ctypes.c_int32), ("pages_per_frame", ctypes.c_int32),
                ("max_frames", ctypes.c_int32), ("max_summary_pages", ctypes.c_int32),
                ("device_error", ctypes.c_int32),
                ("used_bitmap", ctypes.POINTER(ctypes.c_uint32)),
                ("frame_table", ctypes.POINTER(ctypes.c_int32)),
                ("summary_pages", ctypes.POINTER(ctypes.c_int32))]


class gca_profile(ctypes.Structure):
    _fields_ = [("attn_ms", ctypes.c_double), ("attn_launches", ctypes.c_int64),
                ("attn_flop", ctypes.c_double), ("attn_kv_bytes", ctypes.c_double),
                ("attn_clock_ghz", ctypes.c_double), ("phase_cycles", ctypes.c_double * 16)]


class GcaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"GCA error {code}: {msg}")
        self.code = code


_lib = None

_VP = ctypes.c_void_p
_I32 = ctypes.c_int32
_SIGS = {
    "gca_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(gca_config)]),
    "gca_create": (ctypes.c_int, [ctypes.POINTER(gca_config), _VP, ctypes.c_size_t, _VP,
                                  ctypes.POINTER(_VP)]),
    "gca_anchor_init": (ctypes.c_int, [_VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP]),
    "gca_step": (ctypes.c_int, [_VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP]),
    "gca_reset": (ctypes.c_int, [_VP, _VP]),
    "gca_destroy": (None, [_VP]),
    "gca_last_error": (ctypes.c_char_p, []),
    "gca_plan": (ctypes.c_int, [ctypes.POINTER(gca_config), _I32, ctypes.POINTER(gca_plan_info)]),
    "gca_export_state": (ctypes.c_int, [_VP, _I32, ctypes.POINTER(gca_state_host), _VP]),
    "gca_pool_views": (ctypes.c_int, [_VP, _I32, ctypes.POINTER(_VP), ctypes.POINTER(_VP),
                                      ctypes.POINTER(ctypes.c_size_t)]),
    "gca_step_keyframe": (ctypes.c_int, [_VP, _I32, _VP, _VP, _VP, _VP, _VP, _I32, _VP]),
    "gca_step_noalloc": (ctypes.c_int, [_VP, _I32, _VP, _VP, _VP, _VP, _VP, _VP]),
    "gca_frame_attention": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP]),
    "gca_set_rotary": (ctypes.c_int, [_VP, _VP]),
    "gca_debug_set_table_entry": (ctypes.c_int, [_VP, _I32, _I32, ctypes.c_int64, _I32, _VP]),
    "gca_profile_enable": (ctypes.c_int, [_VP, _I32]),
    "gca_profile_read": (ctypes.c_int, [_VP, ctypes.POINTER(gca_profile)]),
}


def lib():
    """Load libgca.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return list(_SIGS)


def _check(rc: int):
    if rc != GCA_OK:
        raise GcaError(rc, lib().gca_last_error().decode())


def make_config(*, num_layers=1, num_heads, head_dim=64, image_tokens, summary_tokens=6,
                n_anchor=3, k_window, max_frames, page_tokens=64, dtype=GCA_BF16, scale=0.0,
                pool_pages=0, max_splits=0, keyframe_interval=1) -> gca_config:
    return gca_config(num_layers, num_heads, head_dim, image_tokens, summary_tokens, n_anchor,
                      k_window, max_frames, page_tokens, dtype, scale, pool_pages, max_splits,
                      keyframe_interval)


def _stream_ptr(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t: torch.Tensor | None, dtype=None, shape=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


# ---------------------------------------------------------------- entry points

def gca_workspace_bytes(cfg: gca_config) -> int:
    n = lib().gca_workspace_bytes(ctypes.byref(cfg))
    if n == 0:
        raise GcaError(GCA_E_INVALID_ARG, lib().gca_last_error().decode())
    return n


def gca_create(cfg: gca_config, workspace: torch.Tensor, stream=None):
    ctx = ctypes.c_void_p()
    _check(lib().gca_create(ctypes.byref(cfg), _ptr(workspace, name="workspace"),
                            workspace.numel() * workspace.element_size(), _stream_ptr(stream),
                            ctypes.byref(ctx)))
    return ctx


def gca_anchor_init(ctx, layer, q, k, v, out, lse=None, stream=None):
    _check(lib().gca_anchor_init(ctx, layer, _ptr(q, name="q"), _ptr(k, name="k"),
                                 _ptr(v, name="v"), _ptr(out, name="out"),
                                 _ptr(lse, torch.float32, name="lse"), _stream_ptr(stream)))


def gca_step(ctx, layer, q, k, v, out, lse=None, stream=None):
    _check(lib().gca_step(ctx, layer, _ptr(q, name="q"), _ptr(k, name="k"), _ptr(v, name="v"),
                          _ptr(out, name="out"), _ptr(lse, torch.float32, name="lse"),
                          _stream_ptr(stream)))


def gca_step_keyframe(ctx, layer, q, k, v, out, lse=None, append=True, stream=None):
    _check(lib().gca_step_keyframe(ctx, layer, _ptr(q, name="q"), _ptr(k, name="k"), _ptr(v, name="v"),
                                   _ptr(out, name="out"), _ptr(lse, torch.float32, name="lse"),
                                   1 if append else 0, _stream_ptr(stream)))


def gca_step_noalloc(ctx, layer, q, k, v, out, lse=None, stream=None):
    _check(lib().gca_step_noalloc(ctx, layer, _ptr(q, name="q"), _ptr(k, name="k"), _ptr(v, name="v"),
                                  _ptr(out, name="out"), _ptr(lse, torch.float32, name="lse"),
                                  _stream_ptr(stream)))


def gca_frame_attention(ctx, q, k, v, out, lse=None, frames=1, stream=None):
    _check(lib().gca_frame_attention(ctx, _ptr(q, name="q"), _ptr(k, name="k"), _ptr(v, name="v"),
                                     _ptr(out, name="out"), _ptr(lse, torch.float32, name="lse"),
                                     frames, _stream_ptr(stream)))


def gca_set_rotary(ctx, cos_sin=None):
    """cos_sin: device fp32 tensor [rows, D/2, 2] for the following calls, or None."""
    _check(lib().gca_set_rotary(ctx, _ptr(cos_sin, torch.float32, name="cos_sin")))


def gca_reset(ctx, stream=None):
    _check(lib().gca_reset(ctx, _stream_ptr(stream)))


def gca_destroy(ctx):
    lib().gca_destroy(ctx)


def gca_plan(cfg: gca_config, t: int) -> dict:
    info = gca_plan_info()
    _check(lib().gca_plan(ctypes.byref(cfg), t, ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in gca_plan_info._fields_}


def gca_export_state(ctx, layer, stream=None) -> dict:
    st = gca_state_host()
    _check(lib().gca_export_state(ctx, layer, ctypes.byref(st), _stream_ptr(stream)))
    words = (st.pool_pages + 31) // 32
    bm = np.zeros(words, dtype=np.uint32)
    ft = np.zeros(st.max_frames * st.pages_per_frame, dtype=np.int32)
    sp = np.zeros(st.max_summary_pages, dtype=np.int32)
    st.used_bitmap = bm.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))
    st.frame_table = ft.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    st.summary_pages = sp.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    _check(lib().gca_export_state(ctx, layer, ctypes.byref(st), _stream_ptr(stream)))
    out = {name: getattr(st, name) for name, _ in gca_state_host._fields_[:9]}
    out["used_bitmap"] = bm
    out["frame_table"] = ft.reshape(st.max_frames, st.pages_per_frame)
    out["summary_pages"] = sp
    return out


def gca_debug_set_table_entry(ctx, layer, table, index, value, stream=None):
    """Failure injection: overwrite one device frame-table (table 0) or
    summary-list (table 1) entry."""
    _check(lib().gca_debug_set_table_entry(ctx, layer, table, index, value, _stream_ptr(stream)))


def gca_pool_views(ctx, layer):
    kp, vp, nb = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_size_t()
    _check(lib().gca_pool_views(ctx, layer, ctypes.byref(kp), ctypes.byref(vp), ctypes.byref(nb)))
    return kp.value, vp.value, nb.value


def gca_profile_enable(ctx, on, every: int = 1):
    """Time every `every`-th attention launch with HIP events (on=True), or stop (on=False)."""
    _check(lib().gca_profile_enable(ctx, int(every) if on else 0))


def gca_profile_read(ctx) -> dict:
    p = gca_profile()
    _check(lib().gca_profile_read(ctx, ctypes.byref(p)))
    out = {name: getattr(p, name) for name, _ in gca_profile._fields_}
    out["phase_cycles"] = list(p.phase_cycles)
    return out


# ---------------------------------------------------------------- convenience

class GcaStack:
    """A context plus its workspace (a torch device allocation)."""

    def __init__(self, cfg: gca_config, device="cuda", stream=None):
        self.cfg = cfg
        self.dtype = _DTYPES[cfg.dtype]
        nbytes = gca_workspace_bytes(cfg)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.ctx = gca_create(cfg, self.workspace, stream)
        self.F = cfg.image_tokens + cfg.summary_tokens

    def close(self):
        if self.ctx is not None:
            gca_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _outputs(self, rows, like, want_lse):
        out = torch.empty((rows, self.cfg.num_heads, self.cfg.head_dim), dtype=self.dtype,
                          device=like.device)
        lse = (torch.empty((self.cfg.num_heads, rows), dtype=torch.float32, device=like.device)
               if want_lse else None)
        return out, lse

    def anchor_init(self, layer, q, k, v, want_lse=True, stream=None):
        rows = self.cfg.n_anchor * self.F
        shape = (rows, self.cfg.num_heads, self.cfg.head_dim)
        for name, t in (("q", q), ("k", k), ("v", v)):
            _ptr(t, self.dtype, shape, name)
        out, lse = self._outputs(rows, q, want_lse)
        gca_anchor_init(self.ctx, layer, q, k, v, out, lse, stream)
        return out, lse

    def step(self, layer, q, k, v, want_lse=True, out=None, lse=None, stream=None, append=None):
        """One step; append=None follows the keyframe schedule, True/False decides."""
        shape = (self.F, self.cfg.num_heads, self.cfg.head_dim)
        for name, t in (("q", q), ("k", k), ("v", v)):
            _ptr(t, self.dtype, shape, name)
        if out is None:
            out, lse = self._outputs(self.F, q, want_lse)
        if append is None:
            gca_step(self.ctx, layer, q, k, v, out, lse, stream)
        else:
            gca_step_keyframe(self.ctx, layer, q, k, v, out, lse, append, stream)
        return out, lse

    def frame_attention(self, q, k, v, want_lse=True, stream=None):
        """Intra-frame attention of q, k, v [frames, M+S, H, D]."""
        B = q.shape[0]
        shape = (B, self.F, self.cfg.num_heads, self.cfg.head_dim)
        for name, t in (("q", q), ("k", k), ("v", v)):
            _ptr(t, self.dtype, shape, name)
        out = torch.empty(shape, dtype=self.dtype, device=q.device)
        lse = (torch.empty((B, self.cfg.num_heads, self.F), dtype=torch.float32, device=q.device)
               if want_lse else None)
        gca_frame_attention(self.ctx, q, k, v, out, lse, B, stream)
        return out, lse

    def reset(self, stream=None):
        gca_reset(self.ctx, stream)

    def export_state(self, layer, stream=None):
        return gca_export_state(self.ctx, layer, stream)

    def pools(self, layer):
        """(K pool, V pool) as typed views of the workspace: [pages, H, P, D] / [pages, H, D, P]."""
        kp, vp, nb = gca_pool_views(self.ctx, layer)
        st = self.export_state(layer)
        base = self.workspace.data_ptr()
        H, D, P = self.cfg.num_heads, self.cfg.head_dim, self.cfg.page_tokens
        es = torch.tensor([], dtype=self.dtype).element_size()
        npg = st["pool_pages"]
        kv = self.workspace[kp - base: kp - base + npg * nb].view(self.dtype).view(npg, H, P, D)
        vv = self.workspace[vp - base: vp - base + npg * nb].view(self.dtype).view(npg, H, D, P)
        assert nb == H * P * D * es
        return kv, vv
