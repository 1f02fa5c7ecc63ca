"""ctypes binding of libsvgear.so (C ABI in include/svgear.h).

Argument marshalling only: torch tensors are passed as raw device pointers on the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsvgear.so")

OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_WORKSPACE, E_RHO, E_HIP, E_ARG, E_RANGE = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
F32, BF16 = 0, 1
LABELS_GIVEN, DEBUG_EPS, DEBUG_SYNC, PROBE_LOGIT, PROBE_SCORE = 1, 2, 4, 8, 16

EXPORTS = ("svgear_workspace_bytes", "svgear_cluster", "svgear_probe", "svgear_probe_noalloc", "svgear_route",
           "svgear_route_rows", "svgear_attention", "svgear_forward", "svgear_status_string", "svgear_version")

NOALLOC_SCRATCH_BYTES = 64 << 20   # svgear_probe_noalloc's per-device scratch array


class Shape(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("Nq", ctypes.c_int32), ("Nk", ctypes.c_int32),
                ("d", ctypes.c_int32), ("Cq", ctypes.c_int32), ("Ck", ctypes.c_int32),
                ("iters", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_IM_FIELDS = ["labels_q", "qbar", "counts_q", "offsets_q", "perm_q", "inv_perm_q", "Qp",
              "labels_k", "kbar", "vbar", "counts_k", "offsets_k", "perm_k", "inv_perm_k", "Kp",
              "Vp", "log_ratio", "mask", "sel_cost"]


class Intermediates(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in _IM_FIELDS]


class SvgearError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s failed: %s (%d)" % (where, status_string(code), code))


_lib = None


def load():
    """Load libsvgear.so; raises OSError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError("libsvgear.so is not built (run `python -m sparse_attention_video_flash_amd.build`)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_double
        sp = ctypes.POINTER(Shape)
        L.svgear_workspace_bytes.argtypes = [sp, ctypes.POINTER(ctypes.c_size_t)]
        L.svgear_cluster.argtypes = [sp, i32, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                     vp, sz, vp]
        L.svgear_probe.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp]
        L.svgear_probe_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp]
        L.svgear_route.argtypes = [sp, f64, vp, vp, vp, vp, vp, vp, sz, vp]
        L.svgear_route_rows.argtypes = [sp, f64, vp, vp, vp, vp, vp, vp, sz, vp]
        L.svgear_attention.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.svgear_forward.argtypes = [sp, f64, vp, vp, vp, vp, vp, vp, ctypes.POINTER(Intermediates),
                                     i32, vp, sz, vp]
        L.svgear_status_string.argtypes = [i32]
        L.svgear_status_string.restype = ctypes.c_char_p
        L.svgear_version.argtypes = []
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return load().svgear_status_string(int(code)).decode()


def _check(rc: int, where: str):
    if rc != 0:
        raise SvgearError(rc, where)


def make_shape(H, Nq, Nk, d, Cq, Ck, iters=10, dtype=BF16) -> Shape:
    return Shape(int(H), int(Nq), int(Nk), int(d), int(Cq), int(Ck), int(iters), int(dtype))


def workspace_bytes(shape: Shape) -> int:
    n = ctypes.c_size_t(0)
    _check(load().svgear_workspace_bytes(ctypes.byref(shape), ctypes.byref(n)), "svgear_workspace_bytes")
    return int(n.value)


# ----------------------------------------------------------------------------- torch glue

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream=None) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError("svgear supports float32 and bfloat16 tensors, got %s" % t.dtype)


def alloc_workspace(shape: Shape, device="cuda"):
    torch = _torch()
    return torch.empty(workspace_bytes(shape), dtype=torch.uint8, device=device)


def cluster(shape: Shape, side: int, X, init_idx, out: Dict, ws, V=None, flags=0, stream=None):
    """Run svgear_cluster; ``out`` holds the output tensors (see svgear.h)."""
    rc = load().svgear_cluster(ctypes.byref(shape), int(side), _ptr(X), _ptr(V), _ptr(init_idx), int(flags),
                               _ptr(out["labels"]), _ptr(out["cent"]), _ptr(out.get("vbar")),
                               _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["perm"]),
                               _ptr(out["inv_perm"]), _ptr(out["Xp"]), _ptr(out.get("Vp")),
                               _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "svgear_cluster")


def probe(shape: Shape, qbar, counts_q, Kp, Vp, kbar, vbar, counts_k, offsets_k, log_ratio, ws,
          log_eps2=None, flags=0, stream=None):
    if log_eps2 is not None:
        flags |= DEBUG_EPS
    rc = load().svgear_probe(ctypes.byref(shape), _ptr(qbar), _ptr(counts_q), _ptr(Kp), _ptr(Vp), _ptr(kbar),
                             _ptr(vbar), _ptr(counts_k), _ptr(offsets_k), int(flags), _ptr(log_ratio),
                             _ptr(log_eps2), _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "svgear_probe")


def probe_noalloc(shape: Shape, qbar, counts_q, Kp, Vp, kbar, vbar, counts_k, offsets_k, log_ratio,
                  log_eps2=None, flags=0, stream=None):
    """svgear_probe without a workspace (the library's per-device scratch array)."""
    if log_eps2 is not None:
        flags |= DEBUG_EPS
    rc = load().svgear_probe_noalloc(ctypes.byref(shape), _ptr(qbar), _ptr(counts_q), _ptr(Kp), _ptr(Vp),
                                     _ptr(kbar), _ptr(vbar), _ptr(counts_k), _ptr(offsets_k), int(flags),
                                     _ptr(log_ratio), _ptr(log_eps2), _stream(stream))
    _check(rc, "svgear_probe_noalloc")



def route(shape: Shape, rho: float, log_ratio, counts_q, counts_k, mask, sel_cost, ws, stream=None):
    rc = load().svgear_route(ctypes.byref(shape), float(rho), _ptr(log_ratio), _ptr(counts_q), _ptr(counts_k),
                             _ptr(mask), _ptr(sel_cost), _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "svgear_route")


def route_rows(shape: Shape, rho: float, log_ratio, counts_q, counts_k, mask, sel_cost, ws, stream=None):
    """Route with one budget per query cluster (same arguments as ``route``)."""
    rc = load().svgear_route_rows(ctypes.byref(shape), float(rho), _ptr(log_ratio), _ptr(counts_q),
                                  _ptr(counts_k), _ptr(mask), _ptr(sel_cost), _ptr(ws), ws.numel(),
                                  _stream(stream))
    _check(rc, "svgear_route_rows")


def attention(shape: Shape, Qp, offsets_q, perm_q, Kp, Vp, kbar, vbar, counts_k, offsets_k, mask, O, ws,
              stream=None):
    rc = load().svgear_attention(ctypes.byref(shape), _ptr(Qp), _ptr(offsets_q), _ptr(perm_q), _ptr(Kp),
                                 _ptr(Vp), _ptr(kbar), _ptr(vbar), _ptr(counts_k), _ptr(offsets_k), _ptr(mask),
                                 _ptr(O), _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "svgear_attention")


def forward(shape: Shape, rho: float, Q, K, V, init_q, init_k, O, ws, intermediates: Optional[Dict] = None,
            stream=None, flags=0):
    im = None
    if intermediates:
        im = Intermediates(**{k: _ptr(v) for k, v in intermediates.items()})
    rc = load().svgear_forward(ctypes.byref(shape), float(rho), _ptr(Q), _ptr(K), _ptr(V), _ptr(init_q),
                               _ptr(init_k), _ptr(O), ctypes.byref(im) if im is not None else None,
                               int(flags), _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "svgear_forward")


def alloc_intermediates(shape: Shape, device="cuda") -> Dict:
    """Device tensors for every intermediate of svgear_forward."""
    torch = _torch()
    H, Nq, Nk, d, Cq, Ck = shape.H, shape.Nq, shape.Nk, shape.d, shape.Cq, shape.Ck
    et = torch.bfloat16 if shape.dtype == BF16 else torch.float32
    i32, f32 = torch.int32, torch.float32
    e = lambda *s, dt=i32: torch.empty(*s, dtype=dt, device=device)  # noqa: E731
    return dict(labels_q=e(H, Nq), qbar=e(H, Cq, d, dt=f32), counts_q=e(H, Cq), offsets_q=e(H, Cq + 1),
                perm_q=e(H, Nq), inv_perm_q=e(H, Nq), Qp=e(H, Nq, d, dt=et),
                labels_k=e(H, Nk), kbar=e(H, Ck, d, dt=f32), vbar=e(H, Ck, d, dt=f32), counts_k=e(H, Ck),
                offsets_k=e(H, Ck + 1), perm_k=e(H, Nk), inv_perm_k=e(H, Nk), Kp=e(H, Nk, d, dt=et),
                Vp=e(H, Nk, d, dt=et), log_ratio=e(H, Cq, Ck, dt=f32), mask=e(H, Cq, Ck, dt=torch.uint8),
                sel_cost=e(H, dt=torch.int64))
