"""MI355X (gfx950) chunked scalar-decay SSD scan: Python binding of the C ABI.

The binding marshals arguments only: it checks dtypes, shapes and devices,
allocates outputs and workspace with PyTorch on the inputs' device, and
calls ``ssd_fwd`` / ``ssd_bwd`` of ``libssd_hip.so`` on PyTorch's current
stream.  Every step of the computation runs in the library's HIP kernels.
There is no CPU or PyTorch fallback: if the library is missing this module
raises when it is used.

Layouts (float32, contiguous):
    q, k [B,G,T,dk]   v, dy [B,H,T,dv]   log_alpha [B,H,T]   h0 [B,H,dk,dv]
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["fwd", "bwd", "library", "ShapeArg", "SsdError", "workspace_size",
           "workspace_layout", "kernel_timing", "CHUNK", "bwd_from_fwd"]

CHUNK = 64
_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssd_hip.so")
_lib = None


class SsdError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = library().ssd_strerror(status).decode() if _lib is not None else str(status)
        super().__init__(f"{where}: status {status} ({msg})")
        self.status = status


class ShapeArg(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("G", ctypes.c_int64), ("H", ctypes.c_int64),
                ("T", ctypes.c_int64), ("dk", ctypes.c_int64), ("dv", ctypes.c_int64)]


def library(path: str | None = None):
    """Load libssd_hip.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"HIP library {p} is missing; build it with __graft_entry__.build()")
    lib = ctypes.CDLL(p)
    vp, sz, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64
    sp = ctypes.POINTER(ShapeArg)
    lib.ssd_fwd_workspace_size.argtypes = [sp]
    lib.ssd_fwd_workspace_size.restype = sz
    lib.ssd_bwd_workspace_size.argtypes = [sp]
    lib.ssd_bwd_workspace_size.restype = sz
    lib.ssd_fwd.argtypes = [sp] + [vp] * 6 + [vp, sz, vp]
    lib.ssd_fwd.restype = ctypes.c_int
    lib.ssd_bwd.argtypes = [sp] + [vp] * 11 + [vp, sz, vp]
    lib.ssd_bwd.restype = ctypes.c_int
    lib.ssd_bwd_from_fwd.argtypes = [sp] + [vp] * 11 + [vp, sz, vp]
    lib.ssd_bwd_from_fwd.restype = ctypes.c_int
    lib.ssd_workspace_layout.argtypes = [sp, ctypes.c_int, ctypes.POINTER(sz)]
    lib.ssd_workspace_layout.restype = ctypes.c_int
    lib.ssd_strerror.argtypes = [ctypes.c_int]
    lib.ssd_strerror.restype = ctypes.c_char_p
    lib.ssd_chunk_size.restype = ctypes.c_int
    lib.ssd_kernel_timing_enable.argtypes = [ctypes.c_int]
    lib.ssd_kernel_timing_enable.restype = ctypes.c_int
    lib.ssd_kernel_timing_reset.restype = ctypes.c_int
    lib.ssd_kernel_timing_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                           ctypes.POINTER(i64)]
    lib.ssd_kernel_timing_read.restype = ctypes.c_int
    lib.ssd_kernel_count.restype = ctypes.c_int
    lib.ssd_kernel_name.argtypes = [ctypes.c_int]
    lib.ssd_kernel_name.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _shape_of(q, v) -> ShapeArg:
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be [B,G,T,dk] and v [B,H,T,dv]")
    B, G, T, dk = q.shape
    H, dv = v.shape[1], v.shape[3]
    return ShapeArg(B, G, H, T, dk, dv)


def _check(t, name, shape, device):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device or t.device.type != "cuda":
        raise ValueError(f"{name} must be on {device} (a HIP device)")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def workspace_size(shape: ShapeArg, backward: bool) -> int:
    lib = library()
    n = (lib.ssd_bwd_workspace_size if backward else lib.ssd_fwd_workspace_size)(ctypes.byref(shape))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError(f"unsupported or invalid shape {tuple(getattr(shape, f) for f, _ in ShapeArg._fields_)}")
    return int(n)


def workspace_layout(shape: ShapeArg, backward: bool) -> list:
    lib = library()
    arr = (ctypes.c_size_t * 5)()
    rc = lib.ssd_workspace_layout(ctypes.byref(shape), int(backward), arr)
    if rc != 0:
        raise SsdError(rc, "ssd_workspace_layout")
    return list(arr)


def _workspace(shape, backward, device, workspace):
    import torch
    need = workspace_size(shape, backward)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace too small")
    return workspace, need


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def fwd(q, k, v, log_alpha, h0, *, out=None, workspace=None):
    """y[B,H,T,dv] = SSD scan of (q, k, v, log_alpha, h0), on the current stream."""
    import torch
    lib = library()
    s = _shape_of(q, v)
    dev = q.device
    _check(q, "q", (s.B, s.G, s.T, s.dk), dev)
    _check(k, "k", (s.B, s.G, s.T, s.dk), dev)
    _check(v, "v", (s.B, s.H, s.T, s.dv), dev)
    _check(log_alpha, "log_alpha", (s.B, s.H, s.T), dev)
    _check(h0, "h0", (s.B, s.H, s.dk, s.dv), dev)
    if out is None:
        out = torch.empty((s.B, s.H, s.T, s.dv), dtype=torch.float32, device=dev)
    _check(out, "out", (s.B, s.H, s.T, s.dv), dev)
    ws, need = _workspace(s, False, dev, workspace)
    rc = lib.ssd_fwd(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(h0),
                     _ptr(out), _ptr(ws), ctypes.c_size_t(ws.numel() * ws.element_size()),
                     _stream(dev))
    if rc != 0:
        raise SsdError(rc, "ssd_fwd")
    return out


def bwd(q, k, v, log_alpha, h0, dy, *, out=None, workspace=None):
    """Gradients (dq, dk, dv, dlog_alpha, dh0) of L = sum(dy * y)."""
    return _bwd_call("ssd_bwd", q, k, v, log_alpha, h0, dy, out, workspace)


def bwd_from_fwd(q, k, v, log_alpha, h0, dy, *, workspace, out=None):
    """Like `bwd`, reusing the residuals that `fwd` left in `workspace`.

    `workspace` must be a backward-sized workspace (``workspace_size(shape,
    True)`` bytes) that was passed to `fwd` on the same inputs, with that
    forward enqueued earlier on the current stream."""
    if workspace is None:
        raise ValueError("bwd_from_fwd needs the workspace the forward wrote")
    return _bwd_call("ssd_bwd_from_fwd", q, k, v, log_alpha, h0, dy, out, workspace)


def _bwd_call(fn, q, k, v, log_alpha, h0, dy, out, workspace):
    import torch
    lib = library()
    s = _shape_of(q, v)
    dev = q.device
    _check(q, "q", (s.B, s.G, s.T, s.dk), dev)
    _check(k, "k", (s.B, s.G, s.T, s.dk), dev)
    _check(v, "v", (s.B, s.H, s.T, s.dv), dev)
    _check(log_alpha, "log_alpha", (s.B, s.H, s.T), dev)
    _check(h0, "h0", (s.B, s.H, s.dk, s.dv), dev)
    _check(dy, "dy", (s.B, s.H, s.T, s.dv), dev)
    shapes = [(s.B, s.G, s.T, s.dk), (s.B, s.G, s.T, s.dk), (s.B, s.H, s.T, s.dv),
              (s.B, s.H, s.T), (s.B, s.H, s.dk, s.dv)]
    if out is None:
        out = tuple(torch.empty(sh, dtype=torch.float32, device=dev) for sh in shapes)
    for t, sh, name in zip(out, shapes, ("dq", "dk", "dv", "dlog_alpha", "dh0")):
        _check(t, name, sh, dev)
    ws, need = _workspace(s, True, dev, workspace)
    rc = getattr(lib, fn)(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(h0), _ptr(dy),
                          *[_ptr(t) for t in out], _ptr(ws),
                          ctypes.c_size_t(ws.numel() * ws.element_size()), _stream(dev))
    if rc != 0:
        raise SsdError(rc, fn)
    return out


class kernel_timing:
    """Context manager: per-kernel HIP-event timing of ssd_fwd/ssd_bwd launches.

    ``with kernel_timing() as kt: ...`` then ``kt.results`` maps kernel name
    to (total_ms, launches).  ``kernels`` names the kernels to time (default:
    all); each timed dispatch costs a few microseconds of stream time."""

    def __init__(self, kernels=None):
        self.kernels = kernels

    def __enter__(self):
        lib = library()
        mask = -1
        if self.kernels is not None:
            names = [lib.ssd_kernel_name(i).decode() for i in range(lib.ssd_kernel_count())]
            unknown = set(self.kernels) - set(names)
            if unknown:
                raise ValueError(f"unknown kernels {sorted(unknown)}; known: {names}")
            mask = sum(1 << names.index(n) for n in self.kernels)
        lib.ssd_kernel_timing_reset()
        lib.ssd_kernel_timing_enable(mask)
        self.results = {}
        return self

    def __exit__(self, *exc):
        lib = library()
        lib.ssd_kernel_timing_enable(0)
        for kid in range(lib.ssd_kernel_count()):
            tot = ctypes.c_double()
            cnt = ctypes.c_int64()
            lib.ssd_kernel_timing_read(kid, ctypes.byref(tot), ctypes.byref(cnt))
            self.results[lib.ssd_kernel_name(kid).decode()] = (tot.value, cnt.value)
        return False
