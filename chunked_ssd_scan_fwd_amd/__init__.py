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
           "workspace_layout", "KernelTimer", "CHUNK", "bwd_from_fwd", "WS_REGIONS", "fwd_noalloc",
           "NOALLOC_WORKSPACE_BYTES"]

CHUNK = 64
WS_REGIONS = 4   # SSD_WS_REGIONS: decay weights, states, dstates, split partial sums
NOALLOC_WORKSPACE_BYTES = 96 << 20   # SSD_NOALLOC_WORKSPACE_BYTES
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
    lib.ssd_fwd_noalloc.argtypes = [sp] + [vp] * 6 + [vp]
    lib.ssd_fwd_noalloc.restype = ctypes.c_int
    lib.ssd_bwd.argtypes = [sp] + [vp] * 11 + [vp, sz, vp]
    lib.ssd_bwd.restype = ctypes.c_int
    lib.ssd_bwd_from_fwd.argtypes = [sp] + [vp] * 11 + [vp, sz, vp]
    lib.ssd_bwd_from_fwd.restype = ctypes.c_int
    lib.ssd_workspace_layout.argtypes = [sp, ctypes.c_int, ctypes.POINTER(sz)]
    lib.ssd_workspace_layout.restype = ctypes.c_int
    lib.ssd_strerror.argtypes = [ctypes.c_int]
    lib.ssd_strerror.restype = ctypes.c_char_p
    lib.ssd_chunk_size.restype = ctypes.c_int
    lib.ssd_fwd_state_stride.argtypes = [sp]
    lib.ssd_fwd_state_stride.restype = ctypes.c_int
    lib.ssd_timer_create.argtypes = [ctypes.c_int]
    lib.ssd_timer_create.restype = vp
    lib.ssd_timer_destroy.argtypes = [vp]
    lib.ssd_timer_destroy.restype = ctypes.c_int
    lib.ssd_timer_reset.argtypes = [vp]
    lib.ssd_timer_reset.restype = ctypes.c_int
    lib.ssd_timer_read.argtypes = [vp, ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    lib.ssd_timer_read.restype = ctypes.c_int
    lib.ssd_fwd_timed.argtypes = [vp, sp] + [vp] * 6 + [vp, sz, vp]
    lib.ssd_fwd_timed.restype = ctypes.c_int
    lib.ssd_bwd_timed.argtypes = [vp, sp] + [vp] * 11 + [vp, sz, vp]
    lib.ssd_bwd_timed.restype = ctypes.c_int
    lib.ssd_kernel_count.restype = ctypes.c_int
    lib.ssd_kernel_name.argtypes = [ctypes.c_int]
    lib.ssd_kernel_name.restype = ctypes.c_char_p
    mp = ctypes.POINTER(MambaShapeArg)
    lib.mamba_fwd_workspace_size.argtypes = [mp]
    lib.mamba_fwd_workspace_size.restype = sz
    lib.mamba_fwd.argtypes = [mp] + [vp] * 7 + [vp, sz, vp]
    lib.mamba_fwd.restype = ctypes.c_int
    lib.mamba_bwd_workspace_size.argtypes = [mp]
    lib.mamba_bwd_workspace_size.restype = sz
    lib.mamba_bwd.argtypes = [mp] + [vp] * 13 + [vp, sz, vp]
    lib.mamba_bwd.restype = ctypes.c_int
    lib.mamba_fwd_bwd.argtypes = [mp] + [vp] * 14 + [vp, sz, vp]
    lib.mamba_fwd_bwd.restype = ctypes.c_int
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
    arr = (ctypes.c_size_t * (WS_REGIONS + 1))()
    rc = lib.ssd_workspace_layout(ctypes.byref(shape), int(backward), arr)
    if rc != 0:
        raise SsdError(rc, "ssd_workspace_layout")
    return list(arr)


def fwd_state_stride(shape: ShapeArg) -> int:
    """1 if ssd_fwd leaves the state of every chunk in the workspace, 2 if
    only that of every even chunk (the forward on chunk pairs)."""
    n = library().ssd_fwd_state_stride(ctypes.byref(shape))
    if n < 0:
        raise SsdError(3, "ssd_fwd_state_stride")
    return n


def _workspace(shape, backward, device, workspace):
    """The workspace to pass: a new one, or the caller's after checking that
    it lives on `device` and owns at least the bytes the size query asks for
    (contiguous, counted from its own start to the end of its storage)."""
    return _workspace_bytes(workspace_size(shape, backward), device, workspace)


def _workspace_bytes(need, device, workspace):
    import torch
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
        return workspace, need
    if not isinstance(workspace, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if workspace.device != device or workspace.device.type != "cuda":
        raise ValueError(f"workspace must be on {device} (a HIP device), got {workspace.device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    nbytes = workspace.numel() * workspace.element_size()
    room = workspace.untyped_storage().nbytes() - workspace.storage_offset() * workspace.element_size()
    if min(nbytes, room) < need:
        raise ValueError(f"workspace too small: {min(nbytes, room)} bytes, {need} needed")
    return workspace, need


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def fwd(q, k, v, log_alpha, h0, *, out=None, workspace=None, timer=None):
    """y[B,H,T,dv] = SSD scan of (q, k, v, log_alpha, h0), on the current stream.
    With a `KernelTimer`, its kernels are timed (ssd_fwd_timed)."""
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
    args = (ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(h0),
            _ptr(out), _ptr(ws), ctypes.c_size_t(ws.numel() * ws.element_size()), _stream(dev))
    rc = lib.ssd_fwd(*args) if timer is None else lib.ssd_fwd_timed(timer.handle, *args)
    if rc != 0:
        raise SsdError(rc, "ssd_fwd")
    return out


def fwd_noalloc(q, k, v, log_alpha, h0, *, out=None):
    """`fwd` through ssd_fwd_noalloc: the library takes the workspace from its
    static per-device array (SSD_NOALLOC_WORKSPACE_BYTES), so the C call
    allocates nothing.  Pass `out` to allocate nothing here either.  Calls
    that overlap in time on one GPU share that array and race."""
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
    rc = lib.ssd_fwd_noalloc(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(h0),
                             _ptr(out), _stream(dev))
    if rc != 0:
        raise SsdError(rc, "ssd_fwd_noalloc")
    return out


def bwd(q, k, v, log_alpha, h0, dy, *, out=None, workspace=None, timer=None):
    """Gradients (dq, dk, dv, dlog_alpha, dh0) of L = sum(dy * y).
    With a `KernelTimer`, its kernels are timed (ssd_bwd_timed)."""
    if timer is not None:
        return _bwd_call("ssd_bwd_timed", q, k, v, log_alpha, h0, dy, out, workspace, timer)
    return _bwd_call("ssd_bwd", q, k, v, log_alpha, h0, dy, out, workspace)


def bwd_from_fwd(q, k, v, log_alpha, h0, dy, *, workspace, out=None):
    """Like `bwd`, reusing the residuals that `fwd` left in `workspace`.

    `workspace` must be a backward-sized workspace (``workspace_size(shape,
    True)`` bytes) that was passed to `fwd` on the same inputs, with that
    forward enqueued earlier on the current stream."""
    if workspace is None:
        raise ValueError("bwd_from_fwd needs the workspace the forward wrote")
    return _bwd_call("ssd_bwd_from_fwd", q, k, v, log_alpha, h0, dy, out, workspace)


def _bwd_call(fn, q, k, v, log_alpha, h0, dy, out, workspace, timer=None):
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
    pre = () if timer is None else (timer.handle,)
    rc = getattr(lib, fn)(*pre, ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(h0), _ptr(dy),
                          *[_ptr(t) for t in out], _ptr(ws),
                          ctypes.c_size_t(ws.numel() * ws.element_size()), _stream(dev))
    if rc != 0:
        raise SsdError(rc, fn)
    return out


class KernelTimer:
    """A caller-owned per-kernel timer (ssd_timer_create): pass it to `fwd` /
    `bwd` as ``timer=``; ``results()`` maps kernel name to (total_ms,
    launches) since the last ``reset()``.  ``kernels`` names the kernels to
    time (default: all); each timed dispatch costs a few microseconds of
    stream time."""

    def __init__(self, kernels=None):
        lib = library()
        names = [lib.ssd_kernel_name(i).decode() for i in range(lib.ssd_kernel_count())]
        mask = -1
        if kernels is not None:
            unknown = set(kernels) - set(names)
            if unknown:
                raise ValueError(f"unknown kernels {sorted(unknown)}; known: {names}")
            mask = sum(1 << names.index(n) for n in kernels)
        self.names = names
        self.handle = ctypes.c_void_p(lib.ssd_timer_create(mask))
        if not self.handle.value:
            raise MemoryError("ssd_timer_create failed")

    def reset(self):
        library().ssd_timer_reset(self.handle)

    def results(self) -> dict:
        lib = library()
        out = {}
        for kid, name in enumerate(self.names):
            tot = ctypes.c_double()
            cnt = ctypes.c_int64()
            rc = lib.ssd_timer_read(self.handle, kid, ctypes.byref(tot), ctypes.byref(cnt))
            if rc != 0:
                raise SsdError(rc, "ssd_timer_read")
            out[name] = (tot.value, cnt.value)
        return out

    def close(self):
        if self.handle is not None and self.handle.value:
            library().ssd_timer_destroy(self.handle)
        self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
        return False


# ---- selective (Mamba-style) scan


class MambaShapeArg(ctypes.Structure):
    """mamba_shape of ssd.h: batch B, sequence L, channels D, states N."""
    _fields_ = [(n, ctypes.c_int64) for n in ("B", "L", "D", "N")]


def mamba_workspace_size(shape: MambaShapeArg, backward: bool = False) -> int:
    lib = library()
    return int((lib.mamba_bwd_workspace_size if backward else lib.mamba_fwd_workspace_size)(ctypes.byref(shape)))


def mamba_fwd(x, delta, A, B, C, Dskip, *, out=None, workspace=None):
    """y[B,L,D] = selective scan of (x, delta, A, B, C, Dskip) (mamba_fwd),
    on the current stream."""
    import torch
    lib = library()
    if x.dim() != 3 or A.dim() != 2:
        raise ValueError("x must be [B,L,D] and A [D,N]")
    s = MambaShapeArg(x.shape[0], x.shape[1], x.shape[2], A.shape[1])
    dev = x.device
    _check(x, "x", (s.B, s.L, s.D), dev)
    _check(delta, "delta", (s.B, s.L, s.D), dev)
    _check(A, "A", (s.D, s.N), dev)
    _check(B, "B", (s.B, s.L, s.N), dev)
    _check(C, "C", (s.B, s.L, s.N), dev)
    _check(Dskip, "Dskip", (s.D,), dev)
    if out is None:
        out = torch.empty((s.B, s.L, s.D), dtype=torch.float32, device=dev)
    _check(out, "out", (s.B, s.L, s.D), dev)
    ws, need = _workspace_bytes(mamba_workspace_size(s), dev, workspace)
    rc = lib.mamba_fwd(ctypes.byref(s), _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip), _ptr(out),
                       _ptr(ws), ctypes.c_size_t(ws.numel() * ws.element_size()), _stream(dev))
    if rc != 0:
        raise SsdError(rc, "mamba_fwd")
    return out


def _mamba_grads(name, x, delta, A, B, C, Dskip, dy, out, workspace, with_y):
    import torch
    lib = library()
    if x.dim() != 3 or A.dim() != 2:
        raise ValueError("x must be [B,L,D] and A [D,N]")
    s = MambaShapeArg(x.shape[0], x.shape[1], x.shape[2], A.shape[1])
    dev = x.device
    shapes = {"x": (s.B, s.L, s.D), "delta": (s.B, s.L, s.D), "A": (s.D, s.N), "B": (s.B, s.L, s.N),
              "C": (s.B, s.L, s.N), "Dskip": (s.D,), "dy": (s.B, s.L, s.D)}
    for nm, t in zip(shapes, (x, delta, A, B, C, Dskip, dy)):
        _check(t, nm, shapes[nm], dev)
    outs = (("y",) if with_y else ()) + ("dx", "ddelta", "dA", "dB", "dC", "dDskip")
    oshape = ([shapes["x"]] if with_y else []) + [shapes["x"], shapes["x"], shapes["A"], shapes["B"], shapes["C"],
                                                   shapes["Dskip"]]
    if out is None:
        out = tuple(torch.empty(sh, dtype=torch.float32, device=dev) for sh in oshape)
    if len(out) != len(outs):
        raise ValueError(f"out must hold {len(outs)} tensors: {', '.join(outs)}")
    for nm, t, sh in zip(outs, out, oshape):
        _check(t, nm, sh, dev)
    ws, need = _workspace_bytes(mamba_workspace_size(s, True), dev, workspace)
    rc = getattr(lib, name)(ctypes.byref(s), _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(Dskip), _ptr(dy),
                            *[_ptr(t) for t in out], _ptr(ws), ctypes.c_size_t(ws.numel() * ws.element_size()),
                            _stream(dev))
    if rc != 0:
        raise SsdError(rc, name)
    return tuple(out)


def mamba_bwd(x, delta, A, B, C, Dskip, dy, *, out=None, workspace=None):
    """(dx, ddelta, dA, dB, dC, dDskip): the gradients of sum(dy * y) for the
    selective scan (mamba_bwd), on the current stream."""
    return _mamba_grads("mamba_bwd", x, delta, A, B, C, Dskip, dy, out, workspace, False)


def mamba_fwd_bwd(x, delta, A, B, C, Dskip, dy, *, out=None, workspace=None):
    """(y, dx, ddelta, dA, dB, dC, dDskip) in one call (mamba_fwd_bwd), on the
    current stream; the workspace is the backward's."""
    return _mamba_grads("mamba_fwd_bwd", x, delta, A, B, C, Dskip, dy, out, workspace, True)
