"""fp64 CPU oracle for the scalar-decay SSD scan (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
this package. The GPU product path never imports it and has no fallback to it.

The arithmetic lives in ``ssd_oracle.c`` (plain recurrence and its
hand-derived adjoint, in IEEE double); this module builds it with gcc and
marshals NumPy arrays. See the header of ``ssd_oracle.c`` for the definition
followed and the passages of the benchmark pages it rests on.

Parity pins: every function here is pinned by CPU tests that do not reuse its
formula (brute-force quadratic form, central finite differences, closed
forms, identities and textbook special cases); see tests/test_oracle_pins.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB = os.path.join(_HERE, "libssd_oracle.so")
_lib = None

_I64 = ctypes.c_int64
_DP = ctypes.POINTER(ctypes.c_double)


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle into a shared library with gcc (IEEE double, OpenMP)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str | None = None):
    """Load the compiled oracle (building it if it is missing)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB
    if not os.path.exists(p) or (path is None and
                                 os.path.getmtime(p) < os.path.getmtime(_SRC)):
        build(out=p)
    lib = ctypes.CDLL(p)
    lib.ssd_oracle_fwd.restype = ctypes.c_int
    lib.ssd_oracle_fwd.argtypes = [_I64] * 6 + [_DP] * 7 + [_I64]
    lib.ssd_oracle_bwd.restype = ctypes.c_int
    lib.ssd_oracle_bwd.argtypes = [_I64] * 6 + [_DP] * 11
    lib.ssd_oracle_num_threads.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_DP)


def _dims(q, v, G):
    B, Gq, T, dk = q.shape
    H, dv = v.shape[1], v.shape[3]
    if Gq != G:
        raise ValueError("q has the wrong group count")
    return B, G, H, T, dk, dv


def fwd(q, k, v, log_alpha, h0, chunk: int = 0, lib=None):
    """y[B,H,T,dv] in float64.  With ``chunk > 0`` also returns the state
    entering every chunk of ``chunk`` steps, layout [B,H,NC,dk,dv]."""
    lib = lib or load()
    q, k, v, la, h0 = map(_f64, (q, k, v, log_alpha, h0))
    B, G, H, T, dk, dv = _dims(q, v, q.shape[1])
    y = np.zeros((B, H, T, dv), np.float64)
    states = None
    if chunk > 0:
        NC = (T + chunk - 1) // chunk
        states = np.zeros((B, H, NC, dk, dv), np.float64)
    rc = lib.ssd_oracle_fwd(B, G, H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(la),
                            _ptr(h0), _ptr(y),
                            _ptr(states) if states is not None else None, chunk)
    if rc != 0:
        raise RuntimeError(f"ssd_oracle_fwd failed ({rc})")
    return (y, states) if chunk > 0 else y


def bwd(q, k, v, log_alpha, h0, dy, lib=None):
    """Gradients of L = sum(dy * y): dict dq, dk, dv, dlog_alpha, dh0 (float64)."""
    lib = lib or load()
    q, k, v, la, h0, dy = map(_f64, (q, k, v, log_alpha, h0, dy))
    B, G, H, T, dk, dv = _dims(q, v, q.shape[1])
    out = {
        "dq": np.zeros(q.shape, np.float64),
        "dk": np.zeros(k.shape, np.float64),
        "dv": np.zeros(v.shape, np.float64),
        "dlog_alpha": np.zeros(la.shape, np.float64),
        "dh0": np.zeros(h0.shape, np.float64),
    }
    rc = lib.ssd_oracle_bwd(B, G, H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(la),
                            _ptr(h0), _ptr(dy), _ptr(out["dq"]), _ptr(out["dk"]),
                            _ptr(out["dv"]), _ptr(out["dlog_alpha"]), _ptr(out["dh0"]))
    if rc != 0:
        raise RuntimeError(f"ssd_oracle_bwd failed ({rc})")
    return out


def num_threads(lib=None) -> int:
    lib = lib or load()
    return int(lib.ssd_oracle_num_threads())
