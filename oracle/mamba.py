"""fp64 CPU oracle for the selective (Mamba-style) scan (test infrastructure).

Only the test suite and the benchmark's CPU-baseline leg use this module.
The GPU product path never imports it and has no fallback to it.

The arithmetic lives in ``mamba_oracle.c`` (plain recurrence and its
hand-derived adjoint, in IEEE double); this module builds it with gcc and
marshals NumPy arrays.  The header of ``mamba_oracle.c`` states the
definition followed and the page it rests on (kernel_mamba_cpu.json).

Parity pins: tests/test_mamba_oracle.py checks both functions against a
brute-force closed form, central finite differences, homogeneity identities
and special cases, none of which reuse this formula.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mamba_oracle.c")
_LIB = os.path.join(_HERE, "libmamba_oracle.so")
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
    """Load the compiled oracle (building it if it is missing or stale)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB
    if not os.path.exists(p) or (path is None and os.path.getmtime(p) < os.path.getmtime(_SRC)):
        build(out=p)
    lib = ctypes.CDLL(p)
    lib.mamba_oracle_fwd.restype = ctypes.c_int
    lib.mamba_oracle_fwd.argtypes = [_I64] * 4 + [_DP] * 7
    lib.mamba_oracle_bwd.restype = ctypes.c_int
    lib.mamba_oracle_bwd.argtypes = [_I64] * 4 + [_DP] * 13
    lib.mamba_oracle_num_threads.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_DP)


def _dims(x, A):
    B, L, D = x.shape
    if A.shape[0] != D:
        raise ValueError("A must be [D, N]")
    return B, L, D, A.shape[1]


def fwd(x, delta, A, Bm, Cm, Ds, lib=None):
    """y[B,L,D] in float64."""
    lib = lib or load()
    x, delta, A, Bm, Cm, Ds = map(_f64, (x, delta, A, Bm, Cm, Ds))
    B, L, D, N = _dims(x, A)
    y = np.zeros((B, L, D), np.float64)
    rc = lib.mamba_oracle_fwd(B, L, D, N, _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Ds), _ptr(y))
    if rc != 0:
        raise RuntimeError(f"mamba_oracle_fwd failed ({rc})")
    return y


def bwd(x, delta, A, Bm, Cm, Ds, dy, lib=None):
    """Gradients of L = sum(dy * y): dict dx, ddelta, dA, dB, dC, dD (float64)."""
    lib = lib or load()
    x, delta, A, Bm, Cm, Ds, dy = map(_f64, (x, delta, A, Bm, Cm, Ds, dy))
    B, L, D, N = _dims(x, A)
    out = {"dx": np.zeros(x.shape), "ddelta": np.zeros(x.shape), "dA": np.zeros(A.shape),
           "dB": np.zeros(Bm.shape), "dC": np.zeros(Cm.shape), "dD": np.zeros(Ds.shape)}
    rc = lib.mamba_oracle_bwd(B, L, D, N, _ptr(x), _ptr(delta), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Ds), _ptr(dy),
                              _ptr(out["dx"]), _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dB"]),
                              _ptr(out["dC"]), _ptr(out["dD"]))
    if rc != 0:
        raise RuntimeError(f"mamba_oracle_bwd failed ({rc})")
    return out


def num_threads(lib=None) -> int:
    lib = lib or load()
    return int(lib.mamba_oracle_num_threads())
