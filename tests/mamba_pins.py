"""Independent checks ("pins") for the selective-scan oracle.

None of these re-types the oracle's recurrence or adjoint.  They use:

* the closed form of the scan, every decay product formed as the
  exponential of a direct sum of delta_r A[d,n] (no running state);
* central finite differences of the loss L = sum(dy * y);
* identities from homogeneity (y is linear in x; its state part is linear
  in B and in C) and from the invariance of every decay under
  delta -> s delta, A -> A / s;
* special cases: A = 0 (a running sum), delta = 0 (the skip term alone),
  one step.

``run_battery(lib)`` runs a fast subset and returns the names of the checks
that fail; the mutation tests use it on deliberately broken copies of the
oracle.
"""
from __future__ import annotations

import numpy as np

from oracle import mamba as mo
from ssd_workload.mamba import MambaShape, make_mamba_inputs

ARGS = ("x", "delta", "A", "B", "C", "Dskip")


def f64(inp):
    return {k: np.asarray(v, np.float64) for k, v in inp.items()}


def brute_y(x, delta, A, Bm, Cm, Ds):
    """y_t[d] = sum_{s<=t} sum_n C_t[n] exp(A[d,n] sum_{r=s+1..t} delta_r[d]) delta_s[d] B_s[n] x_s[d]
    + Ds[d] x_t[d]."""
    Bb, L, D = x.shape
    N = A.shape[1]
    y = np.zeros((Bb, L, D))
    for b in range(Bb):
        for d in range(D):
            for t in range(L):
                acc = 0.0
                for s in range(t + 1):
                    ssum = float(np.sum(delta[b, s + 1:t + 1, d]))
                    for n in range(N):
                        acc += Cm[b, t, n] * np.exp(A[d, n] * ssum) * delta[b, s, d] * Bm[b, s, n] * x[b, s, d]
                y[b, t, d] = acc + Ds[d] * x[b, t, d]
    return y


def call_fwd(inp, lib=None):
    return mo.fwd(*(inp[k] for k in ARGS), lib=lib)


def call_bwd(inp, lib=None):
    return mo.bwd(*(inp[k] for k in ARGS), inp["dy"], lib=lib)


def loss(inp, lib=None):
    return float(np.sum(inp["dy"] * call_fwd(inp, lib)))


GRAD_OF = {"x": "dx", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "Dskip": "dD"}


def fd_grads(inp, eps=1e-6, lib=None):
    """Central differences of L for every element of every argument."""
    out = {}
    for a in ARGS:
        g = np.zeros_like(inp[a])
        it = np.nditer(inp[a], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            p = {k: v.copy() for k, v in inp.items()}
            m = {k: v.copy() for k, v in inp.items()}
            p[a][idx] += eps
            m[a][idx] -= eps
            g[idx] = (loss(p, lib) - loss(m, lib)) / (2 * eps)
        out[GRAD_OF[a]] = g
    return out


def max_rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den)


def tiny_inputs(seed=3, shape=MambaShape(2, 7, 3, 4)):
    """Small inputs with decays spread between ~0.1 and ~1 per step."""
    inp = f64(make_mamba_inputs(shape, seed))
    inp["delta"] = 0.3 + 0.5 * inp["delta"]
    return inp


def run_battery(lib) -> list:
    """Fast checks against `lib`; returns the names of those that fail."""
    bad = []
    inp = tiny_inputs()
    y = call_fwd(inp, lib)
    if max_rel(y, brute_y(*(inp[k] for k in ARGS))) > 1e-12:
        bad.append("closed_form")
    g = call_bwd(inp, lib)
    fd = fd_grads(inp, lib=lib)
    for k in fd:
        if max_rel(g[k], fd[k]) > 1e-6:
            bad.append("fd_" + k)
    Lval = float(np.sum(inp["dy"] * y))
    skip = float(np.sum(inp["dy"] * inp["Dskip"][None, None, :] * inp["x"]))
    if abs(np.sum(inp["x"] * g["dx"]) - Lval) > 1e-10 * max(1.0, abs(Lval)):
        bad.append("homogeneous_x")
    if abs(np.sum(inp["B"] * g["dB"]) - (Lval - skip)) > 1e-10 * max(1.0, abs(Lval)):
        bad.append("homogeneous_B")
    if abs(np.sum(inp["C"] * g["dC"]) - (Lval - skip)) > 1e-10 * max(1.0, abs(Lval)):
        bad.append("homogeneous_C")
    if abs(np.sum(inp["Dskip"] * g["dD"]) - skip) > 1e-10 * max(1.0, abs(skip)):
        bad.append("skip_term")
    if abs(np.sum(inp["delta"] * g["ddelta"]) - np.sum(inp["A"] * g["dA"]) - (Lval - skip)) > \
            1e-10 * max(1.0, abs(Lval)):
        bad.append("delta_A_scaling")
    return bad
