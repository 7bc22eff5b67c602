"""Independent checks ("pins") for the fp64 oracle.

None of these re-types the oracle's recurrence or adjoint.  They use:

* the quadratic (attention-like) closed form of the scan, with every decay
  factor formed as a direct sum of log-decays (no running state, no cumsum);
* the closed form of the state itself;
* central finite differences of the loss L = sum(dy * y);
* identities that follow from homogeneity and from the invariance of the
  closed form under q_t -> e^{B_t} q_t, k_s -> e^{-B_s} k_s;
* textbook special cases (causal linear attention, Toeplitz decay).

``run_battery(lib)`` runs a small fast subset and returns the names of the
checks that fail; the mutation tests use it on deliberately broken copies of
the oracle.
"""
from __future__ import annotations

import numpy as np

import oracle
from ssd_workload import Shape, make_inputs


def f64(x):
    return {k: np.asarray(v, np.float64) for k, v in x.items()}


def decay(la_bh, s, t):
    """exp of the direct sum la[s+1] + ... + la[t] (empty sum -> 1)."""
    return np.exp(np.sum(la_bh[s + 1:t + 1]))


def brute_y(q, k, v, la, h0):
    """y_t = sum_{s<=t} exp(sum_{r=s+1..t} la_r) (q_t . k_s) v_s + exp(sum_{r<=t} la_r) h0^T q_t."""
    B, G, T, dk = q.shape
    H, dv = v.shape[1], v.shape[3]
    hpg = H // G
    y = np.zeros((B, H, T, dv))
    for b in range(B):
        for h in range(H):
            g = h // hpg
            for t in range(T):
                acc = np.zeros(dv)
                for s in range(t + 1):
                    acc += decay(la[b, h], s, t) * float(q[b, g, t] @ k[b, g, s]) * v[b, h, s]
                acc += np.exp(np.sum(la[b, h, :t + 1])) * (h0[b, h].T @ q[b, g, t])
                y[b, h, t] = acc
    return y


def brute_state(q, k, v, la, h0, t):
    """Closed form of the state after step t, for every (b, h): [B,H,dk,dv]."""
    B, G, T, dk = q.shape
    H, dv = v.shape[1], v.shape[3]
    hpg = H // G
    S = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            g = h // hpg
            acc = np.exp(np.sum(la[b, h, :t + 1])) * h0[b, h]
            for s in range(t + 1):
                acc = acc + decay(la[b, h], s, t) * np.outer(k[b, g, s], v[b, h, s])
            S[b, h] = acc
    return S


def loss(x, lib=None):
    y = oracle.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], lib=lib)
    return float(np.sum(np.asarray(x["dy"], np.float64) * y))


def fd_grads(x, eps=1e-6, lib=None):
    """Central finite differences of L = sum(dy * y) for every input element."""
    x = f64(x)
    out = {}
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"),
                        ("log_alpha", "dlog_alpha"), ("h0", "dh0")):
        base = x[name]
        g = np.zeros_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = dict(x)
            xm = dict(x)
            p = base.copy()
            m = base.copy()
            p[idx] += eps
            m[idx] -= eps
            xp[name] = p
            xm[name] = m
            g[idx] = (loss(xp, lib) - loss(xm, lib)) / (2 * eps)
        out[gname] = g
    return out


def max_rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = max(float(np.max(np.abs(b))), 1e-300)
    return float(np.max(np.abs(a - b))) / den


def tiny_inputs(seed=3, shape=Shape(2, 2, 4, 9, 3, 2), mu=-0.5):
    x = make_inputs(shape, seed, mu=mu, qk_scale=1.0)
    return f64(x)


def run_battery(lib) -> list:
    """Fast subset of the pins; returns the list of failing check names."""
    fails = []
    x = tiny_inputs(seed=11, shape=Shape(1, 2, 4, 6, 3, 2))
    y = oracle.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], lib=lib)
    if max_rel(y, brute_y(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])) > 1e-12:
        fails.append("brute_y")
    g = oracle.bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], x["dy"], lib=lib)
    fd = fd_grads(x, lib=lib)
    for name in fd:
        if max_rel(g[name], fd[name]) > 1e-6:
            fails.append("fd_" + name)
    return fails
