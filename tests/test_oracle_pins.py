"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than its own formula:
a closed form, finite differences, an identity, a textbook special case, a
hand-worked example, or the benchmark pages' printed byte counts.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from ssd_workload import Shape, make_inputs, WORKLOADS, PAGE_GRID
from oracle_pins import (brute_y, brute_state, fd_grads, max_rel, tiny_inputs, f64, loss)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run_fwd(x, **kw):
    return oracle.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], **kw)


def run_bwd(x):
    return oracle.bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], x["dy"])


# (a) quadratic closed form with direct decay sums ----------------------------------

@pytest.mark.parametrize("shape", [Shape(2, 2, 4, 13, 3, 2), Shape(1, 1, 3, 20, 4, 3),
                                   Shape(2, 3, 3, 7, 1, 1)])
def test_forward_matches_quadratic_form(shape):
    x = tiny_inputs(seed=shape.T, shape=shape)
    y = run_fwd(x)
    assert max_rel(y, brute_y(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])) < 1e-13


def test_chunk_states_match_state_closed_form():
    shape = Shape(1, 2, 4, 11, 3, 2)
    x = tiny_inputs(seed=5, shape=shape)
    _, states = run_fwd(x, chunk=4)
    assert states.shape == (1, 4, 3, 3, 2)
    np.testing.assert_array_equal(states[:, :, 0], x["h0"])
    for c in (1, 2):
        ref = brute_state(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], 4 * c - 1)
        assert max_rel(states[:, :, c], ref) < 1e-13


# (b) central finite differences on all five gradients -------------------------------

@pytest.mark.parametrize("shape", [Shape(1, 2, 4, 6, 3, 2), Shape(2, 1, 1, 5, 2, 3)])
def test_gradients_match_finite_differences(shape):
    x = tiny_inputs(seed=7, shape=shape)
    g = run_bwd(x)
    fd = fd_grads(x)
    for name in ("dq", "dk", "dv", "dlog_alpha", "dh0"):
        assert g[name].shape == fd[name].shape
        assert max_rel(g[name], fd[name]) < 1e-7, name


# (c) closed form for dh0 ---------------------------------------------------------------

def test_dh0_closed_form():
    shape = Shape(2, 2, 4, 17, 3, 4)
    x = tiny_inputs(seed=9, shape=shape)
    g = run_bwd(x)
    B, G, H, T = shape.B, shape.G, shape.H, shape.T
    ref = np.zeros_like(g["dh0"])
    for b in range(B):
        for h in range(H):
            gg = h // shape.hpg
            for t in range(T):
                ref[b, h] += np.exp(np.sum(x["log_alpha"][b, h, :t + 1])) * np.outer(
                    x["q"][b, gg, t], x["dy"][b, h, t])
    assert max_rel(g["dh0"], ref) < 1e-13


# (d) homogeneity (Euler) identities ------------------------------------------------

def test_euler_identities():
    shape = Shape(2, 2, 6, 40, 5, 3)
    x = tiny_inputs(seed=13, shape=shape, mu=-1.0)
    y = run_fwd(x)
    g = run_bwd(x)
    L = float(np.sum(x["dy"] * y))
    h0term = float(np.sum(x["h0"] * g["dh0"]))
    assert abs(np.sum(x["q"] * g["dq"]) - L) < 1e-11 * max(1.0, abs(L))
    assert abs(np.sum(x["k"] * g["dk"]) - (L - h0term)) < 1e-11 * max(1.0, abs(L))
    assert abs(np.sum(x["v"] * g["dv"]) - (L - h0term)) < 1e-11 * max(1.0, abs(L))
    per_head = np.sum(x["h0"] * g["dh0"], axis=(2, 3))
    np.testing.assert_allclose(g["dlog_alpha"][:, :, 0], per_head, rtol=1e-11, atol=1e-13)


# (e) log-decay gradient as a suffix sum (one head per group) -------------------------

def test_dlog_alpha_suffix_identity():
    shape = Shape(2, 3, 3, 25, 4, 3)   # G == H: group sums are per-head values
    x = tiny_inputs(seed=17, shape=shape)
    g = run_bwd(x)
    dB = np.sum(x["q"] * g["dq"], axis=-1) - np.sum(x["k"] * g["dk"], axis=-1)
    ref = np.cumsum(dB[:, :, ::-1], axis=-1)[:, :, ::-1]
    assert max_rel(g["dlog_alpha"], ref) < 1e-12


# (f) textbook special cases --------------------------------------------------------

def test_zero_decay_is_causal_linear_attention():
    shape = Shape(2, 2, 4, 16, 5, 3)
    x = tiny_inputs(seed=19, shape=shape)
    x["log_alpha"][:] = 0.0
    x["h0"][:] = 0.0
    y = run_fwd(x)
    g = run_bwd(x)
    ref_y = np.zeros_like(y)
    dq_ref = np.zeros_like(g["dq"])
    dk_ref = np.zeros_like(g["dk"])
    dv_ref = np.zeros_like(g["dv"])
    M = np.tril(np.ones((shape.T, shape.T)))
    for b in range(shape.B):
        for h in range(shape.H):
            gg = h // shape.hpg
            Q, K, V, dY = x["q"][b, gg], x["k"][b, gg], x["v"][b, h], x["dy"][b, h]
            A = M * (Q @ K.T)
            ref_y[b, h] = A @ V
            dP = M * (dY @ V.T)
            dq_ref[b, gg] += dP @ K
            dk_ref[b, gg] += dP.T @ Q
            dv_ref[b, h] = A.T @ dY
    assert max_rel(y, ref_y) < 1e-13
    assert max_rel(g["dq"], dq_ref) < 1e-13
    assert max_rel(g["dk"], dk_ref) < 1e-13
    assert max_rel(g["dv"], dv_ref) < 1e-13


def test_constant_decay_is_toeplitz_retention():
    shape = Shape(1, 1, 2, 21, 4, 3)
    x = tiny_inputs(seed=23, shape=shape)
    c = -0.3
    x["log_alpha"][:] = c
    y = run_fwd(x)
    t = np.arange(shape.T)
    D = np.where(t[:, None] >= t[None, :], np.exp(c * (t[:, None] - t[None, :])), 0.0)
    for h in range(shape.H):
        Q, K, V = x["q"][0, 0], x["k"][0, 0], x["v"][0, h]
        ref = (D * (Q @ K.T)) @ V + np.exp(c * (t + 1))[:, None] * (Q @ x["h0"][0, h])
        assert max_rel(y[0, h], ref) < 1e-13


def test_single_step():
    shape = Shape(2, 1, 2, 1, 3, 4)
    x = tiny_inputs(seed=29, shape=shape)
    y = run_fwd(x)
    for b in range(2):
        for h in range(2):
            a = np.exp(x["log_alpha"][b, h, 0])
            S = a * x["h0"][b, h] + np.outer(x["k"][b, 0, 0], x["v"][b, h, 0])
            np.testing.assert_allclose(y[b, h, 0], S.T @ x["q"][b, 0, 0], rtol=1e-14)


def test_strong_decay_forgets_the_past():
    shape = Shape(1, 1, 1, 12, 3, 2)
    x = tiny_inputs(seed=31, shape=shape)
    x["log_alpha"][:] = -80.0
    x["h0"][:] = 0.0
    y = run_fwd(x)
    ref = np.sum(x["q"][0, 0] * x["k"][0, 0], axis=-1)[:, None] * x["v"][0, 0]
    assert max_rel(y[0, 0], ref) < 1e-15  # e^-80 ~ 1.8e-35: only rounding remains


def test_hand_worked_example():
    d = json.load(open(os.path.join(GOLDEN, "hand_example_T2.json")))
    i, e = d["inputs"], d["expected"]
    x = {
        "q": np.array(i["q"]).reshape(1, 1, 2, 1),
        "k": np.array(i["k"]).reshape(1, 1, 2, 1),
        "v": np.array(i["v"]).reshape(1, 1, 2, 1),
        "log_alpha": np.log(np.array(i["alpha"])).reshape(1, 1, 2),
        "h0": np.array([[[[i["h0"]]]]]),
        "dy": np.array(i["dy"]).reshape(1, 1, 2, 1),
    }
    y = run_fwd(x)
    g = run_bwd(x)
    np.testing.assert_allclose(y.ravel(), e["y"], rtol=1e-14)
    for name in ("dq", "dk", "dv", "dlog_alpha"):
        np.testing.assert_allclose(g[name].ravel(), e[name], rtol=1e-14)
    np.testing.assert_allclose(g["dh0"].ravel(), [e["dh0"]], rtol=1e-14)


# (g) structural --------------------------------------------------------------------

def test_group_replication():
    shape = Shape(2, 2, 6, 15, 3, 2)
    x = tiny_inputs(seed=37, shape=shape)
    y = run_fwd(x)
    g = run_bwd(x)
    rep = dict(x)
    idx = np.arange(shape.H) // shape.hpg
    rep["q"] = x["q"][:, idx]
    rep["k"] = x["k"][:, idx]
    y2 = run_fwd(rep)
    g2 = run_bwd(rep)
    assert max_rel(y2, y) < 1e-15
    for gg in range(shape.G):
        sl = slice(gg * shape.hpg, (gg + 1) * shape.hpg)
        assert max_rel(g2["dq"][:, sl].sum(axis=1), g["dq"][:, gg]) < 1e-14
        assert max_rel(g2["dk"][:, sl].sum(axis=1), g["dk"][:, gg]) < 1e-14
    assert max_rel(g2["dv"], g["dv"]) < 1e-15
    assert max_rel(g2["dlog_alpha"], g["dlog_alpha"]) < 1e-15


def test_linearity_in_v_and_h0():
    x = tiny_inputs(seed=41, shape=Shape(1, 1, 2, 10, 3, 3))
    y = run_fwd(x)
    x2 = dict(x)
    x2["v"] = 2.5 * x["v"]
    x2["h0"] = 2.5 * x["h0"]
    assert max_rel(run_fwd(x2), 2.5 * y) < 1e-14


def test_deterministic_and_thread_independent():
    x = tiny_inputs(seed=43, shape=Shape(3, 2, 4, 70, 6, 5))
    g1 = run_bwd(x)
    g2 = run_bwd(x)
    for name in g1:
        np.testing.assert_array_equal(g1[name], g2[name])


def test_float32_inputs_promote_exactly():
    x32 = make_inputs(Shape(1, 1, 1, 9, 3, 2), 47)
    y_a = run_fwd(x32)
    y_b = run_fwd({k: v.astype(np.float64) for k, v in x32.items()})
    np.testing.assert_array_equal(y_a, y_b)


def test_empty_sequence():
    x = make_inputs(Shape(1, 1, 2, 0, 3, 2), 1)
    y = run_fwd(x)
    g = run_bwd(x)
    assert y.shape == (1, 2, 0, 2)
    np.testing.assert_array_equal(g["dh0"], 0.0)


# layout pin: the pages' argument/output byte counts ----------------------------------

def test_layouts_reproduce_page_byte_counts():
    d = json.load(open(os.path.join(GOLDEN, "page_layout_bytes.json")))
    assert len(d["rows"]) == 24
    MiB = 1024.0 * 1024.0
    for r in d["rows"]:
        s = Shape(r["B"], r["G"], r["H"], r["T"], r["dk"], r["dv"])
        n = s.numel()
        arg = 4 * (n["q"] + n["k"] + n["v"] + n["log_alpha"] + n["h0"]) / MiB
        assert arg == r["xla_arg_mb"], r["record"]
        if r["mode"] == "fwd":
            assert 4 * n["y"] / MiB == r["xla_out_mb"], r["record"]
        else:
            # five gradients with the inputs' shapes, plus 40 bytes of tuple overhead
            assert abs(r["xla_out_mb"] - arg - 40 / MiB) < 1e-9, r["record"]


def test_workload_table_matches_page_grid():
    for w in WORKLOADS:
        name = w.name.rsplit("_T", 1)[0]
        T = int(w.name.rsplit("_T", 1)[1])
        assert PAGE_GRID[(name, T)] == w.shape
