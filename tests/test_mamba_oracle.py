"""Pins of the selective-scan oracle (CPU only), and the mistakes they catch.

The page (kernel_mamba_cpu.json) prints no values of y or of the gradients,
so every pin is mathematical: the closed form of the scan, central finite
differences, homogeneity identities and special cases (see mamba_pins.py).
"""
import os
import shutil
import tempfile

import numpy as np
import pytest

from oracle import mamba as mo
from mamba_pins import (ARGS, brute_y, call_bwd, call_fwd, f64, fd_grads, max_rel, run_battery,
                        tiny_inputs)
from ssd_workload.mamba import MambaShape, MAMBA_GRID, make_mamba_inputs


def test_byte_counts_match_the_page():
    """kernel_mamba_cpu.json: fwd records give xla_arg_mb 4.27 / 8.28 and
    xla_out_mb 2.0 / 4.0 at batch 4, seq 512, state 16, dim 256 / 512; the
    fwd_bwd records output as many bytes as the arguments (six gradients)."""
    for D, arg_mb, out_mb in ((256, 4.27, 2.0), (512, 8.28, 4.0)):
        inp = make_mamba_inputs(MambaShape(4, 512, D, 16), 0)
        args = sum(inp[k].nbytes for k in ARGS) / 2**20
        assert round(args, 2) == arg_mb
        assert inp["x"].nbytes / 2**20 == out_mb


def test_closed_form():
    inp = tiny_inputs(seed=11)
    assert max_rel(call_fwd(inp), brute_y(*(inp[k] for k in ARGS))) <= 1e-12


def test_closed_form_strong_and_weak_decay():
    for scale in (0.01, 4.0):
        inp = tiny_inputs(seed=5)
        inp["delta"] = inp["delta"] * scale
        assert max_rel(call_fwd(inp), brute_y(*(inp[k] for k in ARGS))) <= 1e-12


def test_gradients_match_finite_differences():
    inp = tiny_inputs(seed=7, shape=MambaShape(2, 6, 2, 3))
    g = call_bwd(inp)
    fd = fd_grads(inp)
    for k in fd:
        assert max_rel(g[k], fd[k]) <= 1e-6, k


def test_zero_A_is_a_running_sum():
    """A = 0: every decay is 1, so h_t = sum_{s<=t} delta_s B_s x_s."""
    inp = tiny_inputs(seed=2)
    inp["A"][:] = 0.0
    u = inp["delta"][..., None] * inp["B"][:, :, None, :] * inp["x"][..., None]   # [B,L,D,N]
    h = np.cumsum(u, axis=1)
    y = np.einsum("bln,bldn->bld", inp["C"], h) + inp["Dskip"] * inp["x"]
    assert max_rel(call_fwd(inp), y) <= 1e-13


def test_zero_delta_leaves_the_skip_term():
    inp = tiny_inputs(seed=4)
    inp["delta"][:] = 0.0
    assert max_rel(call_fwd(inp), inp["Dskip"] * inp["x"]) <= 1e-15


def test_one_step():
    inp = tiny_inputs(seed=6, shape=MambaShape(3, 1, 5, 4))
    cb = np.sum(inp["C"] * inp["B"], axis=-1)   # [B, 1]
    y = inp["delta"] * inp["x"] * cb[..., None] + inp["Dskip"] * inp["x"]
    assert max_rel(call_fwd(inp), y) <= 1e-14


def test_identities_on_a_larger_case():
    inp = f64(make_mamba_inputs(MambaShape(2, 40, 8, 16), 9))
    y = call_fwd(inp)
    g = call_bwd(inp)
    Lval = float(np.sum(inp["dy"] * y))
    skip = float(np.sum(inp["dy"] * inp["Dskip"] * inp["x"]))
    assert np.isclose(np.sum(inp["x"] * g["dx"]), Lval, rtol=1e-10)
    assert np.isclose(np.sum(inp["B"] * g["dB"]), Lval - skip, rtol=1e-10)
    assert np.isclose(np.sum(inp["C"] * g["dC"]), Lval - skip, rtol=1e-10)
    assert np.isclose(np.sum(inp["delta"] * g["ddelta"]) - np.sum(inp["A"] * g["dA"]), Lval - skip, rtol=1e-9)


def test_workload_recipe_is_seeded_and_in_range():
    s = MAMBA_GRID[(256, 512)]
    a, b = make_mamba_inputs(s, 1), make_mamba_inputs(s, 1)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    assert np.all(a["delta"] > 0) and np.all(a["A"] < 0)
    assert a["x"].dtype == np.float32 and a["A"].shape == (256, 16)


def test_battery_passes():
    assert run_battery(mo.load()) == []


SRC = os.path.join(os.path.dirname(mo.__file__), "mamba_oracle.c")

MUTANTS = {
    "dropped_decay": ("h[n] = a * h[n] + dl * Bt[n] * xv;", "h[n] = h[n] + dl * Bt[n] * xv;"),
    "no_delta_on_input": ("h[n] = a * h[n] + dl * Bt[n] * xv;", "h[n] = a * h[n] + Bt[n] * xv;"),
    "A_state_reversed": ("const double a = exp(dl * A[d * N + n]);\n                h[n]",
                         "const double a = exp(dl * A[d * N + (N - 1 - n)]);\n                h[n]"),
    "exclusive_output": ("acc += Ct[n] * h[n];\n            }", "acc += Ct[n] * h[n] * (t > 0);\n            }"),
    "skip_missing": ("y[i] = acc + Ds[d] * xv;", "y[i] = acc;"),
    "adjoint_decay_index": ("exp(delta[(b * L + t + 1) * D + d] * A[d * N + n])", "exp(delta[i] * A[d * N + n])"),
    "dx_missing_delta": ("sx += G[n] * dl * Bt[n];", "sx += G[n] * Bt[n];"),
    "ddelta_sign": ("sdl += G[n] * (A[d * N + n] * a * prev + Bt[n] * xv);",
                    "sdl += G[n] * (-A[d * N + n] * a * prev + Bt[n] * xv);"),
    "dA_uses_current_state": ("dA[d * N + n] += G[n] * dl * a * prev;", "dA[d * N + n] += G[n] * dl * a * hs[t * N + n];"),
    "dB_missing_x": ("dB[(b * L + t) * N + n] += G[n] * dl * xv;", "dB[(b * L + t) * N + n] += G[n] * dl;"),
    "dC_previous_state": ("dC[(b * L + t) * N + n] += g * hs[t * N + n];", "dC[(b * L + t) * N + n] += g * prev;"),
    "dD_missing": ("dD[d] += g * xv;", "dD[d] += g;"),
}


@pytest.fixture(scope="module")
def tmpdir_mod():
    d = tempfile.mkdtemp(prefix="mamba_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def _build_variant(tmp, name, text):
    path = os.path.join(tmp, name + ".c")
    with open(path, "w") as f:
        f.write(text)
    so = os.path.join(tmp, name + ".so")
    mo.build(src=path, out=so)
    return mo.load(so)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmpdir_mod, name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    lib = _build_variant(tmpdir_mod, name, src.replace(old, new))
    assert run_battery(lib), f"mutant {name} passed every pin"
