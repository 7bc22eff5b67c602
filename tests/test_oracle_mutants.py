"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a temporary copy of the oracle's C source
(on the CPU), builds it, and checks that the fast pin battery fails.  The
unmodified source must pass the same battery.
"""
import os
import shutil
import tempfile

import pytest

import oracle
from oracle_pins import run_battery

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")

MUTANTS = {
    "dropped_decay": ("row[j] = a * row[j] + ki * vt[j];", "row[j] = row[j] + ki * vt[j];"),
    "wrong_group_map": ("g = h / hpg;\n        double *S = (double *)malloc(sizeof(double) * dk * dv);",
                        "g = h % G;\n        double *S = (double *)malloc(sizeof(double) * dk * dv);"),
    "exclusive_output": ("yt[j] += row[j] * qi;", "yt[j] += row[j] * qi * (t > 0);"),
    "k_instead_of_q": ("const double qi = qt[i];\n                const double *row = S + i * dv;",
                       "const double qi = kt[i];\n                const double *row = S + i * dv;"),
    "adjoint_decay_index": ("exp(lab[t + 1]) : 0.0", "exp(lab[t]) : 0.0"),
    "dk_uses_dy": ("acc += row[j] * vt[j];", "acc += row[j] * dyt[j];"),
    "dv_transposed": ("dvo[j] += row[j] * ki;", "dvo[j] += row[j] * qt[i];"),
    "dla_missing_factor": ("dla[bh * T + t] = exp(lab[t]) * acc;", "dla[bh * T + t] = acc;"),
    "dla_wrong_state": ("seg + (t - 1 - t0) * E", "seg + (t - t0) * E"),
    "dh0_missing_factor": ("dh0[bh * E + e] = a0 * Gb[e];", "dh0[bh * E + e] = Gb[e];"),
    "dq_sign": ("                o[i] = acc;\n            }\n        }\n\n", "                o[i] = -acc;\n            }\n        }\n\n"),
    "group_sum_first_head_only": ("for (int64_t hh = 0; hh < hpg; ++hh)", "for (int64_t hh = 0; hh < 1; ++hh)"),
}


def _build_variant(tmp, name, text):
    path = os.path.join(tmp, name + ".c")
    with open(path, "w") as f:
        f.write(text)
    so = os.path.join(tmp, name + ".so")
    oracle.build(src=path, out=so)
    return oracle.load(so)


@pytest.fixture(scope="module")
def tmpdir_mod():
    d = tempfile.mkdtemp(prefix="oracle_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_unmodified_oracle_passes_battery(tmpdir_mod):
    lib = _build_variant(tmpdir_mod, "orig", open(SRC).read())
    assert run_battery(lib) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmpdir_mod, name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    lib = _build_variant(tmpdir_mod, name, src.replace(old, new))
    assert run_battery(lib), f"mutant {name} passed every pin"
