"""Seeded synthetic inputs for the selective (Mamba-style) scan.

Shared by the tests and the benchmark.  It holds the workload table and the
random-input recipe only: none of the scan's arithmetic lives here.

Shapes follow the configuration block of the benchmark page
``kernel_mamba_cpu.json``: batch 4, state 16, float32, dim D in 256, 512,
1024 and seq L in 512, 2048, 8192.  The page does not state input
distributions; the recipe used here is:

* x      ~ N(0, 1)                          [B, L, D]
* delta  = softplus(-2 + N(0, 1))           [B, L, D]  (positive step sizes)
* A      = -(n + 1) * exp(0.2 N(0, 1))      [D, N]     (negative real, state n)
* B, C   ~ N(0, 1)                          [B, L, N]
* Dskip  ~ N(0, 1)                          [D]
* dy     ~ N(0, 1)                          [B, L, D]  (upstream gradient)

Every array is drawn in float64 from NumPy's PCG64 generator in the order
x, z_delta, z_A, B, C, Dskip, dy and rounded to float32 once.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = ["MambaShape", "MAMBA_GRID", "make_mamba_inputs"]


@dataclass(frozen=True)
class MambaShape:
    B: int
    L: int
    D: int
    N: int

    def __post_init__(self):
        for name in ("B", "L", "D", "N"):
            if getattr(self, name) < 0:
                raise ValueError(f"{name} must be >= 0")


# The page's grid: (dim, seq) at batch 4, state 16.
MAMBA_GRID = {(D, L): MambaShape(4, L, D, 16) for D in (256, 512, 1024) for L in (512, 2048, 8192)}


def _softplus(z: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, z)


def make_mamba_inputs(shape: MambaShape, seed: int) -> dict:
    """float32 arrays x, delta, A, B, C, Dskip, dy for `shape`."""
    rng = np.random.default_rng(seed)
    Bb, L, D, N = shape.B, shape.L, shape.D, shape.N
    x = rng.standard_normal((Bb, L, D))
    zd = rng.standard_normal((Bb, L, D))
    za = rng.standard_normal((D, N))
    Bm = rng.standard_normal((Bb, L, N))
    Cm = rng.standard_normal((Bb, L, N))
    Ds = rng.standard_normal(D)
    dy = rng.standard_normal((Bb, L, D))
    out = {
        "x": x,
        "delta": _softplus(-2.0 + zd),
        "A": -(np.arange(N, dtype=np.float64) + 1.0)[None, :] * np.exp(0.2 * za),
        "B": Bm,
        "C": Cm,
        "Dskip": Ds,
        "dy": dy,
    }
    return {k: np.ascontiguousarray(v.astype(np.float32)) for k, v in out.items()}
