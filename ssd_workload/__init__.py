"""Seeded synthetic inputs for the chunked scalar-decay SSD scan.

This module is shared by the tests, the benchmark and the smoke check. It
holds the workload table and the random-input recipe only: none of the
scan's arithmetic lives here, so the GPU path and the fp64 oracle stay
independent of each other.

Workload shapes follow the configuration blocks of the benchmark pages
``kernel_ssd_cpu.json`` and ``kernel_ssd_gpu.json`` (``config.configs``,
tuples ``(batch, groups, heads, dk, dv)``, and ``config.seq_lens``). The pages
do not state input distributions; the recipe used here is:

* q, k  ~ N(0, 1) / sqrt(128)        layout [B, G, T, dk]
* v     ~ N(0, 1)                    layout [B, H, T, dv]
* log_alpha = -softplus(mu + N(0,1))  layout [B, H, T], mu = -2 (mu = -4 for
  the 24-head long-memory workload)
* h0    ~ 0.1 * N(0, 1)              layout [B, H, dk, dv]
* dy    ~ N(0, 1)                    layout [B, H, T, dv] (upstream gradient)

Every array is drawn in float64 from NumPy's PCG64 generator in the order
q, k, v, z_la, h0, dy and rounded to float32 once. The GPU path and the
oracle consume the same float32 bits.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

__all__ = ["Shape", "Workload", "WORKLOADS", "PAGE_GRID", "make_inputs", "workload", "rel_err"]


@dataclass(frozen=True)
class Shape:
    B: int
    G: int
    H: int
    T: int
    dk: int
    dv: int

    def __post_init__(self):
        for name in ("B", "G", "H", "T", "dk", "dv"):
            if getattr(self, name) < 0:
                raise ValueError(f"{name} must be >= 0")
        if self.G > 0 and self.H % self.G != 0:
            raise ValueError("H must be a multiple of G")

    @property
    def hpg(self) -> int:
        return self.H // self.G

    # Element counts of each tensor, in the layouts above.
    def numel(self) -> dict:
        B, G, H, T, dk, dv = self.B, self.G, self.H, self.T, self.dk, self.dv
        return {
            "q": B * G * T * dk,
            "k": B * G * T * dk,
            "v": B * H * T * dv,
            "log_alpha": B * H * T,
            "h0": B * H * dk * dv,
            "y": B * H * T * dv,
        }


@dataclass(frozen=True)
class Workload:
    name: str
    shape: Shape
    mu: float = -2.0
    seed: int = 0
    note: str = ""


# The five workloads the project is measured on. Seeds are 1000 + index.
WORKLOADS = [
    Workload("g1h1_d128_T512", Shape(4, 1, 1, 512, 128, 128), -2.0, 1000),
    Workload("g2h4_dk48_dv40_T2048", Shape(4, 2, 4, 2048, 48, 40), -2.0, 1001),
    Workload("g2h8_d128_T2048", Shape(4, 2, 8, 2048, 128, 128), -2.0, 1002),
    Workload("g1h24_dk128_dv64_T8192", Shape(2, 1, 24, 8192, 128, 64), -4.0, 1003),
    Workload("g2h8_d128_T8192", Shape(4, 2, 8, 8192, 128, 128), -2.0, 1004,
             note="headline throughput point"),
]

# The benchmark pages' own grid: 4 shapes x T in {512, 2048, 8192}.
_PAGE_SHAPES = {
    "g2h8_d128": (4, 2, 8, 128, 128),
    "g1h24_dk128_dv64": (2, 1, 24, 128, 64),
    "g1h1_d128": (4, 1, 1, 128, 128),
    "g2h4_dk48_dv40": (4, 2, 4, 48, 40),
}
PAGE_GRID = {
    (name, T): Shape(b, g, h, T, dk, dv)
    for name, (b, g, h, dk, dv) in _PAGE_SHAPES.items()
    for T in (512, 2048, 8192)
}


def workload(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def make_inputs(shape: Shape, seed: int, mu: float = -2.0,
                qk_scale: float = 1.0 / math.sqrt(128.0),
                with_dy: bool = True) -> dict:
    """Draw one seeded set of float32 inputs (and the upstream gradient dy).

    Returns a dict of C-contiguous float32 NumPy arrays keyed
    q, k, v, log_alpha, h0 and (if ``with_dy``) dy.
    """
    s = shape
    rng = np.random.default_rng(seed)

    def draw(*dims):
        return rng.standard_normal(dims, dtype=np.float64)

    q = draw(s.B, s.G, s.T, s.dk) * qk_scale
    k = draw(s.B, s.G, s.T, s.dk) * qk_scale
    v = draw(s.B, s.H, s.T, s.dv)
    z_la = draw(s.B, s.H, s.T)
    h0 = 0.1 * draw(s.B, s.H, s.dk, s.dv)
    out = {
        "q": q.astype(np.float32),
        "k": k.astype(np.float32),
        "v": v.astype(np.float32),
        "log_alpha": (-_softplus(mu + z_la)).astype(np.float32),
        "h0": h0.astype(np.float32),
    }
    if with_dy:
        out["dy"] = draw(s.B, s.H, s.T, s.dv).astype(np.float32)
    return out


def rel_err(out, ref) -> float:
    """The benchmark pages' accuracy metric: max|out - ref| / max|ref| over the
    whole tensor (kernel_mamba_cpu.json, config note on rel_err).  When the
    reference is identically zero the denominator falls back to max|out|
    (and the error is 0 when both are zero)."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if out.shape != ref.shape:
        raise ValueError(f"shape mismatch {out.shape} vs {ref.shape}")
    if out.size == 0:
        return 0.0
    num = float(np.max(np.abs(out - ref)))
    den = float(np.max(np.abs(ref)))
    if den == 0.0:
        den = float(np.max(np.abs(out)))
    if den == 0.0:
        return 0.0
    return num / den
