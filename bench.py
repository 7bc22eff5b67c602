"""Benchmark of the chunked SSD scan on one MI355X.

One step = ssd_fwd followed by ssd_bwd (y and all five gradients) on the
headline workload g2h8_d128: B=4, G=2, H=8, T=8192, dk=dv=128, float32,
seeded synthetic inputs resident in HBM.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
    python bench.py --copy-mib N      # plain device copy of N MiB, 5 times: the
                                      # reference kernel for scaling HBM counters
    python bench.py --max-len         # T-doubling search: the longest sequence whose
                                      # fwd_bwd fits in HBM at g2h8_d128, B=4
    python bench.py --grid            # fwd and fwd_bwd at every shape of the pages'
                                      # grid (4 shapes x T in 512, 2048, 8192), one
                                      # JSON line per shape

Throughput (`value`) is the nominal fwd+bwd FLOP count of the step divided
by the measured step time.  Nominal FLOPs per (token, head), with chunk
length C = 64 and causal tiles counted as half:
    forward  C(dk+dv) + 4 dk dv
    backward C(3dk+2dv) + 10 dk dv   (includes recomputing the chunk states)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSD fwd & fwd_bwd ms + TFLOP/s (% roofline), g2h8_d128 B=4 T=8192 fp32"
PEAK_FP32_MFMA = 157.3e12   # MI355X dense fp32 matrix, FLOP/s
PEAK_HBM = 8.0e12           # MI355X HBM3E, B/s
C_NOM = 64
# The benchmark pages' JAX "chunked" fwd_bwd at this workload on an RTX 3090
# (kernel_ssd_gpu.json, record chunked·fwd_bwd·g2h8_d128·T8192, median_ms).
PAGE_FWD_BWD_MS = 11.883384999237023
# kernel_mamba_cpu.json, results: the CPU medians (ms) of impls scan and
# chunked at batch 4, state 16, modes fwd and fwd_bwd -- context for --mamba,
# not a target.
MAMBA_PAGE_CPU_MS = {
    (256, 512): {"scan": 17.20, "chunked": 6.40}, (256, 2048): {"scan": 28.61, "chunked": 21.79},
    (256, 8192): {"scan": 120.3, "chunked": 107.4}, (512, 512): {"scan": 14.21, "chunked": 14.48},
    (512, 2048): {"scan": 56.86, "chunked": 92.16}, (512, 8192): {"scan": 231.8, "chunked": 205.5},
    (1024, 512): {"scan": 20.82, "chunked": 16.61}, (1024, 2048): {"scan": 176.1, "chunked": 95.43},
    (1024, 8192): {"scan": 319.1, "chunked": 298.9},
}
MAMBA_PAGE_CPU_FWD_BWD_MS = {
    (256, 512): {"scan": 173.6, "chunked": 41.06}, (256, 2048): {"scan": 700.5, "chunked": 235.8},
    (256, 8192): {"scan": 2619., "chunked": 644.9}, (512, 512): {"scan": 369.1, "chunked": 84.71},
    (512, 2048): {"scan": 1934., "chunked": 383.1}, (512, 8192): {"scan": 5166., "chunked": 1037.},
    (1024, 512): {"scan": 587.1, "chunked": 215.8}, (1024, 2048): {"scan": 2677., "chunked": 567.6},
    (1024, 8192): {"scan": 7782., "chunked": 1868.},
}

# The same page's chunked path over its whole grid, (fwd, fwd_bwd) median ms on
# the RTX 3090: context for --grid, not a target.
PAGE_CHUNKED_MS = {
    ("g2h8_d128", 512): (0.332, 0.901), ("g2h8_d128", 2048): (1.170, 3.210),
    ("g2h8_d128", 8192): (4.182, 11.883),
    ("g1h24_dk128_dv64", 512): (0.258, 0.725), ("g1h24_dk128_dv64", 2048): (0.943, 2.632),
    ("g1h24_dk128_dv64", 8192): (3.461, 10.695),
    ("g1h1_d128", 512): (0.0890, 0.252), ("g1h1_d128", 2048): (0.284, 0.656),
    ("g1h1_d128", 8192): (0.909, 2.439),
    ("g2h4_dk48_dv40", 512): (0.112, 0.296), ("g2h4_dk48_dv40", 2048): (0.371, 0.968),
    ("g2h4_dk48_dv40", 8192): (1.448, 3.736),
}


def nominal_flops(s):
    N = s.B * s.H * s.T
    f = N * (C_NOM * (s.dk + s.dv) + 4 * s.dk * s.dv)
    b = N * (C_NOM * (3 * s.dk + 2 * s.dv) + 10 * s.dk * s.dv)
    return f, b


def io_bytes(s):
    inp = 4 * (2 * s.B * s.G * s.T * s.dk + s.B * s.H * s.T * s.dv + s.B * s.H * s.T + s.B * s.H * s.dk * s.dv)
    y = 4 * s.B * s.H * s.T * s.dv
    return inp + y, 3 * inp + 2 * y


def kernel_work(s):
    """Algorithmic work per launch of each kernel: (bound, amount, unit)."""
    N = s.B * s.H * s.T
    E = s.dk * s.dv
    return {
        "state_scan": ("mfma", N * 2 * E, "FLOP"),
        "chunk_output": ("mfma", N * (C_NOM * (s.dk + s.dv) + 2 * E), "FLOP"),
        "state_scan_bidir": ("mfma", 2 * N * 2 * E, "FLOP"),
        "bwd_grads": ("mfma", N * (C_NOM * (3 * s.dk + 2 * s.dv) + 6 * E), "FLOP"),
        "state_scan_rev": ("mfma", N * 2 * E, "FLOP"),
        "aux": ("hbm", 0, "B"),
    }


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "chunked_ssd_scan_fwd_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    or None if absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = d.get(kernel)
    if not ent or ent.get("workload") != workload or ent.get("source_hash") != source_hash():
        return None
    return ent.get("bytes_per_launch")


def cpu_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model


def fwd_bwd_bytes(B, G, H, T, dk, dv, ws):
    """Device bytes of one fwd_bwd: inputs, y, the five gradients and the workspace."""
    f = 4
    return (f * (4 * B * G * T * dk            # q, k, dq, dk
                 + 4 * B * H * T * dv          # v, dy, y, dv
                 + 2 * B * H * T               # log_alpha, dlog_alpha
                 + 2 * B * H * dk * dv)        # h0, dh0
            + ws)


def max_len_search(args, torch, ssd):
    """Longest T (doubling from 8192) whose fwd_bwd at g2h8_d128, B=4, fits in HBM.

    Inputs follow the synthetic recipe but are drawn on the device (a host copy
    of the largest sizes would need some hundred GiB of host memory).  A size is
    run only if its predicted bytes fit in the free HBM, so the search never
    relies on an allocation failure; every run checks that y and the gradients
    are finite.
    """
    import math
    B, G, H, dk, dv = 4, 2, 8, 128, 128
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    runs = []
    T = 8192
    best = 0
    stop = None
    while T <= args.max_len_cap:
        sa = ssd.ShapeArg(B, G, H, T, dk, dv)
        ws_b = ssd.workspace_size(sa, True)
        need = fwd_bwd_bytes(B, G, H, T, dk, dv, ws_b)
        free, total = torch.cuda.mem_get_info()
        if need > 0.92 * free:
            stop = {"T": T, "predicted_bytes": need, "free_bytes": free, "total_bytes": total}
            break
        gen.manual_seed(T)
        q = torch.randn((B, G, T, dk), device=dev, generator=gen) / math.sqrt(128.0)
        k = torch.randn((B, G, T, dk), device=dev, generator=gen) / math.sqrt(128.0)
        v = torch.randn((B, H, T, dv), device=dev, generator=gen)
        la = -torch.nn.functional.softplus(-2.0 + torch.randn((B, H, T), device=dev, generator=gen))
        h0 = 0.1 * torch.randn((B, H, dk, dv), device=dev, generator=gen)
        dy = torch.randn((B, H, T, dv), device=dev, generator=gen)
        y = torch.empty((B, H, T, dv), device=dev)
        grads = (torch.empty((B, G, T, dk), device=dev), torch.empty((B, G, T, dk), device=dev),
                 torch.empty((B, H, T, dv), device=dev), torch.empty((B, H, T), device=dev),
                 torch.empty((B, H, dk, dv), device=dev))
        ws = torch.empty(ws_b, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()

        def step():
            ssd.fwd(q, k, v, la, h0, out=y, workspace=ws)
            ssd.bwd(q, k, v, la, h0, dy, out=grads, workspace=ws)

        step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        finite = bool(torch.isfinite(y).all()) and all(bool(torch.isfinite(g).all()) for g in grads)
        runs.append({"T": T, "fwd_bwd_ms": e0.elapsed_time(e1), "workspace_bytes": ws_b,
                     "predicted_bytes": need, "peak_allocated_bytes": torch.cuda.max_memory_allocated(),
                     "finite": finite})
        print(json.dumps(runs[-1]), file=sys.stderr, flush=True)
        if not finite:
            stop = {"T": T, "reason": "non-finite output"}
            break
        best = T
        del q, k, v, la, h0, dy, y, grads, ws
        torch.cuda.empty_cache()
        T *= 2
    print(json.dumps({"metric": "max_len fwd_bwd g2h8_d128 B=4 fp32 (T doubling from 8192)", "value": best,
                      "unit": "tokens", "higher_is_better": True, "device": torch.cuda.get_device_name(0),
                      "runs": runs, "stopped_at": stop, "data": "synthetic, drawn on the device"}), flush=True)


def grid_sweep(args, torch, ssd):
    """fwd and fwd_bwd at every shape of the pages' grid, timed by the pages'
    protocol (`protocol_ms`, `--repeats` samples): median ms per call, nominal
    TFLOP/s, GB/s of the inputs and outputs, and the fraction of the step
    roofline (the larger of the nominal FLOPs at the fp32 MFMA peak and those
    bytes at the HBM peak).  Inputs follow the synthetic recipe (mu = -4 for
    the 24-head shape)."""
    from ssd_workload import PAGE_GRID, make_inputs
    for i, ((name, T), s) in enumerate(PAGE_GRID.items()):
        x = make_inputs(s, 2000 + i, mu=-4.0 if name.startswith("g1h24") else -2.0)
        d = {k: torch.from_numpy(v).to("cuda") for k, v in x.items()}
        sa = ssd.ShapeArg(s.B, s.G, s.H, s.T, s.dk, s.dv)
        ws = torch.empty(ssd.workspace_size(sa, True), dtype=torch.uint8, device="cuda")
        y = torch.empty((s.B, s.H, s.T, s.dv), device="cuda")
        grads = (torch.empty((s.B, s.G, s.T, s.dk), device="cuda"), torch.empty((s.B, s.G, s.T, s.dk), device="cuda"),
                 torch.empty((s.B, s.H, s.T, s.dv), device="cuda"), torch.empty((s.B, s.H, s.T), device="cuda"),
                 torch.empty((s.B, s.H, s.dk, s.dv), device="cuda"))

        def fwd():
            ssd.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], out=y, workspace=ws)

        def step():
            fwd()
            ssd.bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], d["dy"], out=grads, workspace=ws)

        f_fwd, f_bwd = nominal_flops(s)
        b_fwd, b_fb = io_bytes(s)
        out = {"workload": f"{name}_T{T}", "shape": {"B": s.B, "G": s.G, "H": s.H, "T": s.T, "dk": s.dk, "dv": s.dv},
               "fwd_chunk": 64 * ssd.fwd_state_stride(sa)}
        for key, fn, fl, by in (("fwd", fwd, f_fwd, b_fwd), ("fwd_bwd", step, f_fwd + f_bwd, b_fb)):
            for _ in range(args.warmup):
                fn()
            r = protocol_ms(torch, fn, repeats=args.repeats)
            ms = r["median_ms"]
            out[key] = {"median_ms": ms, "q1_ms": r["q1_ms"], "q3_ms": r["q3_ms"], "inner": r["inner"], "tflops": fl / (ms * 1e-3) / 1e12, "gbps_io": by / (ms * 1e-3) / 1e9,
                        "roofline_frac": max(fl / PEAK_FP32_MFMA, by / PEAK_HBM) / (ms * 1e-3)}
        pf, pfb = PAGE_CHUNKED_MS[(name, T)]
        out["page_chunked_rtx3090_ms"] = {"fwd": pf, "fwd_bwd": pfb}
        out["dtype"] = "f32"
        out["data"] = "synthetic"
        print(json.dumps(out), flush=True)
        del d, ws, y, grads
        torch.cuda.empty_cache()


# The selective scan's own roofline.  It is no contraction: per element
# (b, t, d) and state n the recurrence takes one exponential and three
# single-rate operations (the exponent's product, the input's product, the
# multiply-add into the state) and the output one more multiply-add.  An
# exponential costs two fp32 issue slots: the probe in device_facts measures
# its throughput at half that of v_fma_f32 on this chip.  So the work is
# N (4 + 2) lane slots per element against 256 CUs x 4 SIMDs x 16 lanes x
# 2.4 GHz; the bytes are the inputs and y.
EXP_SLOTS = 2
PEAK_VALU_SLOTS = 256 * 4 * 16 * 2.4e9


def mamba_work(s, backward=False):
    """(lane slots, bytes) of the least work: the forward's N (4 + 2) slots
    per element, and for fwd_bwd N 14 more -- one exponential (2) and its
    exponent's product for the decay, shared by the recomputed state and the
    adjoint, and eleven single-rate operations (the state's 2, the
    adjoint's 2, dx, ddelta 2, dA 2, dB, dC); the bytes are every argument
    read once and every result written once."""
    elems, bln, dn = s.B * s.L * s.D, s.B * s.L * s.N, s.D * s.N
    fwd_slots = 4 + EXP_SLOTS
    if not backward:
        return elems * s.N * fwd_slots, 4 * (3 * elems + 2 * bln + dn + s.D)
    # fwd: x, delta, B, C, A, Dskip in, y out; bwd: those and dy in, six gradients out
    io_f = 4 * (3 * elems + 2 * bln + dn + s.D)
    io_b = 4 * (3 * elems + 2 * bln + dn + s.D) + 4 * (2 * elems + 2 * bln + dn + s.D)
    return elems * s.N * (fwd_slots + 1 + EXP_SLOTS + 11), io_f + io_b


def mamba_cpu_baseline(point):
    """The selective scan's fp64 oracle on the host cores at one point of its
    page's grid (the whole workload): the forward alone, then forward +
    backward, one run each (at the largest point some 10 s of host work)."""
    from oracle import mamba as mo
    from ssd_workload.mamba import MAMBA_GRID, make_mamba_inputs
    s = MAMBA_GRID[point]
    inp = make_mamba_inputs(s, 3000 + point[0] + point[1])
    a = [inp[k] for k in ("x", "delta", "A", "B", "C", "Dskip")]
    t0 = time.perf_counter()
    mo.fwd(*a)
    t1 = time.perf_counter()
    mo.fwd(*a)
    mo.bwd(*a, inp["dy"])
    t2 = time.perf_counter()
    fwd_ms, fb_ms = (t1 - t0) * 1e3, (t2 - t1) * 1e3
    sl, _ = mamba_work(s)
    slb, _ = mamba_work(s, backward=True)
    return {"value": fb_ms, "unit": "ms", "cores": mo.num_threads(), "kind": "oracle", "cpu_model": cpu_info(),
            "fwd_ms": fwd_ms, "fwd_bwd_ms": fb_ms,
            "fwd_lane_ops_per_s": sl / (fwd_ms * 1e-3), "fwd_bwd_lane_ops_per_s": slb / (fb_ms * 1e-3),
            "sample": f"whole mamba_d{point[0]}_L{point[1]} workload in fp64: forward alone, then forward + "
                      "backward, one run each (value: fwd_bwd ms)"}


def mamba_sweep(args, torch, ssd, points=None):
    """mamba_fwd (fwd), mamba_fwd_bwd (fwd_bwd: y and the gradients in one
    call) and mamba_fwd then mamba_bwd (fwd_then_bwd) at the points of
    kernel_mamba_cpu.json's grid (batch 4, state 16), timed by the pages'
    protocol; the page's CPU medians go along as context."""
    from ssd_workload.mamba import MAMBA_GRID, make_mamba_inputs
    out = []
    for (D, L), s in MAMBA_GRID.items():
        if points is not None and (D, L) not in points:
            continue
        inp = make_mamba_inputs(s, 3000 + D + L)
        d = {k: torch.from_numpy(v).to("cuda") for k, v in inp.items()}
        sa = ssd.MambaShapeArg(s.B, s.L, s.D, s.N)
        ws = torch.empty(max(1, ssd.mamba_workspace_size(sa)), dtype=torch.uint8, device="cuda")
        wsb = torch.empty(max(1, ssd.mamba_workspace_size(sa, backward=True)), dtype=torch.uint8, device="cuda")
        y = torch.empty((s.B, s.L, s.D), device="cuda")
        grads = (torch.empty_like(d["x"]), torch.empty_like(d["x"]), torch.empty_like(d["A"]),
                 torch.empty_like(d["B"]), torch.empty_like(d["C"]), torch.empty_like(d["Dskip"]))

        def fwd():
            ssd.mamba_fwd(d["x"], d["delta"], d["A"], d["B"], d["C"], d["Dskip"], out=y, workspace=ws)

        def fwd_bwd():
            # the value (y) and all six gradients in one call
            ssd.mamba_fwd_bwd(d["x"], d["delta"], d["A"], d["B"], d["C"], d["Dskip"], d["dy"], out=(y,) + grads,
                              workspace=wsb)

        def fwd_then_bwd():
            # the same through the two separate calls (the backward forms the
            # forward's states again)
            fwd()
            ssd.mamba_bwd(d["x"], d["delta"], d["A"], d["B"], d["C"], d["Dskip"], d["dy"], out=grads,
                          workspace=wsb)

        line = {"workload": f"mamba_d{D}_L{L}", "shape": {"B": s.B, "L": s.L, "D": s.D, "N": s.N}}
        for mode, fn in (("fwd", fwd), ("fwd_bwd", fwd_bwd), ("fwd_then_bwd", fwd_then_bwd)):
            for _ in range(args.warmup):
                fn()
            r = protocol_ms(torch, fn, repeats=args.repeats)
            t = r["median_ms"] * 1e-3
            slots, io = mamba_work(s, backward=mode != "fwd")
            line[mode] = {"median_ms": r["median_ms"], "q1_ms": r["q1_ms"], "q3_ms": r["q3_ms"],
                          "gbps_io": io / t / 1e9, "hbm_frac": io / t / PEAK_HBM,
                          "alu_frac": slots / t / PEAK_VALU_SLOTS,
                          "roofline_frac": max(io / PEAK_HBM, slots / PEAK_VALU_SLOTS) / t}
        line.update({"page_cpu_ms": {"fwd": MAMBA_PAGE_CPU_MS.get((D, L)),
                                     "fwd_bwd": MAMBA_PAGE_CPU_FWD_BWD_MS.get((D, L))},
                     "dtype": "f32", "data": "synthetic"})
        out.append(line)
        del d, ws, wsb, y, grads
        torch.cuda.empty_cache()
    return out


def quartiles(vals):
    import numpy as np
    a = np.asarray(vals, dtype=np.float64)
    return {"median_ms": float(np.median(a)), "q1_ms": float(np.percentile(a, 25)),
            "q3_ms": float(np.percentile(a, 75))}


def protocol_ms(torch, fn, repeats=5, target_ms=50.0):
    """The pages' timing protocol: one warm-up call (first-call latency), three
    more untimed calls, then `repeats` samples, each `inner` back-to-back calls
    between two events, inner = clamp(ceil(50 ms / single call), 1, 200).
    Returns per-call quartiles (ms), inner and the first-call latency."""
    import math
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    first_ms = (time.perf_counter() - t0) * 1e3
    for _ in range(3):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    fn()
    e1.record()
    torch.cuda.synchronize()
    single = max(e0.elapsed_time(e1), 1e-3)
    inner = int(min(200, max(1, math.ceil(target_ms / single))))
    per = []
    for _ in range(repeats):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        evs[0].record()
        for _ in range(inner):
            fn()
        evs[1].record()
        torch.cuda.synchronize()
        per.append(evs[0].elapsed_time(evs[1]) / inner)
    return {**quartiles(per), "inner": inner, "repeats": repeats, "first_call_ms": first_ms}


def config_rows(torch, ssd, args):
    """fwd and fwd_bwd of the five measured workloads: ms quartiles, nominal
    TFLOP/s, GB/s of the algorithmic input/output bytes, and the fraction of
    the step roofline (the longer of the nominal FLOPs at the fp32 MFMA peak
    and those bytes at the HBM peak)."""
    from ssd_workload import WORKLOADS, make_inputs
    rows = {}
    for w in WORKLOADS:
        s = w.shape
        x = make_inputs(s, w.seed, mu=w.mu)
        d = {k: torch.from_numpy(v).to("cuda") for k, v in x.items()}
        sa = ssd.ShapeArg(s.B, s.G, s.H, s.T, s.dk, s.dv)
        ws = torch.empty(max(1, ssd.workspace_size(sa, True)), dtype=torch.uint8, device="cuda")
        y = torch.empty((s.B, s.H, s.T, s.dv), device="cuda")
        grads = (torch.empty((s.B, s.G, s.T, s.dk), device="cuda"), torch.empty((s.B, s.G, s.T, s.dk), device="cuda"),
                 torch.empty((s.B, s.H, s.T, s.dv), device="cuda"), torch.empty((s.B, s.H, s.T), device="cuda"),
                 torch.empty((s.B, s.H, s.dk, s.dv), device="cuda"))

        def fwd():
            ssd.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], out=y, workspace=ws)

        def step():
            fwd()
            ssd.bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], d["dy"], out=grads, workspace=ws)

        f_fwd, f_bwd = nominal_flops(s)
        b_fwd, b_fb = io_bytes(s)
        row = {"shape": {"B": s.B, "G": s.G, "H": s.H, "T": s.T, "dk": s.dk, "dv": s.dv}}
        for key, fn, fl, by in (("fwd", fwd, f_fwd, b_fwd), ("fwd_bwd", step, f_fwd + f_bwd, b_fb)):
            for _ in range(args.warmup):
                fn()
            r = protocol_ms(torch, fn, repeats=args.repeats)
            t = r["median_ms"] * 1e-3
            r.update({"tflops": fl / t / 1e12, "gbps_io": by / t / 1e9,
                      "mfma_frac": fl / t / PEAK_FP32_MFMA, "hbm_frac": by / t / PEAK_HBM,
                      "roofline_frac": max(fl / PEAK_FP32_MFMA, by / PEAK_HBM) / t,
                      "bound": "mfma" if fl / PEAK_FP32_MFMA >= by / PEAK_HBM else "hbm"})
            row[key] = r
        rows[w.name] = row
        print(json.dumps({"config": w.name, **{k: row[k]["median_ms"] for k in ("fwd", "fwd_bwd")}}),
              file=sys.stderr, flush=True)
        del d, ws, y, grads
        torch.cuda.empty_cache()
    return rows


def device_facts(torch):
    """Measured on this device: plain-copy HBM bandwidth, and the fp32 MFMA
    rate and shader clock of an MFMA loop on every SIMD (benchmark probe
    library; absent if it was not built)."""
    import ctypes
    import numpy as np
    out = {}
    n = (1 << 30) // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty(n, device="cuda")
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    out["copy_gbps"] = 2 * 4 * n / (ms * 1e-3) / 1e9
    out["copy_note"] = "1 GiB device-to-device copy, read + write bytes / time"
    del src, dst
    path = os.path.join(ROOT, "chunked_ssd_scan_fwd_amd", "libssd_probe.so")
    if not os.path.exists(path):
        out["mfma_loop"] = None
        return out
    lib = ctypes.CDLL(path)
    lib.probe_mfma_loop_bytes.argtypes = [ctypes.c_int]
    lib.probe_mfma_loop_bytes.restype = ctypes.c_size_t
    lib.probe_mfma_loop.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.probe_mfma_loop.restype = ctypes.c_int
    lib.probe_mfma_chains.restype = ctypes.c_int
    lib.probe_wall_clock_khz.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = cus, 20000
    buf = torch.empty(int(lib.probe_mfma_loop_bytes(blocks)), dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(2):
        if lib.probe_mfma_loop(ctypes.c_void_p(buf.data_ptr()), blocks, iters, stream) != 0:
            raise RuntimeError("probe_mfma_loop failed")
    e0.record()
    lib.probe_mfma_loop(ctypes.c_void_p(buf.data_ptr()), blocks, iters, stream)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    flops = blocks * 4 * iters * lib.probe_mfma_chains() * 32 * 32 * 2 * 2
    ticks = buf[blocks * 1024:].view(torch.int64).view(blocks, 4).cpu().numpy().astype(np.float64)
    khz = lib.probe_wall_clock_khz()
    mhz = None
    if khz > 0:
        rates = (ticks[:, 1] - ticks[:, 0]) / ((ticks[:, 3] - ticks[:, 2]) / (khz * 1e3)) / 1e6
        mhz = float(np.median(rates))
    out["mfma_loop"] = {"tflops": flops / (ms * 1e-3) / 1e12, "frac_of_spec": flops / (ms * 1e-3) / PEAK_FP32_MFMA,
                        "shader_clock_mhz": mhz, "blocks": blocks, "waves_per_cu": 4,
                        "note": "independent v_mfma_f32_32x32x2f32 chains on every SIMD; clock = shader-clock "
                                "counter over the real-time counter during the loop"}
    # lane-operation rates of fp32 multiply-adds and of exponentials (8 waves per SIMD)
    lib.probe_valu_loop_bytes.argtypes = [ctypes.c_int]
    lib.probe_valu_loop_bytes.restype = ctypes.c_size_t
    lib.probe_valu_loop.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.probe_valu_loop.restype = ctypes.c_int
    lib.probe_valu_chains.restype = ctypes.c_int
    vblocks, viters = cus * 8, 4096
    vbuf = torch.empty(int(lib.probe_valu_loop_bytes(vblocks)), dtype=torch.uint8, device="cuda")
    rates = {}
    for mode, name in ((0, "fma"), (1, "exp")):
        for _ in range(2):
            if lib.probe_valu_loop(ctypes.c_void_p(vbuf.data_ptr()), vblocks, viters, mode, stream) != 0:
                raise RuntimeError("probe_valu_loop failed")
        e0.record()
        for _ in range(3):
            lib.probe_valu_loop(ctypes.c_void_p(vbuf.data_ptr()), vblocks, viters, mode, stream)
        e1.record()
        torch.cuda.synchronize()
        ops = 3 * vblocks * 256 * viters * lib.probe_valu_chains()
        rates[name] = ops / (e0.elapsed_time(e1) * 1e-3)
    out["valu_loop"] = {"fma_tlane_ops": rates["fma"] / 1e12, "exp_tlane_ops": rates["exp"] / 1e12,
                        "exp_cost_in_fma_slots": rates["fma"] / rates["exp"],
                        "fma_frac_of_spec": rates["fma"] / PEAK_VALU_SLOTS,
                        "note": "independent chains of v_fma_f32 or v_exp_f32, 8 waves per SIMD on every CU"}
    return out


def cpu_baseline(x, w, f_fwd, f_bwd, repeats):
    """The fp64 oracle on the host cores: fwd alone and fwd + bwd, `repeats`
    each, on the whole workload; nominal TFLOP/s of the median."""
    import oracle
    rec = {}
    for key, fl in (("fwd", f_fwd), ("fwd_bwd", f_fwd + f_bwd)):
        per = []
        for _ in range(repeats):
            t0 = time.perf_counter()
            oracle.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])
            if key == "fwd_bwd":
                oracle.bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], x["dy"])
            per.append((time.perf_counter() - t0) * 1e3)
        r = quartiles(per)
        r["tflops"] = fl / (r["median_ms"] * 1e-3) / 1e12
        rec[key] = r
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed steps first; the GPU needs some 20 ms of work to reach its working clocks")
    ap.add_argument("--workload", default="g2h8_d128_T8192")
    ap.add_argument("--repeats", type=int, default=5, help="samples per config in the per-config table")
    ap.add_argument("--cpu-repeats", type=int, default=3, help="oracle repeats per mode for the CPU baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-config table")
    ap.add_argument("--no-reuse", action="store_true",
                    help="skip the secondary fwd + bwd_from_fwd timing (profiling runs: its reverse-only "
                         "state scan would add launches of another kernel)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (5 launches) and exit")
    ap.add_argument("--max-len", action="store_true",
                    help="only run the T-doubling maximum-length search for fwd_bwd and exit")
    ap.add_argument("--max-len-cap", type=int, default=1 << 22, help="largest T the search tries")
    ap.add_argument("--grid", action="store_true",
                    help="only time fwd and fwd_bwd at every shape of the pages' grid, one JSON line each, and exit")
    ap.add_argument("--mamba-point", default="",
                    help="with --mamba: only this point of the grid, as DIM,SEQ (e.g. 1024,8192)")
    ap.add_argument("--mamba", action="store_true",
                    help="only time the selective (Mamba-style) scan at every point of its page's grid, one JSON "
                         "line each, and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import chunked_ssd_scan_fwd_amd as ssd
    from ssd_workload import workload, make_inputs, rel_err

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    if args.copy_mib > 0:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty(n, device="cuda")
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 4 * n, "launches": 5}), flush=True)
        return
    if args.max_len:
        max_len_search(args, torch, ssd)
        return
    if args.mamba:
        pts = None
        if args.mamba_point:
            pts = {tuple(int(v) for v in args.mamba_point.split(","))}
        for line in mamba_sweep(args, torch, ssd, points=pts):
            print(json.dumps(line), flush=True)
        return
    if args.grid:
        grid_sweep(args, torch, ssd)
        return
    w = workload(args.workload)
    s = w.shape
    x = make_inputs(s, w.seed, mu=w.mu)
    d = {k: torch.from_numpy(v).to("cuda") for k, v in x.items()}
    sa = ssd.ShapeArg(s.B, s.G, s.H, s.T, s.dk, s.dv)
    ws = torch.empty(ssd.workspace_size(sa, True), dtype=torch.uint8, device="cuda")
    y = torch.empty((s.B, s.H, s.T, s.dv), device="cuda")
    grads = (torch.empty((s.B, s.G, s.T, s.dk), device="cuda"), torch.empty((s.B, s.G, s.T, s.dk), device="cuda"),
             torch.empty((s.B, s.H, s.T, s.dv), device="cuda"), torch.empty((s.B, s.H, s.T), device="cuda"),
             torch.empty((s.B, s.H, s.dk, s.dv), device="cuda"))

    def fwd(timer=None):
        ssd.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], out=y, workspace=ws, timer=timer)

    def bwd(timer=None):
        ssd.bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], d["dy"], out=grads, workspace=ws, timer=timer)

    def step(timer=None):
        fwd(timer)
        bwd(timer)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step()
    torch.cuda.synchronize()
    first_call_ms = (time.perf_counter() - t0) * 1e3
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def timed(fn, K, kernels=(), per_step=True):
        """K calls of fn between two events, with an event after every call
        when `per_step` (each is a marker packet on the stream, a few
        microseconds of stream time); `kernels` (names, or None for all) are
        timed per launch with events bound to their dispatches."""
        timer = None if (kernels is not None and len(kernels) == 0) else ssd.KernelTimer(kernels)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        evs[0].record()
        for i in range(K):
            fn(timer)
            if per_step or i == K - 1:
                evs[i + 1].record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - wall0) * 1e3
        res = None
        if timer is not None:
            res = timer.results()
            timer.close()
        per = [evs[i].elapsed_time(evs[i + 1]) for i in range(K)] if per_step else []
        total = evs[0].elapsed_time(evs[K])
        return total / K, per, wall / K, res

    K = args.steps
    # Per-kernel pass (not the headline): K steps with every kernel timed by
    # events bound to its dispatch, for the per-kernel table and to find the
    # dominant kernel.  Each timed dispatch costs a few microseconds of stream
    # time, so the headline region below times the dominant kernel only.
    _, _, _, kern_all = timed(step, K, kernels=None)
    dom = max((n for n in kern_all if kern_all[n][1] and n != "aux"), key=lambda n: kern_all[n][0])
    # Timed region: exactly K steps between two events; the dominant kernel's
    # launches carry HIP events on the launch stream, for its roofline.
    step_ms, _, wall_ms, kern_dom = timed(step, K, kernels=[dom], per_step=False)
    # The per-step distribution (median, quartiles) comes from a pass of its
    # own with an event after every step.
    _, per_step, _, _ = timed(step, K)
    # fwd and bwd alone: K back-to-back calls between two events (as the
    # step), and their per-call quartiles from a pass of their own
    fwd_ms, _, _, _ = timed(fwd, K, per_step=False)
    _, fwd_per, _, _ = timed(fwd, K)
    bwd_ms, _, _, _ = timed(bwd, K, per_step=False)
    _, bwd_per, _, _ = timed(bwd, K)

    # Secondary (not the headline): the backward that reuses the forward's
    # residuals from the shared workspace instead of recomputing them.
    def step_reuse(timer=None):
        fwd()
        ssd.bwd_from_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], d["dy"], out=grads, workspace=ws)

    reuse_ms, reuse_per = None, []
    if not args.no_reuse:
        for _ in range(3):
            step_reuse()
        reuse_ms, reuse_per, _, _ = timed(step_reuse, K)

    f_fwd, f_bwd = nominal_flops(s)
    b_fwd, b_fwd_bwd = io_bytes(s)
    value = (f_fwd + f_bwd) / (step_ms * 1e-3) / 1e12
    t_roof_fb = max((f_fwd + f_bwd) / PEAK_FP32_MFMA, b_fwd_bwd / PEAK_HBM)
    t_roof_f = max(f_fwd / PEAK_FP32_MFMA, b_fwd / PEAK_HBM)
    # The nominal count takes Q K^T once per head; the kernels form it once per
    # (b, g, chunk) and share it over the group's heads.  The group-aware count
    # takes it once per group (forward once, backward once).
    hpg = s.H // s.G
    qk_per_group = s.B * s.G * s.T * C_NOM * s.dk
    f_fwd_g = f_fwd - qk_per_group * (hpg - 1)
    f_bwd_g = f_bwd - qk_per_group * (hpg - 1)

    work = kernel_work(s)
    kernels = {}
    for name, (tot, cnt) in kern_all.items():
        if cnt:
            kernels[name] = {"avg_us": 1e3 * tot / cnt, "launches": cnt, "share": tot / (step_ms * K)}
    bound, amount, unit = work[dom]
    dom_tot, dom_cnt = kern_dom[dom]
    avg_s = dom_tot / dom_cnt * 1e-3
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": amount / avg_s / 1e12, "peak": PEAK_FP32_MFMA / 1e12,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": amount / avg_s / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = dom
    roof["avg_us"] = avg_s * 1e6
    roof["launches"] = dom_cnt
    roof["work_per_launch"] = amount
    roof["traffic"] = traffic_from_profiles(dom, w.name)
    for name in kernels:
        bnd, amt, _ = work[name]
        if amt == 0:
            continue
        a = amt / (kernels[name]["avg_us"] * 1e-6)
        kernels[name]["achieved"] = a / 1e12 if bnd == "mfma" else a / 1e9
        kernels[name]["unit"] = "TFLOP/s" if bnd == "mfma" else "GB/s"
        kernels[name]["frac"] = a / (PEAK_FP32_MFMA if bnd == "mfma" else PEAK_HBM)

    # Parity of the timed path against the oracle on the whole tensors, and
    # the CPU baseline (the oracle timed on the host cores).
    cpu = None
    parity = None
    if not args.no_cpu:
        import oracle
        fwd()
        bwd()
        torch.cuda.synchronize()
        ref_y = oracle.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])
        ref = oracle.bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], x["dy"])
        parity = {"y": rel_err(y.cpu().numpy(), ref_y)}
        for name, t in zip(("dq", "dk", "dv", "dlog_alpha", "dh0"), grads):
            parity[name] = rel_err(t.cpu().numpy(), ref[name])
        del ref_y, ref
        rec = cpu_baseline(x, w, f_fwd, f_bwd, args.cpu_repeats)
        cpu = {"value": rec["fwd_bwd"]["tflops"], "unit": "TFLOP/s", "cores": oracle.num_threads(),
               "kind": "oracle", "cpu_model": cpu_info(), "fwd": rec["fwd"], "fwd_bwd": rec["fwd_bwd"],
               "sample": f"whole {w.name} workload in fp64: forward alone and forward + backward, "
                         f"{args.cpu_repeats} runs each (value: nominal fwd_bwd FLOPs / median wall time)"}

    configs = None if args.no_configs else config_rows(torch, ssd, args)
    # the second workload of the pages (kernel_mamba_cpu.json) at its largest point
    mamba = None if args.no_configs else mamba_sweep(args, torch, ssd, points={(1024, 8192)})
    if mamba and not args.no_cpu:
        mamba[0]["cpu_baseline"] = mamba_cpu_baseline((1024, 8192))
    facts = device_facts(torch)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        # the pages' chunked fwd_bwd at this workload (RTX 3090, 11.883 ms, i.e.
        # 6.3 nominal TFLOP/s): another machine's number, context only
        "vs_baseline": (PAGE_FWD_BWD_MS / step_ms) if w.name == "g2h8_d128_T8192" else None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={s.B} G={s.G} H={s.H} T={s.T} dk={s.dk} dv={s.dv}, "
                               "step = ssd_fwd + ssd_bwd",
                   # the forward's chunk length (128: on chunk pairs) and the backward's
                   "chunk": {"fwd": 64 * ssd.fwd_state_stride(sa), "bwd": 64}, "seed": w.seed},
        "roofline": roof,
        "cpu_baseline": cpu,
        "fwd_bwd": {**quartiles(per_step), "tflops": value, "roofline_frac": t_roof_fb / (step_ms * 1e-3),
                    "gbps_io": b_fwd_bwd / (step_ms * 1e-3) / 1e9, "wall_ms": wall_ms,
                    "roofline_frac_group_qk": max((f_fwd_g + f_bwd_g) / PEAK_FP32_MFMA, b_fwd_bwd / PEAK_HBM)
                    / (step_ms * 1e-3)},
        "fwd": {**quartiles(fwd_per), "ms": fwd_ms, "tflops": f_fwd / (fwd_ms * 1e-3) / 1e12,
                "roofline_frac": t_roof_f / (fwd_ms * 1e-3), "gbps_io": b_fwd / (fwd_ms * 1e-3) / 1e9,
                "roofline_frac_group_qk": max(f_fwd_g / PEAK_FP32_MFMA, b_fwd / PEAK_HBM) / (fwd_ms * 1e-3)},
        "bwd": {**quartiles(bwd_per), "ms": bwd_ms, "tflops": f_bwd / (bwd_ms * 1e-3) / 1e12},
        "flop_convention": "nominal: per token-head, C=64, causal tiles as half, Q K^T counted once per head "
                           "(fwd C(dk+dv)+4 dk dv, bwd C(3dk+2dv)+10 dk dv); *_group_qk: Q K^T once per group",
        "fwd_bwd_reuse": None if reuse_ms is None else {**quartiles(reuse_per), "ms": reuse_ms,
                          "note": "secondary: ssd_fwd then ssd_bwd_from_fwd, which reuses the forward's "
                                  "chunk states from the workspace (not the stateless headline step)"},
        "page_context_ms": {"fwd": PAGE_CHUNKED_MS[("g2h8_d128", 8192)][0],
                            "fwd_bwd": PAGE_CHUNKED_MS[("g2h8_d128", 8192)][1],
                            "note": "the pages' JAX chunked path on an RTX 3090 at this workload: context only"},
        "kernels": kernels,
        "parity_rel_err": parity,
        "configs": configs,
        "mamba": mamba,
        "device_facts": facts,
        "first_call_ms": first_call_ms,
        "memory": {"workspace_bytes_fwd": ssd.workspace_size(sa, False), "workspace_bytes_bwd": ssd.workspace_size(sa, True),
                   "fwd_bwd_bytes": fwd_bwd_bytes(s.B, s.G, s.H, s.T, s.dk, s.dv, ssd.workspace_size(sa, True)),
                   "peak_allocated_bytes": torch.cuda.max_memory_allocated()},
        "device": torch.cuda.get_device_name(0),
        "source_hash": source_hash(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
