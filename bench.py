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
    NC = (s.T + 63) // 64
    E = s.dk * s.dv
    states = 4 * s.B * s.H * NC * E
    return {
        "chunk_cumsum": ("hbm", 4 * N + 4 * s.B * s.H * NC * 64 + 4 * s.B * s.H * NC, "B"),
        "state_scan": ("mfma", N * 2 * E, "FLOP"),
        "chunk_output": ("mfma", N * (C_NOM * (s.dk + s.dv) + 2 * E), "FLOP"),
        "state_scan_bidir": ("mfma", 2 * N * 2 * E, "FLOP"),
        "bwd_grads": ("mfma", N * (C_NOM * (3 * s.dk + 2 * s.dv) + 6 * E), "FLOP"),
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
    """fwd and fwd_bwd at every shape of the pages' grid: median ms over
    `--steps` calls (events after every call), nominal TFLOP/s, GB/s of the
    inputs and outputs, and the fraction of the step roofline (the larger of
    the nominal FLOPs at the fp32 MFMA peak and those bytes at the HBM peak).
    Inputs follow the synthetic recipe (mu = -4 for the 24-head shape)."""
    import numpy as np
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

        def med_ms(fn):
            for _ in range(args.warmup):
                fn()
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
            torch.cuda.synchronize()
            evs[0].record()
            for j in range(args.steps):
                fn()
                evs[j + 1].record()
            torch.cuda.synchronize()
            return float(np.median([evs[j].elapsed_time(evs[j + 1]) for j in range(args.steps)]))

        f_fwd, f_bwd = nominal_flops(s)
        b_fwd, b_fb = io_bytes(s)
        out = {"workload": f"{name}_T{T}", "shape": {"B": s.B, "G": s.G, "H": s.H, "T": s.T, "dk": s.dk, "dv": s.dv}}
        for key, fn, fl, by in (("fwd", fwd, f_fwd, b_fwd), ("fwd_bwd", step, f_fwd + f_bwd, b_fb)):
            ms = med_ms(fn)
            out[key] = {"median_ms": ms, "tflops": fl / (ms * 1e-3) / 1e12, "gbps_io": by / (ms * 1e-3) / 1e9,
                        "roofline_frac": max(fl / PEAK_FP32_MFMA, by / PEAK_HBM) / (ms * 1e-3)}
        pf, pfb = PAGE_CHUNKED_MS[(name, T)]
        out["page_chunked_rtx3090_ms"] = {"fwd": pf, "fwd_bwd": pfb}
        out["dtype"] = "f32"
        out["data"] = "synthetic"
        print(json.dumps(out), flush=True)
        del d, ws, y, grads
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed steps first; the GPU needs some 20 ms of work to reach its working clocks")
    ap.add_argument("--workload", default="g2h8_d128_T8192")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-reuse", action="store_true",
                    help="skip the secondary fwd + bwd_from_fwd timing (profiling runs: its reverse-only "
                         "state scan shares the forward scan's kernel name and grid)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (5 launches) and exit")
    ap.add_argument("--max-len", action="store_true",
                    help="only run the T-doubling maximum-length search for fwd_bwd and exit")
    ap.add_argument("--max-len-cap", type=int, default=1 << 22, help="largest T the search tries")
    ap.add_argument("--grid", action="store_true",
                    help="only time fwd and fwd_bwd at every shape of the pages' grid, one JSON line each, and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "this build has no multi-GPU path", file=sys.stderr)
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

    def fwd():
        ssd.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], out=y, workspace=ws)

    def bwd():
        ssd.bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], d["dy"], out=grads, workspace=ws)

    def step():
        fwd()
        bwd()

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
        with_kernels = kernels is None or len(kernels) > 0
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        if with_kernels:
            kt = ssd.kernel_timing(kernels).__enter__()
        evs[0].record()
        for i in range(K):
            fn()
            if per_step or i == K - 1:
                evs[i + 1].record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - wall0) * 1e3
        if with_kernels:
            kt.__exit__(None, None, None)
        per = [evs[i].elapsed_time(evs[i + 1]) for i in range(K)] if per_step else []
        total = evs[0].elapsed_time(evs[K])
        return total / K, per, wall / K, (kt.results if with_kernels else None)

    K = args.steps
    # Per-kernel pass (not the headline): K steps with every kernel timed by
    # events bound to its dispatch, for the per-kernel table and to find the
    # dominant kernel.  Each timed dispatch costs a few microseconds of stream
    # time, so the headline region below times the dominant kernel only.
    _, _, _, kern_all = timed(step, K, kernels=None)
    dom = max((n for n in kern_all if kern_all[n][1]), key=lambda n: kern_all[n][0])
    # Timed region: exactly K steps between two events; the dominant kernel's
    # launches carry HIP events on the launch stream, for its roofline.
    step_ms, _, wall_ms, kern_dom = timed(step, K, kernels=[dom], per_step=False)
    # The per-step distribution (median, quartiles) comes from a pass of its
    # own with an event after every step.
    _, per_step, _, _ = timed(step, K)
    fwd_ms, fwd_per, _, _ = timed(fwd, K)
    bwd_ms, bwd_per, _, _ = timed(bwd, K)

    # Secondary (not the headline): the backward that reuses the forward's
    # residuals from the shared workspace instead of recomputing them.
    def step_reuse():
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
        a = amt / (kernels[name]["avg_us"] * 1e-6)
        kernels[name]["achieved"] = a / 1e12 if bnd == "mfma" else a / 1e9
        kernels[name]["unit"] = "TFLOP/s" if bnd == "mfma" else "GB/s"
        kernels[name]["frac"] = a / (PEAK_FP32_MFMA if bnd == "mfma" else PEAK_HBM)

    cpu = None
    parity = None
    if not args.no_cpu:
        # CPU baseline: the fp64 oracle on the whole workload, on the host cores.
        import oracle
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ref_y = oracle.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])
        ref = oracle.bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], x["dy"])
        cpu_s = time.perf_counter() - t0
        cpu = {"value": (f_fwd + f_bwd) / cpu_s / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
               "kind": "oracle", "seconds": cpu_s, "cpu_model": cpu_info(),
               "sample": f"whole {w.name} workload, one fwd + bwd in fp64 (nominal FLOPs / wall time)"}
        # parity of the last timed GPU step against the oracle (whole tensors)
        fwd()
        bwd()
        torch.cuda.synchronize()
        parity = {"y": rel_err(y.cpu().numpy(), ref_y)}
        for name, t in zip(("dq", "dk", "dv", "dlog_alpha", "dh0"), grads):
            parity[name] = rel_err(t.cpu().numpy(), ref[name])

    def q(vals):
        a = np.asarray(vals)
        return {"median_ms": float(np.median(a)), "q1_ms": float(np.percentile(a, 25)),
                "q3_ms": float(np.percentile(a, 75))}

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
        "vs_baseline": (PAGE_FWD_BWD_MS / step_ms) if w.name == "g2h8_d128_T8192" else None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={s.B} G={s.G} H={s.H} T={s.T} dk={s.dk} dv={s.dv}, "
                               "step = ssd_fwd + ssd_bwd", "chunk": 64, "seed": w.seed},
        "roofline": roof,
        "cpu_baseline": cpu,
        "fwd_bwd": {**q(per_step), "tflops": value, "roofline_frac": t_roof_fb / (step_ms * 1e-3),
                    "gbps_io": b_fwd_bwd / (step_ms * 1e-3) / 1e9, "wall_ms": wall_ms},
        "fwd": {**q(fwd_per), "ms": fwd_ms, "tflops": f_fwd / (fwd_ms * 1e-3) / 1e12,
                "roofline_frac": t_roof_f / (fwd_ms * 1e-3), "gbps_io": b_fwd / (fwd_ms * 1e-3) / 1e9},
        "bwd": {**q(bwd_per), "ms": bwd_ms, "tflops": f_bwd / (bwd_ms * 1e-3) / 1e12},
        "fwd_bwd_reuse": None if reuse_ms is None else {**q(reuse_per), "ms": reuse_ms,
                          "note": "secondary: ssd_fwd then ssd_bwd_from_fwd, which reuses the forward's "
                                  "chunk states from the workspace (not the stateless headline step)"},
        "kernels": kernels,
        "parity_rel_err": parity,
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
