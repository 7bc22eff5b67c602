"""Compile the HIP library (gfx950) in-tree with hipcc.

Each source is compiled to an object of its own, in parallel, and the
objects are linked into ``libssd_hip.so`` next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libssd_hip.so")
# benchmark-only device probes (MFMA loop, shader clock), a library of their own
PROBE_LIB = os.path.join(PKG, "libssd_probe.so")
OBJDIR = os.path.join(ROOT, "_build")
SOURCES = ["ssd_api.hip", "k_scan.hip", "k_output.hip", "k_pair.hip", "k_grads.hip", "k_mamba.hip", "ssd_validate.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), file=sys.stderr, flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + proc.stdout + proc.stderr)
    return proc


def build(verbose: bool = False, extra=(), jobs: int | None = None) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([HIPCC, *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    probe_obj = os.path.join(OBJDIR, "probe.o")
    cmds.append([HIPCC, *FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, "probe.hip"), "-o", probe_obj])
    n = jobs or min(len(cmds), max(1, (os.cpu_count() or 4)))
    with ThreadPoolExecutor(max_workers=n) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", probe_obj, "-o", PROBE_LIB + ".tmp"], verbose)
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
