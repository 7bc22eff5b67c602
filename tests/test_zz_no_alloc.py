"""ssd_fwd_noalloc, the forward that allocates nothing (its workspace is the
library's static per-device array), against ssd_fwd through the C ABI."""
import ctypes

import numpy as np
import pytest

import oracle
from ssd_workload import Shape, make_inputs, rel_err
from gpu_util import need_gpu, say, to_dev, host

TOL_Y = 2e-5


def _call(fn, s, d, y):
    import torch
    import chunked_ssd_scan_fwd_amd as ssd
    lib = ssd.library()
    sa = ssd.ShapeArg(s.B, s.G, s.H, s.T, s.dk, s.dv)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if fn == "ssd_fwd_noalloc":
        return lib.ssd_fwd_noalloc(ctypes.byref(sa), p(d["q"]), p(d["k"]), p(d["v"]), p(d["log_alpha"]),
                                   p(d["h0"]), p(y), st)
    ws = torch.empty(max(1, ssd.workspace_size(sa, False)), dtype=torch.uint8, device="cuda")
    rc = lib.ssd_fwd(ctypes.byref(sa), p(d["q"]), p(d["k"]), p(d["v"]), p(d["log_alpha"]), p(d["h0"]), p(y),
                     p(ws), ctypes.c_size_t(ws.numel()), st)
    torch.cuda.synchronize()
    return rc


@pytest.mark.gpu
def test_noalloc_matches_fwd_twice_second_smaller():
    """Two calls in a row, the second on a smaller problem (the array keeps the
    first call's contents): each equals ssd_fwd's output and meets the bar
    against the oracle."""
    need_gpu()
    import torch
    for s, seed in ((Shape(2, 2, 8, 1000, 128, 128), 31), (Shape(1, 2, 4, 130, 48, 40), 32)):
        say(f"noalloc B{s.B}G{s.G}H{s.H}T{s.T}dk{s.dk}dv{s.dv}")
        x = make_inputs(s, seed)
        d = to_dev(x)
        y0 = torch.full((s.B, s.H, s.T, s.dv), float("nan"), device="cuda")
        y1 = torch.full((s.B, s.H, s.T, s.dv), float("nan"), device="cuda")
        assert _call("ssd_fwd", s, d, y0) == 0
        assert _call("ssd_fwd_noalloc", s, d, y1) == 0
        a, b = host(y0), host(y1)
        np.testing.assert_array_equal(b, a)
        assert rel_err(b, oracle.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])) <= TOL_Y


@pytest.mark.gpu
def test_noalloc_binding_and_size_limit():
    """The binding's fwd_noalloc gives the same y; a shape whose workspace
    exceeds the static array is refused before anything is enqueued."""
    need_gpu()
    import torch
    import chunked_ssd_scan_fwd_amd as ssd
    s = Shape(1, 1, 3, 257, 64, 64)
    x = make_inputs(s, 33)
    d = to_dev(x)
    say("noalloc binding")
    y = ssd.fwd_noalloc(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"])
    y0 = ssd.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"])
    np.testing.assert_array_equal(host(y), host(y0))
    big = ssd.ShapeArg(4, 2, 8, 8192, 128, 128)
    assert ssd.workspace_size(big, False) > ssd.NOALLOC_WORKSPACE_BYTES
    lib = ssd.library()
    p = ctypes.c_void_p(16)
    assert lib.ssd_fwd_noalloc(ctypes.byref(big), *([p] * 6), None) == 4
