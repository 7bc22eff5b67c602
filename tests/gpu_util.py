"""Helpers shared by the GPU tests: device transfer and the HIP path calls."""
import sys

import numpy as np
import pytest


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def say(msg):
    """Name the case before a GPU step, flushed, so a crash still shows it."""
    print(msg, file=sys.stderr, flush=True)


def to_dev(x: dict):
    import torch
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda") for k, v in x.items()}


def hip_fwd(d):
    import chunked_ssd_scan_fwd_amd as ssd
    return ssd.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"])


def hip_bwd(d):
    import chunked_ssd_scan_fwd_amd as ssd
    dq, dk, dv, dla, dh0 = ssd.bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], d["dy"])
    return {"dq": dq, "dk": dk, "dv": dv, "dlog_alpha": dla, "dh0": dh0}


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()
