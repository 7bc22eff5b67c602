"""GPU parity of the selective (Mamba-style) scan: the HIP path (mamba_fwd
through the C ABI) against the fp64 oracle, rel_err = max|out - ref| /
max|ref| over the whole tensor, y <= 2e-5."""
import numpy as np
import pytest

from oracle import mamba as mo
from ssd_workload import rel_err
from ssd_workload.mamba import MambaShape, MAMBA_GRID, make_mamba_inputs
from gpu_util import need_gpu, say, host

pytestmark = pytest.mark.gpu

TOL_Y = 2e-5
ARGS = ("x", "delta", "A", "B", "C", "Dskip")


def _dev(inp):
    import torch
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda") for k, v in inp.items()}


def _fwd(d, **kw):
    import chunked_ssd_scan_fwd_amd as ssd
    return ssd.mamba_fwd(*(d[k] for k in ARGS), **kw)


def _id(s):
    return f"B{s.B}L{s.L}D{s.D}N{s.N}"


# A channel count that is not a multiple of the 256-channel block, fewer
# states than 16, one step, one channel, and sequences cut into segments.
SHAPES = [MambaShape(1, 1, 3, 16), MambaShape(1, 9, 1, 1), MambaShape(3, 77, 5, 7), MambaShape(2, 1000, 100, 16),
          MambaShape(2, 4096, 64, 16), MambaShape(1, 3001, 300, 11), MambaShape(4, 512, 256, 16),
          MambaShape(4, 2048, 512, 16)]


@pytest.mark.parametrize("shape", SHAPES, ids=_id)
def test_mamba_forward(shape):
    need_gpu()
    say(f"mamba fwd {_id(shape)}")
    inp = make_mamba_inputs(shape, seed=shape.L + shape.D)
    y = host(_fwd(_dev(inp)))
    assert rel_err(y, mo.fwd(*(inp[k] for k in ARGS))) <= TOL_Y


def test_mamba_forward_page_largest():
    """The page's largest point, dim 1024 and seq 8192 at batch 4, state 16:
    the whole tensor against the oracle."""
    need_gpu()
    s = MAMBA_GRID[(1024, 8192)]
    say(f"mamba fwd {_id(s)}")
    inp = make_mamba_inputs(s, seed=77)
    y = host(_fwd(_dev(inp)))
    assert rel_err(y, mo.fwd(*(inp[k] for k in ARGS))) <= TOL_Y


def test_mamba_forward_strong_and_weak_decay():
    need_gpu()
    s = MambaShape(2, 2000, 128, 16)
    for scale in (0.01, 20.0):
        say(f"mamba fwd decay scale {scale}")
        inp = make_mamba_inputs(s, seed=3)
        inp["delta"] = (inp["delta"] * scale).astype(np.float32)
        y = host(_fwd(_dev(inp)))
        assert rel_err(y, mo.fwd(*(inp[k] for k in ARGS))) <= TOL_Y, scale


def test_mamba_forward_deterministic_and_inputs_untouched():
    need_gpu()
    s = MambaShape(2, 3000, 256, 16)
    say("mamba determinism")
    inp = make_mamba_inputs(s, seed=5)
    d = _dev(inp)
    y1, y2 = host(_fwd(d)), host(_fwd(d))
    np.testing.assert_array_equal(y1, y2)
    for k in ARGS:
        np.testing.assert_array_equal(host(d[k]), inp[k])


def test_mamba_empty_and_refused():
    need_gpu()
    import torch
    import chunked_ssd_scan_fwd_amd as ssd
    say("mamba empty / refused")
    for s in (MambaShape(0, 10, 4, 16), MambaShape(2, 0, 4, 16)):
        y = _fwd(_dev(make_mamba_inputs(s, 1)))
        assert tuple(y.shape) == (s.B, s.L, s.D)
    big = _dev(make_mamba_inputs(MambaShape(1, 4, 2, 17), 1))
    with pytest.raises(ssd.SsdError):
        _fwd(big)
    # a short caller workspace is refused before anything runs
    s = MambaShape(2, 4096, 64, 16)
    d = _dev(make_mamba_inputs(s, 1))
    need = ssd.mamba_workspace_size(ssd.MambaShapeArg(s.B, s.L, s.D, s.N))
    assert need > 0
    with pytest.raises(ValueError):
        _fwd(d, workspace=torch.empty(need - 1, dtype=torch.uint8, device="cuda"))
