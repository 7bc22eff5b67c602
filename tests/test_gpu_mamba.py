"""GPU parity of the selective (Mamba-style) scan: the HIP path (mamba_fwd,
mamba_bwd and mamba_fwd_bwd through the C ABI) against the fp64 oracle,
rel_err = max|out - ref| / max|ref| over the whole tensor, y <= 2e-5 and
each of the six gradients <= 5e-5."""
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


TOL_G = 5e-5
GRADS = ("dx", "ddelta", "dA", "dB", "dC", "dD")


def _bwd(d, **kw):
    import chunked_ssd_scan_fwd_amd as ssd
    return ssd.mamba_bwd(*(d[k] for k in ARGS), d["dy"], **kw)


def _check_bwd(shape, seed, scale=1.0):
    inp = make_mamba_inputs(shape, seed=seed)
    if scale != 1.0:
        inp["delta"] = (inp["delta"] * scale).astype(np.float32)
    g = [host(t) for t in _bwd(_dev(inp))]
    ref = mo.bwd(*(inp[k] for k in ARGS), inp["dy"])
    errs = {k: rel_err(a, ref[k]) for a, k in zip(g, GRADS)}
    bad = {k: e for k, e in errs.items() if not e <= TOL_G}
    assert not bad, f"gradient rel_err over bar: {bad}"


# one step, one channel, fewer states than 16, channels not a multiple of the
# 32-channel block, a ragged last segment, several channel splits per segment
BWD_SHAPES = [MambaShape(1, 1, 3, 16), MambaShape(1, 9, 1, 1), MambaShape(3, 77, 5, 7), MambaShape(2, 1000, 100, 16),
              MambaShape(2, 4096, 64, 16), MambaShape(1, 3001, 300, 11), MambaShape(4, 512, 256, 16),
              MambaShape(4, 2048, 512, 16)]


@pytest.mark.parametrize("shape", BWD_SHAPES, ids=_id)
def test_mamba_backward(shape):
    need_gpu()
    say(f"mamba bwd {_id(shape)}")
    _check_bwd(shape, seed=shape.L + 3 * shape.D)


def test_mamba_backward_page_largest():
    need_gpu()
    s = MAMBA_GRID[(1024, 8192)]
    say(f"mamba bwd {_id(s)}")
    _check_bwd(s, seed=78)


def test_mamba_backward_strong_and_weak_decay():
    need_gpu()
    s = MambaShape(2, 2000, 128, 16)
    for scale in (0.01, 20.0):
        say(f"mamba bwd decay scale {scale}")
        _check_bwd(s, seed=4, scale=scale)


def test_mamba_backward_deterministic_and_empty():
    need_gpu()
    import torch
    say("mamba bwd determinism / empty")
    s = MambaShape(2, 3000, 256, 16)
    d = _dev(make_mamba_inputs(s, 6))
    g1 = [host(t) for t in _bwd(d)]
    g2 = [host(t) for t in _bwd(d)]
    for a, b in zip(g1, g2):
        np.testing.assert_array_equal(a, b)
    for e in (MambaShape(0, 10, 4, 16), MambaShape(2, 0, 4, 16)):
        g = [host(t) for t in _bwd(_dev(make_mamba_inputs(e, 1)))]
        assert not np.any(g[2]) and not np.any(g[5])   # dA and dDskip are zero


@pytest.mark.parametrize("shape", [MambaShape(1, 9, 1, 1), MambaShape(3, 77, 5, 7), MambaShape(2, 1000, 100, 16),
                                   MambaShape(4, 512, 256, 16), MambaShape(4, 2048, 512, 16)], ids=_id)
def test_mamba_fwd_bwd(shape):
    """y and the gradients in one call: y against the oracle, the gradients
    bit for bit those of mamba_bwd."""
    need_gpu()
    import chunked_ssd_scan_fwd_amd as ssd
    say(f"mamba fwd_bwd {_id(shape)}")
    inp = make_mamba_inputs(shape, seed=shape.L + 5 * shape.D)
    d = _dev(inp)
    out = [host(t) for t in ssd.mamba_fwd_bwd(*(d[k] for k in ARGS), d["dy"])]
    assert rel_err(out[0], mo.fwd(*(inp[k] for k in ARGS))) <= TOL_Y
    for a, b in zip(out[1:], [host(t) for t in _bwd(d)]):
        np.testing.assert_array_equal(a, b)
    ref = mo.bwd(*(inp[k] for k in ARGS), inp["dy"])
    for a, k in zip(out[1:], GRADS):
        assert rel_err(a, ref[k]) <= TOL_G, k


def test_mamba_poisoned_workspace_and_outputs():
    """Every output is written whole and no kernel reads workspace it has not
    written: NaN-filled workspaces and outputs leave the results unchanged."""
    need_gpu()
    import torch
    import chunked_ssd_scan_fwd_amd as ssd
    say("mamba poisoned workspace / outputs")
    for s in (MambaShape(2, 1000, 100, 11), MambaShape(4, 512, 256, 16)):
        inp = make_mamba_inputs(s, seed=9)
        d = _dev(inp)
        args = [d[k] for k in ARGS]
        sa = ssd.MambaShapeArg(s.B, s.L, s.D, s.N)
        clean_y = host(ssd.mamba_fwd(*args))
        clean_g = [host(t) for t in ssd.mamba_fwd_bwd(*args, d["dy"])]
        nan = float("nan")
        wsf = torch.full((max(1, ssd.mamba_workspace_size(sa)) // 4 + 1,), nan, device="cuda")
        wsb = torch.full((max(1, ssd.mamba_workspace_size(sa, True)) // 4 + 1,), nan, device="cuda")
        y = torch.full((s.B, s.L, s.D), nan, device="cuda")
        np.testing.assert_array_equal(host(ssd.mamba_fwd(*args, out=y, workspace=wsf)), clean_y)
        outs = tuple(torch.full_like(t, nan) for t in ssd.mamba_fwd_bwd(*args, d["dy"]))
        got = [host(t) for t in ssd.mamba_fwd_bwd(*args, d["dy"], out=outs, workspace=wsb)]
        for a, b in zip(got, clean_g):
            np.testing.assert_array_equal(a, b)


def _random_mamba_shapes(n=12, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        out.append(MambaShape(int(rng.integers(1, 5)), int(rng.integers(1, 3000)), int(rng.integers(1, 700)),
                              int(rng.integers(1, 17))))
    return out


@pytest.mark.parametrize("shape", _random_mamba_shapes(), ids=_id)
def test_mamba_random_shapes(shape):
    """A seeded sweep of shapes (batch 1-4, seq up to 3000, dim up to 700,
    1-16 states): mamba_fwd, mamba_bwd and mamba_fwd_bwd against the oracle."""
    need_gpu()
    import chunked_ssd_scan_fwd_amd as ssd
    say(f"mamba random {_id(shape)}")
    inp = make_mamba_inputs(shape, seed=shape.L * 7 + shape.D)
    d = _dev(inp)
    ref_y = mo.fwd(*(inp[k] for k in ARGS))
    ref = mo.bwd(*(inp[k] for k in ARGS), inp["dy"])
    assert rel_err(host(_fwd(d)), ref_y) <= TOL_Y
    g = [host(t) for t in _bwd(d)]
    for a, k in zip(g, GRADS):
        assert rel_err(a, ref[k]) <= TOL_G, k
    both = [host(t) for t in ssd.mamba_fwd_bwd(*(d[k] for k in ARGS), d["dy"])]
    assert rel_err(both[0], ref_y) <= TOL_Y
    for a, b in zip(both[1:], g):
        np.testing.assert_array_equal(a, b)
