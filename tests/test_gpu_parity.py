"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar (rel_err = max|out - ref| / max|ref| over the whole tensor):
y <= 2e-5, each of dq, dk, dv, dlog_alpha, dh0 <= 5e-5.
"""
import numpy as np
import pytest

import oracle
from ssd_workload import Shape, make_inputs, rel_err, WORKLOADS, workload
from gpu_util import need_gpu, say, to_dev, hip_fwd, hip_bwd, host

pytestmark = pytest.mark.gpu

TOL_Y = 2e-5
TOL_G = 5e-5
GRADS = ("dq", "dk", "dv", "dlog_alpha", "dh0")

ZOO = [
    Shape(1, 1, 1, 1, 1, 1),
    Shape(2, 1, 1, 2, 3, 5),
    Shape(1, 2, 4, 17, 48, 40),
    Shape(2, 2, 4, 63, 128, 128),
    Shape(1, 1, 3, 65, 128, 64),
    Shape(2, 3, 6, 100, 64, 32),
    Shape(1, 1, 1, 200, 128, 1),
    Shape(1, 2, 2, 130, 1, 128),
    Shape(2, 2, 8, 256, 128, 128),
    Shape(1, 1, 24, 300, 128, 64),
    Shape(3, 1, 2, 129, 33, 97),
    # fewer (b, g, chunk) blocks than CUs: the output and gradient kernels split
    # a group's heads over blocks, here unevenly (2 + 2 + 1 and 2 + 2 + 2 + 1)
    Shape(2, 2, 10, 1024, 48, 40),
    Shape(1, 1, 7, 4096, 64, 64),
    # more (b, g, chunk, head split) units than CUs with a head split: the
    # output and gradient kernels' blocks walk two units each, of different
    # splits (200 chunks x 2 splits = 400 units on a 256-block grid)
    Shape(1, 1, 4, 12793, 64, 64),
]


# dk or dv in 129..256: column-block sub-problems added up in a fixed order
WIDE = [
    Shape(1, 1, 2, 300, 256, 256),
    Shape(2, 2, 4, 150, 200, 136),
    Shape(1, 1, 1, 70, 129, 1),
    Shape(1, 2, 2, 100, 1, 250),
    Shape(2, 1, 3, 65, 136, 200),
]


def _id(s):
    return f"B{s.B}G{s.G}H{s.H}T{s.T}dk{s.dk}dv{s.dv}"


def check_fwd(x, tol=TOL_Y):
    d = to_dev(x)
    y = host(hip_fwd(d))
    ref = oracle.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])
    e = rel_err(y, ref)
    assert e <= tol, f"y rel_err {e:.3e}"
    return e


def check_bwd(x, tol=TOL_G):
    d = to_dev(x)
    g = {k: host(v) for k, v in hip_bwd(d).items()}
    ref = oracle.bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], x["dy"])
    errs = {k: rel_err(g[k], ref[k]) for k in GRADS}
    bad = {k: e for k, e in errs.items() if not e <= tol}
    assert not bad, f"gradient rel_err over bar: {bad}"
    return errs


@pytest.mark.parametrize("shape", ZOO, ids=_id)
def test_forward_shape_zoo(shape):
    need_gpu()
    say(f"fwd {_id(shape)}")
    check_fwd(make_inputs(shape, seed=shape.T * 7 + shape.dk))


@pytest.mark.parametrize("shape", ZOO, ids=_id)
def test_backward_shape_zoo(shape):
    need_gpu()
    say(f"bwd {_id(shape)}")
    check_bwd(make_inputs(shape, seed=shape.T * 11 + shape.dv))


@pytest.mark.parametrize("shape", WIDE, ids=_id)
def test_wide_dims_forward_backward(shape):
    need_gpu()
    say(f"wide {_id(shape)}")
    x = make_inputs(shape, seed=shape.T * 5 + shape.dk + shape.dv)
    check_fwd(x)
    check_bwd(x)


def test_wide_dims_reuse_noalloc_deterministic():
    """A split shape through bwd_from_fwd (which recomputes for such shapes),
    fwd_noalloc, and two runs of each call: all equal bitwise."""
    need_gpu()
    import torch
    import chunked_ssd_scan_fwd_amd as ssd
    s = Shape(1, 2, 4, 200, 160, 144)
    x = make_inputs(s, 41)
    d = to_dev(x)
    say("wide reuse / noalloc")
    sa = ssd.ShapeArg(s.B, s.G, s.H, s.T, s.dk, s.dv)
    ws = torch.empty(ssd.workspace_size(sa, True), dtype=torch.uint8, device="cuda")
    y = host(ssd.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], workspace=ws))
    g1 = ssd.bwd_from_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], d["dy"], workspace=ws)
    g2 = ssd.bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], d["dy"])
    y2 = host(ssd.fwd_noalloc(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"]))
    np.testing.assert_array_equal(y2, y)
    for a, b in zip(g1, g2):
        np.testing.assert_array_equal(host(a), host(b))
    assert rel_err(y, oracle.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])) <= TOL_Y


@pytest.mark.parametrize("shape", [Shape(2, 2, 4, 300, 48, 40), Shape(1, 1, 2, 1500, 64, 64),
                                   Shape(1, 1, 1, 2048, 128, 128), Shape(1, 1, 2, 65536, 128, 128)], ids=_id)
def test_chunk_states_match_oracle(shape):
    """Step-level check: the state entering each chunk that ssd_fwd leaves
    in the workspace (every chunk, or every even one when the forward runs
    on chunk pairs, as ssd_fwd_state_stride says) against the oracle's state
    at the chunk boundary.  The last three shapes fill few CUs, so their
    scan runs in chunk segments joined by the fix-up passes; the last one
    runs on chunk pairs on a 256-CU device."""
    need_gpu()
    import torch
    import chunked_ssd_scan_fwd_amd as ssd
    x = make_inputs(shape, seed=5)
    d = to_dev(x)
    sa = ssd.ShapeArg(shape.B, shape.G, shape.H, shape.T, shape.dk, shape.dv)
    ws = torch.empty(ssd.workspace_size(sa, False), dtype=torch.uint8, device="cuda")
    say(f"chunk states {_id(shape)}")
    ssd.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], workspace=ws)
    off = ssd.workspace_layout(sa, False)
    NC = (shape.T + 63) // 64
    E = shape.dk * shape.dv
    Epad = (E + 63) // 64 * 64
    st = host(ws[off[1]:off[1] + shape.B * shape.H * NC * Epad * 4].view(torch.float32))
    st = st.reshape(shape.B, shape.H, NC, Epad)[..., :E].reshape(shape.B, shape.H, NC, shape.dk, shape.dv)
    _, ref = oracle.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], chunk=64)
    held = list(range(0, NC, ssd.fwd_state_stride(sa)))
    assert rel_err(st[:, :, held], ref[:, :, held]) <= TOL_Y
    # per chunk as well: a state that decays to nothing would hide in the
    # whole-tensor maximum (the within-chunk cumulative log-decay that weighs
    # every contribution is checked through these)
    for c in held:
        assert rel_err(st[:, :, c], ref[:, :, c]) <= 1e-4, c
    # the per-chunk cumulative log-decay, as the decay weights the scan applies:
    # e^{b_L - b_t}, e^{b_t} per position and e^{b_L} per chunk, against the
    # fp64 cumulative sums of the same log_alpha (positions past T add 0)
    BH = shape.B * shape.H
    wts = host(ws[off[0]:off[0] + BH * NC * 128 * 4].view(torch.float32)).reshape(BH, NC, 2, 64)
    cd0 = (BH * NC * 128 * 4 + 255) // 256 * 256
    cdec = host(ws[cd0:cd0 + BH * NC * 4].view(torch.float32)).reshape(BH, NC)
    la = np.zeros((BH, NC * 64))
    la[:, :shape.T] = x["log_alpha"].reshape(BH, shape.T)
    b = np.cumsum(la.reshape(BH, NC, 64), axis=-1)
    bL = b[..., -1:]
    assert rel_err(wts[:, :, 0], np.exp(bL - b)) <= 1e-5
    assert rel_err(wts[:, :, 1], np.exp(b)) <= 1e-5
    assert rel_err(cdec, np.exp(bL[..., 0])) <= 1e-5


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_workload_full_size(idx):
    """Full-size parity on all five workloads, whole tensors (the pages'
    rel_err is a whole-tensor metric)."""
    need_gpu()
    w = WORKLOADS[idx]
    say(f"workload {w.name}")
    x = make_inputs(w.shape, w.seed, mu=w.mu)
    check_fwd(x)
    check_bwd(x)


# Shapes whose forward runs on chunk pairs (128-column states, at least two
# pairs per CU on a 256-CU device): an odd chunk count with a ragged tail,
# padded dk and dv (16-byte and 4-byte addressing), dk = 32, eight heads.
PAIRS = [Shape(2, 2, 4, 32700, 128, 128), Shape(1, 2, 4, 32805, 100, 96), Shape(1, 2, 2, 32768, 32, 97),
         Shape(1, 1, 8, 65536, 64, 128)]


@pytest.mark.parametrize("shape", PAIRS, ids=_id)
def test_chunk_pair_forward(shape):
    """The forward on chunk pairs against the oracle, whole tensor, and the
    backward that reuses its workspace (which then forms the odd chunks'
    states) against the oracle and the stateless backward."""
    need_gpu()
    import torch
    import chunked_ssd_scan_fwd_amd as ssd
    sa = ssd.ShapeArg(shape.B, shape.G, shape.H, shape.T, shape.dk, shape.dv)
    if ssd.fwd_state_stride(sa) != 2:
        pytest.skip("this device's compute-unit count does not put the shape on chunk pairs")
    say(f"chunk pairs {_id(shape)}")
    x = make_inputs(shape, seed=11 + shape.dv)
    d = to_dev(x)
    ws = torch.empty(ssd.workspace_size(sa, True), dtype=torch.uint8, device="cuda")
    y = ssd.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], workspace=ws)
    assert rel_err(host(y), oracle.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])) <= TOL_Y
    g = ssd.bwd_from_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], d["dy"], workspace=ws)
    g0 = ssd.bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], d["dy"])
    ref = oracle.bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], x["dy"])
    for t, t0, name in zip(g, g0, GRADS):
        a = host(t)
        assert rel_err(a, ref[name]) <= TOL_G, name
        assert rel_err(a, host(t0)) <= 1e-6, name


# The forward at chunk 64 and at chunk 128 (SSD_FWD_CHUNK) on the same
# inputs: 64-column states, one chunk (a pair without its odd chunk), padded
# dk and dv with 16- and 4-byte addressing and an odd chunk count, a group's
# heads split over blocks (fewer pair units than CUs), and a scan in chunk
# segments.
CHUNK_LENGTHS = [Shape(2, 2, 4, 300, 48, 40), Shape(1, 1, 3, 65, 128, 64), Shape(2, 2, 4, 63, 128, 128),
                 Shape(1, 2, 4, 1000, 100, 96), Shape(3, 1, 2, 129, 33, 97), Shape(1, 1, 7, 4096, 64, 64),
                 Shape(1, 1, 2, 16384, 128, 128)]


@pytest.mark.parametrize("shape", CHUNK_LENGTHS, ids=_id)
def test_forward_chunk_length_invariance(shape, monkeypatch):
    """The chunked method's result does not depend on its chunk length beyond
    rounding: the forward at chunk 64 and at chunk 128 (chunk pairs) agree
    with the oracle and with each other, and the backward that reuses each
    forward's workspace agrees with the oracle and the stateless backward."""
    need_gpu()
    import torch
    import chunked_ssd_scan_fwd_amd as ssd
    x = make_inputs(shape, seed=23 + shape.T)
    d = to_dev(x)
    sa = ssd.ShapeArg(shape.B, shape.G, shape.H, shape.T, shape.dk, shape.dv)
    ref_y = oracle.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])
    ref = oracle.bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], x["dy"])
    say(f"chunk lengths {_id(shape)}: stateless backward")
    g0 = [host(t) for t in ssd.bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], d["dy"])]
    ys = {}
    for val, stride in (("64", 1), ("128", 2)):
        monkeypatch.setenv("SSD_FWD_CHUNK", val)
        say(f"chunk lengths {_id(shape)}: forward chunk {val}")
        assert ssd.fwd_state_stride(sa) == stride
        ws = torch.empty(ssd.workspace_size(sa, True), dtype=torch.uint8, device="cuda")
        ys[val] = host(ssd.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], workspace=ws))
        assert rel_err(ys[val], ref_y) <= TOL_Y, val
        g = ssd.bwd_from_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], d["dy"], workspace=ws)
        for t, t0, name in zip(g, g0, GRADS):
            a = host(t)
            assert rel_err(a, ref[name]) <= TOL_G, (val, name)
            assert rel_err(a, t0) <= 1e-6, (val, name)
    assert rel_err(ys["128"], ys["64"]) <= 5e-6


@pytest.mark.parametrize("T", [65536, 131072])
def test_long_sequence_unit(T):
    """One independent unit at the headline's head and state sizes (B=1, G=1,
    H=4, dk=dv=128), far beyond the workloads' T: the GPU page's chunked path
    reaches T = 65536 at most (kernel_ssd_gpu.json, max_len record).  The
    whole tensors of y and of all five gradients against the oracle."""
    need_gpu()
    s = Shape(1, 1, 4, T, 128, 128)
    say(f"long sequence T={T}")
    x = make_inputs(s, seed=4000 + T // 65536)
    check_fwd(x)
    check_bwd(x)


def test_headline_identities_full_size():
    """Properties that hold at any size, checked on the whole headline problem:
    <q,dq> = L, <k,dk> = <v,dv> = L - <h0,dh0>, dlog_alpha[:,:,0] = <h0,dh0> per head."""
    need_gpu()
    w = workload("g2h8_d128_T8192")
    say("headline identities")
    x = make_inputs(w.shape, w.seed, mu=w.mu)
    d = to_dev(x)
    y = host(hip_fwd(d)).astype(np.float64)
    g = {k: host(v).astype(np.float64) for k, v in hip_bwd(d).items()}
    L = float(np.sum(x["dy"].astype(np.float64) * y))
    h0t = float(np.sum(x["h0"].astype(np.float64) * g["dh0"]))
    scale = float(np.sum(np.abs(x["dy"].astype(np.float64) * y)))
    assert abs(np.sum(x["q"] * g["dq"]) - L) <= 1e-5 * scale
    assert abs(np.sum(x["k"] * g["dk"]) - (L - h0t)) <= 1e-5 * scale
    assert abs(np.sum(x["v"] * g["dv"]) - (L - h0t)) <= 1e-5 * scale
    per_head = np.sum(x["h0"] * g["dh0"], axis=(2, 3))
    assert rel_err(g["dlog_alpha"][:, :, 0], per_head) <= 1e-4


def test_zero_decay_no_h0():
    need_gpu()
    s = Shape(2, 2, 4, 150, 64, 64)
    x = make_inputs(s, 3)
    x["log_alpha"][:] = 0.0
    x["h0"][:] = 0.0
    say("zero decay")
    check_fwd(x)
    check_bwd(x)


def test_strong_decay():
    need_gpu()
    s = Shape(1, 1, 2, 130, 32, 32)
    x = make_inputs(s, 4)
    x["log_alpha"][:] = -80.0
    say("strong decay")
    check_fwd(x)
    check_bwd(x)


def test_large_within_chunk_exponents():
    """Decay steady at log_alpha = -3: the cumulative exponents reach -192
    inside a chunk while neighbouring positions still weigh e^-3. Rounding b
    itself (b log2(e) stored per position, say) instead of the difference
    b_i - b_j shows up here, in dlog_alpha first."""
    need_gpu()
    s = Shape(1, 1, 2, 130, 64, 64)
    x = make_inputs(s, 6)
    x["log_alpha"][:] = -3.0
    say("steady decay -3")
    check_fwd(x)
    check_bwd(x)


def test_group_replication_matches():
    """Replicating q, k to one group per head gives the grouped result."""
    need_gpu()
    s = Shape(2, 2, 8, 140, 128, 128)
    x = make_inputs(s, 8)
    idx = np.arange(s.H) // s.hpg
    xr = dict(x)
    xr["q"] = np.ascontiguousarray(x["q"][:, idx])
    xr["k"] = np.ascontiguousarray(x["k"][:, idx])
    say("group replication")
    d, dr = to_dev(x), to_dev(xr)
    y, yr = host(hip_fwd(d)), host(hip_fwd(dr))
    assert rel_err(yr, y) <= TOL_Y
    g, gr = hip_bwd(d), hip_bwd(dr)
    dq = host(g["dq"])
    dqr = host(gr["dq"]).reshape(s.B, s.G, s.hpg, s.T, s.dk).sum(axis=2)
    assert rel_err(dqr, dq) <= TOL_G


def test_deterministic():
    need_gpu()
    s = Shape(2, 2, 8, 257, 128, 128)
    x = make_inputs(s, 9)
    d = to_dev(x)
    say("determinism")
    y1, y2 = host(hip_fwd(d)), host(hip_fwd(d))
    np.testing.assert_array_equal(y1, y2)
    g1 = {k: host(v) for k, v in hip_bwd(d).items()}
    g2 = {k: host(v) for k, v in hip_bwd(d).items()}
    for k in GRADS:
        np.testing.assert_array_equal(g1[k], g2[k])


def test_guard_bands_poisoned_workspace_and_side_stream():
    """Outputs inside NaN guard bands, a NaN-filled workspace, a non-default
    stream, and unmodified inputs."""
    need_gpu()
    import torch
    import chunked_ssd_scan_fwd_amd as ssd
    s = Shape(2, 2, 4, 190, 48, 40)
    x = make_inputs(s, 10)
    d = to_dev(x)
    before = {k: v.clone() for k, v in d.items()}
    guard = 256

    def guarded(shape):
        n = int(np.prod(shape))
        buf = torch.full((n + 2 * guard,), float("nan"), device="cuda")
        return buf, buf[guard:guard + n].view(shape)

    sa = ssd.ShapeArg(s.B, s.G, s.H, s.T, s.dk, s.dv)
    ws = torch.full((ssd.workspace_size(sa, True) // 4 + 1,), float("nan"), device="cuda")
    bufs = [guarded(sh) for sh in [(s.B, s.H, s.T, s.dv), (s.B, s.G, s.T, s.dk), (s.B, s.G, s.T, s.dk),
                                   (s.B, s.H, s.T, s.dv), (s.B, s.H, s.T), (s.B, s.H, s.dk, s.dv)]]
    say("guard bands / side stream")
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        ssd.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], out=bufs[0][1], workspace=ws)
        ssd.bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], d["dy"],
                out=tuple(b[1] for b in bufs[1:]), workspace=ws)
    side.synchronize()
    for buf, view in bufs:
        b = buf.cpu().numpy()
        assert np.all(np.isnan(b[:guard])) and np.all(np.isnan(b[-guard:]))
        assert np.all(np.isfinite(view.cpu().numpy()))
    ref_y = oracle.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])
    assert rel_err(bufs[0][1].cpu().numpy(), ref_y) <= TOL_Y
    ref = oracle.bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], x["dy"])
    for (buf, view), name in zip(bufs[1:], GRADS):
        assert rel_err(view.cpu().numpy(), ref[name]) <= TOL_G, name
    for k in d:
        assert torch.equal(d[k], before[k])


# the last runs its forward on chunk pairs (states of even chunks only), in
# chunk segments: the reuse path then stores the odd chunks' states
REUSE = [ZOO[0], ZOO[3], ZOO[4], ZOO[5], ZOO[8], ZOO[10], ZOO[12], Shape(1, 1, 2, 65536, 128, 128)]


@pytest.mark.parametrize("shape", REUSE, ids=_id)
def test_bwd_from_fwd(shape):
    """The backward that reuses the forward's workspace: parity with the oracle,
    and agreement with the stateless backward (same kernels, same sums)."""
    need_gpu()
    import torch
    import chunked_ssd_scan_fwd_amd as ssd
    say(f"bwd_from_fwd {_id(shape)}")
    x = make_inputs(shape, seed=7 * shape.T + shape.dk)
    d = to_dev(x)
    sa = ssd.ShapeArg(shape.B, shape.G, shape.H, shape.T, shape.dk, shape.dv)
    ws = torch.empty(max(1, ssd.workspace_size(sa, True)), dtype=torch.uint8, device="cuda")
    y = ssd.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], workspace=ws)
    g = ssd.bwd_from_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], d["dy"], workspace=ws)
    g0 = ssd.bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], d["dy"])
    ref_y = oracle.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])
    assert rel_err(host(y), ref_y) <= TOL_Y
    ref = oracle.bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], x["dy"])
    for t, t0, name in zip(g, g0, GRADS):
        a = host(t)
        assert rel_err(a, ref[name]) <= TOL_G, name
        assert rel_err(a, host(t0)) <= 1e-6, name


def test_bwd_from_fwd_needs_workspace():
    need_gpu()
    import chunked_ssd_scan_fwd_amd as ssd
    say("bwd_from_fwd without workspace")
    d = to_dev(make_inputs(Shape(1, 1, 1, 8, 8, 8), 3))
    with pytest.raises(ValueError):
        ssd.bwd_from_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], d["dy"], workspace=None)


def _random_cases(n, seed):
    """Seeded random shapes (dims up to 256, T up to 6000, some group sizes
    and head counts) with a forward chunk setting each: unset, 64, or 128
    where the pair kernel takes dv (dv > 32, or above 128 a second block of
    more than 32 columns)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        G = int(rng.integers(1, 4))
        H = G * int(rng.integers(1, 6))
        B = int(rng.integers(1, 4))
        T = int(rng.integers(1, 200)) if rng.random() < 0.4 else int(rng.integers(200, 6000))
        dk = int(rng.integers(1, 129)) if rng.random() < 0.8 else int(rng.integers(129, 257))
        dv = int(rng.integers(1, 129)) if rng.random() < 0.8 else int(rng.integers(129, 257))
        if B * H * T * dk * dv > 4e8:
            continue
        chunk = ("", "64", "128")[len(out) % 3]
        if chunk == "128" and not (dv > 32 if dv <= 128 else dv - 128 > 32):
            chunk = ""
        out.append((Shape(B, G, H, T, dk, dv), chunk))
    return out


RANDOM_CASES = _random_cases(24, 2024)


@pytest.mark.parametrize("case", RANDOM_CASES, ids=lambda c: f"{_id(c[0])}_chunk{c[1] or 'auto'}")
def test_random_shapes(case, monkeypatch):
    """A seeded sweep over shapes and forward chunk settings: the forward,
    the stateless backward and the backward that reuses the forward's
    workspace, each against the oracle on whole tensors."""
    need_gpu()
    import torch
    import chunked_ssd_scan_fwd_amd as ssd
    shape, chunk = case
    monkeypatch.setenv("SSD_FWD_CHUNK", chunk)
    say(f"random {_id(shape)} chunk {chunk or 'auto'}")
    x = make_inputs(shape, seed=shape.T + 7 * shape.dk + 11 * shape.dv)
    d = to_dev(x)
    sa = ssd.ShapeArg(shape.B, shape.G, shape.H, shape.T, shape.dk, shape.dv)
    ws = torch.empty(max(1, ssd.workspace_size(sa, True)), dtype=torch.uint8, device="cuda")
    y = host(ssd.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], workspace=ws))
    assert rel_err(y, oracle.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])) <= TOL_Y
    ref = oracle.bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], x["dy"])
    g = ssd.bwd_from_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], d["dy"], workspace=ws)
    g0 = ssd.bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], d["dy"])
    for t, t0, name in zip(g, g0, GRADS):
        assert rel_err(host(t0), ref[name]) <= TOL_G, name
        assert rel_err(host(t), ref[name]) <= TOL_G, name


def test_empty_shapes():
    need_gpu()
    import torch
    import chunked_ssd_scan_fwd_amd as ssd
    say("empty shapes")
    x = to_dev(make_inputs(Shape(2, 1, 2, 0, 8, 8), 1))
    y = ssd.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])
    assert y.shape == (2, 2, 0, 8)
    dq, dk, dv, dla, dh0 = ssd.bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"], x["dy"])
    torch.cuda.synchronize()
    assert torch.count_nonzero(dh0).item() == 0


def test_timed_calls_match_plain_ones():
    """ssd_fwd_timed / ssd_bwd_timed give bitwise the plain calls' outputs and
    record one launch per timed kernel and call."""
    need_gpu()
    import torch
    import chunked_ssd_scan_fwd_amd as ssd
    s = Shape(2, 2, 4, 300, 64, 64)
    x = make_inputs(s, 21)
    d = to_dev(x)
    say("timed calls")
    y0 = host(hip_fwd(d))
    g0 = {k: host(v) for k, v in hip_bwd(d).items()}
    with ssd.KernelTimer() as t:
        y1 = ssd.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], timer=t)
        g1 = ssd.bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], d["dy"], timer=t)
        torch.cuda.synchronize()
        res = t.results()
    np.testing.assert_array_equal(host(y1), y0)
    for name, a in zip(GRADS, g1):
        np.testing.assert_array_equal(host(a), g0[name])
    for kname in ("state_scan", "chunk_output", "state_scan_bidir", "bwd_grads"):
        assert res[kname][1] == 1 and res[kname][0] > 0, (kname, res[kname])


def test_binding_rejects_short_or_strided_workspace():
    """A workspace view whose storage holds fewer bytes than needed, or a
    strided one, is refused before anything is launched."""
    need_gpu()
    import torch
    import chunked_ssd_scan_fwd_amd as ssd
    s = Shape(1, 1, 2, 100, 32, 32)
    d = to_dev(make_inputs(s, 22))
    sa = ssd.ShapeArg(s.B, s.G, s.H, s.T, s.dk, s.dv)
    need = ssd.workspace_size(sa, False)
    say("workspace checks")
    base = torch.empty(need, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):   # starts 16 bytes in: 16 bytes short
        ssd.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], workspace=base[16:])
    wide = torch.empty(2 * need, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):   # every other byte: not contiguous
        ssd.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], workspace=wide[::2])
    x = make_inputs(s, 22)
    y = ssd.fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["h0"], workspace=base)
    assert rel_err(host(y), oracle.fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["h0"])) <= TOL_Y
