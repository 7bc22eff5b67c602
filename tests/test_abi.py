"""CPU checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments on the host before any GPU work."""
import ctypes
import os
import re

import pytest

import chunked_ssd_scan_fwd_amd as ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ssd.library()
    names = declared_functions()
    assert "ssd_fwd" in names and "ssd_bwd" in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in ssd.h but not exported"


def _call_fwd(shape, ptr=1, ws_bytes=0):
    lib = ssd.library()
    p = ctypes.c_void_p(ptr) if ptr else None
    return lib.ssd_fwd(ctypes.byref(shape), p, p, p, p, p, p, p, ws_bytes, None)


def _call_bwd(shape, ptr=1, ws_bytes=0, fn="ssd_bwd"):
    lib = ssd.library()
    p = ctypes.c_void_p(ptr) if ptr else None
    return getattr(lib, fn)(ctypes.byref(shape), *([p] * 11), p, ws_bytes, None)


@pytest.mark.parametrize("shape,code", [
    (ssd.ShapeArg(1, 3, 4, 10, 8, 8), 2),      # H % G != 0
    (ssd.ShapeArg(1, 0, 4, 10, 8, 8), 2),      # G < 1
    (ssd.ShapeArg(-1, 1, 1, 10, 8, 8), 2),     # negative B
    (ssd.ShapeArg(1, 1, 1, -5, 8, 8), 2),      # negative T
    (ssd.ShapeArg(1, 1, 1, 10, 0, 8), 2),      # dk = 0
    (ssd.ShapeArg(1, 1, 1, 10, 257, 8), 3),    # dk above the supported range
    (ssd.ShapeArg(1, 1, 1, 10, 8, 300), 3),    # dv above the supported range
    (ssd.ShapeArg(1 << 40, 1 << 40, 1 << 40, 10, 8, 8), 2),   # overflow guard
])
def test_bad_shapes_rejected(shape, code):
    assert _call_fwd(shape) == code
    assert _call_bwd(shape) == code
    assert _call_bwd(shape, fn="ssd_bwd_from_fwd") == code


def test_null_shape_and_pointers():
    lib = ssd.library()
    assert lib.ssd_fwd(None, *([None] * 7), 0, None) == 1
    s = ssd.ShapeArg(1, 1, 1, 10, 8, 8)
    assert _call_fwd(s, ptr=0) == 1
    assert _call_bwd(s, ptr=0) == 1
    assert _call_bwd(s, ptr=0, fn="ssd_bwd_from_fwd") == 1


def test_misaligned_pointer_rejected():
    s = ssd.ShapeArg(1, 1, 1, 10, 8, 8)
    assert _call_fwd(s, ptr=0x1004) == 5
    assert _call_bwd(s, ptr=0x1004) == 5


def test_workspace_too_small_rejected():
    s = ssd.ShapeArg(1, 1, 1, 10, 8, 8)
    need = ssd.workspace_size(s, False)
    assert need > 0
    assert _call_fwd(s, ptr=0x1000, ws_bytes=need - 1) == 4
    assert _call_bwd(s, ptr=0x1000, ws_bytes=ssd.workspace_size(s, True) - 1) == 4


def test_empty_problems_need_no_workspace():
    assert ssd.workspace_size(ssd.ShapeArg(0, 1, 1, 10, 8, 8), True) == 0
    assert ssd.workspace_size(ssd.ShapeArg(2, 1, 1, 0, 8, 8), False) == 0
    # empty forward needs no pointers at all
    assert _call_fwd(ssd.ShapeArg(0, 1, 1, 10, 8, 8), ptr=0) == 0


def _scan_segments(B, H, T, dk, dv, ndir, cus=256):
    """Segments of a state-scan launch over `ndir` directions: one block per
    32 x 64 state tile (32 x dv for dv < 64); when that fills at most half
    the CUs the tiles are 32 wide; then the segment count doubles while the
    grid still fills at most half the CUs, every segment keeps at least 8
    chunks and there are at most 64; finally it is recounted so that no
    segment is empty."""
    NC = -(-T // 64)
    pad = lambda d: 32 if d <= 32 else (64 if d <= 64 else 128)
    DKP, DVP = pad(dk), pad(dv)
    wide = ndir * B * H * (DKP // 32) * (DVP // min(DVP, 64))
    blocks = 2 * wide if (DVP >= 64 and 2 * wide <= cus) else wide
    nseg = 1
    while blocks * nseg * 2 <= cus and NC >= nseg * 2 * 8 and nseg < 64:
        nseg *= 2
    seg_len = -(-NC // nseg)
    return -(-NC // seg_len) if seg_len > 0 else nseg


@pytest.mark.parametrize("B,G,H,T,dk,dv", [(4, 2, 8, 8192, 128, 128), (2, 1, 24, 8192, 128, 64),
                                           (4, 2, 4, 2048, 48, 40), (1, 1, 1, 1, 1, 1),
                                           (1, 1, 4, 130, 64, 64), (2, 2, 10, 1024, 48, 40),
                                           (2, 1, 24, 512, 128, 64)])
def test_workspace_layout_formula(B, G, H, T, dk, dv):
    s = ssd.ShapeArg(B, G, H, T, dk, dv)
    off = ssd.workspace_layout(s, True)
    assert len(off) == ssd.WS_REGIONS + 1
    NC = (T + 63) // 64
    Epad = (dk * dv + 63) // 64 * 64
    BH = B * H

    def up(x):
        return (x + 255) // 256 * 256

    assert off[0] == 0
    cdec = up(BH * NC * 128 * 4)
    assert off[1] == up(cdec + BH * NC * 4)
    assert off[2] == up(off[1] + BH * NC * Epad * 4)
    assert off[3] == up(off[2] + BH * NC * Epad * 4)
    # fewer (b, g, chunk) blocks than the device's compute units (256 when no
    # device is visible): the group's heads are split over blocks and the
    # backward keeps per-split dq, dk partial sums
    hpg, blocks = H // G, B * G * NC
    want = min(hpg, -(-256 // blocks)) if blocks < 256 else 1
    hpb = -(-hpg // want)
    hsplit = -(-hpg // hpb)
    parts = 2 * hsplit * (-(-(B * G * T * dk) // 64) * 64) * 4 if hsplit > 1 else 0
    # segment end states and per-chunk decay products when a scan launch
    # (one direction, or both in the backward) runs in chunk segments
    n1, n2 = _scan_segments(B, H, T, dk, dv, 1), _scan_segments(B, H, T, dk, dv, 2)
    nends_b = max(n1 if n1 > 1 else 0, 2 * n2 if n2 > 1 else 0)
    nends_f = n1 if n1 > 1 else 0

    def seg_bytes(nends):
        return up(nends * BH * Epad * 4) + up(2 * BH * NC * 4) if nends else 0

    assert off[4] == up(off[3] + parts) + seg_bytes(nends_b)
    assert ssd.workspace_size(s, True) == off[4]
    fo = ssd.workspace_layout(s, False)
    assert fo[:2] == off[:2] and fo[2] == fo[3] == off[2]
    assert fo[4] == fo[3] + seg_bytes(nends_f)
    assert ssd.workspace_size(s, False) == fo[4]


def test_workspace_layout_segmented_scan():
    """A shape whose state scan runs in chunk segments (few heads, long T):
    region 3 holds the segment end states and the per-chunk decay products.
    B = G = H = 1, T = 8192, dk = dv = 128 on 256 CUs: the forward scan has
    16 narrow tiles, so 16 segments of 8 chunks; the two-direction backward
    launch has 32, so 8 segments per direction; room for 16 end states and
    [2][1][128] decay products."""
    s = ssd.ShapeArg(1, 1, 1, 8192, 128, 128)
    off = ssd.workspace_layout(s, True)
    NC, Epad = 128, 128 * 128

    def up(x):
        return (x + 255) // 256 * 256

    assert off[3] == up(off[2] + NC * Epad * 4)
    ends = 16 * Epad * 4
    assert off[4] == up(off[3] + ends) + up(2 * NC * 4)
    fo = ssd.workspace_layout(s, False)
    assert fo[3] == fo[2] == off[2]
    assert fo[4] == up(fo[3] + ends) + up(2 * NC * 4)
    assert _scan_segments(1, 1, 8192, 128, 128, 1) == 16 and _scan_segments(1, 1, 8192, 128, 128, 2) == 8


@pytest.mark.parametrize("B,G,H,T,dk,dv,stride", [
    (4, 2, 8, 8192, 128, 128, 2),   # 512 pairs of chunks: two per CU
    (4, 2, 8, 8190, 97, 100, 2),    # dv pads to 128, ragged T
    (4, 2, 8, 2048, 128, 128, 1),   # 128 pairs: fewer than two per CU
    (2, 1, 24, 8192, 128, 64, 1),   # 64-column states
    (1, 1, 4, 65536, 128, 128, 2),
    (1, 1, 1, 1, 1, 1, 1),
])
def test_forward_state_stride(B, G, H, T, dk, dv, stride, monkeypatch):
    """The forward runs on chunk pairs (states of even chunks only) for
    128-column states with at least two pairs per CU (256 CUs when no device
    is visible)."""
    monkeypatch.delenv("SSD_FWD_CHUNK", raising=False)
    assert ssd.fwd_state_stride(ssd.ShapeArg(B, G, H, T, dk, dv)) == stride
    monkeypatch.setenv("SSD_FWD_CHUNK", "")
    assert ssd.fwd_state_stride(ssd.ShapeArg(B, G, H, T, dk, dv)) == stride


# shape: state stride under SSD_FWD_CHUNK = 64 and = 128 (-1: refused, the
# pair kernel takes 64- and 128-column states only)
FWD_CHUNK_STRIDES = {
    (4, 2, 8, 8192, 128, 128): (1, 2),
    (4, 2, 8, 2048, 128, 128): (1, 2),
    (2, 1, 24, 8192, 128, 64): (1, 2),
    (2, 2, 4, 300, 48, 40): (1, 2),
    (1, 1, 1, 1, 1, 1): (1, -1),
    (3, 1, 2, 129, 33, 32): (1, -1),
}


def test_forward_chunk_setting(monkeypatch):
    """SSD_FWD_CHUNK fixes the forward's chunk length: 64 keeps every chunk's
    state, 128 runs on chunk pairs wherever the pair kernel takes the shape."""
    lib = ssd.library()
    for i, val in enumerate(("64", "128")):
        monkeypatch.setenv("SSD_FWD_CHUNK", val)
        for sh, strides in FWD_CHUNK_STRIDES.items():
            assert lib.ssd_fwd_state_stride(ctypes.byref(ssd.ShapeArg(*sh))) == strides[i], (val, sh)


@pytest.mark.parametrize("val", ["96", "abc", "64 ", "0", "256"])
def test_forward_chunk_setting_refused(val, monkeypatch):
    """Values other than 64 and 128 are refused by every call that the
    forward's chunk length concerns, before anything is enqueued (the
    workspace passed is one byte short, so a call that went on would stop at
    the workspace check instead)."""
    monkeypatch.setenv("SSD_FWD_CHUNK", val)
    s = ssd.ShapeArg(1, 1, 2, 100, 64, 64)
    assert ssd.library().ssd_fwd_state_stride(ctypes.byref(s)) == -1
    assert _call_fwd(s, ptr=0x1000, ws_bytes=ssd.workspace_size(s, False) - 1) == 3
    assert _call_bwd(s, ptr=0x1000, ws_bytes=ssd.workspace_size(s, True) - 1, fn="ssd_bwd_from_fwd") == 3
    # the stateless backward does not depend on it
    assert _call_bwd(s, ptr=0x1000, ws_bytes=ssd.workspace_size(s, True) - 1) == 4


def test_forward_chunk_128_refused_where_pairs_do_not_fit(monkeypatch):
    """128 on a forward whose dv (or a 128-column block of it) pads to 32:
    refused before anything is enqueued, also for the column-split path,
    which would otherwise enqueue its block copies first."""
    monkeypatch.setenv("SSD_FWD_CHUNK", "128")
    for sh in ((1, 1, 1, 10, 8, 8), (1, 1, 1, 10, 8, 144), (1, 1, 1, 10, 200, 20)):
        s = ssd.ShapeArg(*sh)
        assert _call_fwd(s, ptr=0x1000, ws_bytes=ssd.workspace_size(s, False) - 1) == 3, sh
    # a split shape whose dv blocks both suit the pair kernel passes the check
    # and stops at the workspace
    s = ssd.ShapeArg(1, 1, 1, 10, 8, 200)
    assert _call_fwd(s, ptr=0x1000, ws_bytes=ssd.workspace_size(s, False) - 1) == 4


def test_forward_state_stride_refuses_other_shapes():
    lib = ssd.library()
    for s in (ssd.ShapeArg(1, 3, 4, 10, 8, 8), ssd.ShapeArg(1, 1, 1, 100, 8, 200)):
        assert lib.ssd_fwd_state_stride(ctypes.byref(s)) == -1


def test_status_strings_and_constants():
    lib = ssd.library()
    for code in range(7):
        assert lib.ssd_strerror(code)
    assert lib.ssd_strerror(99) == b"unknown status"
    assert lib.ssd_chunk_size() == ssd.CHUNK == 64
    names = [lib.ssd_kernel_name(i).decode() for i in range(lib.ssd_kernel_count())]
    assert "bwd_grads" in names and "state_scan" in names and "chunk_output" in names
    assert lib.ssd_kernel_name(-1) == b"unknown"


def test_timer_lifecycle_without_launches():
    """A timer is a caller-owned object: created, read, reset and destroyed
    without any launch; the plain compute calls take none."""
    t = ssd.KernelTimer(["bwd_grads"])
    res = t.results()
    assert set(res) == set(t.names) and all(v == (0.0, 0) for v in res.values())
    t.reset()
    t.close()
    lib = ssd.library()
    assert lib.ssd_timer_destroy(None) == 1
    assert lib.ssd_timer_reset(None) == 1
    with pytest.raises(ValueError):
        ssd.KernelTimer(["no_such_kernel"])


def test_timed_calls_validate_like_plain_ones():
    lib = ssd.library()
    t = ssd.KernelTimer()
    p = ctypes.c_void_p(1)
    bad = ssd.ShapeArg(1, 3, 4, 10, 8, 8)
    assert lib.ssd_fwd_timed(t.handle, ctypes.byref(bad), *([p] * 7), 0, None) == 2
    assert lib.ssd_bwd_timed(t.handle, ctypes.byref(bad), *([p] * 12), 0, None) == 2
    assert lib.ssd_fwd_timed(None, ctypes.byref(bad), *([p] * 7), 0, None) == 1
    t.close()


def test_binding_rejects_foreign_workspace():
    """The binding checks a caller's workspace before any launch: device,
    contiguity and the bytes its storage really holds."""
    import torch
    s = ssd.ShapeArg(1, 1, 1, 10, 8, 8)
    need = ssd.workspace_size(s, False)
    dev = torch.device("cuda:0")
    with pytest.raises(ValueError, match="HIP device"):
        ssd._workspace(s, False, dev, torch.empty(need, dtype=torch.uint8))
    with pytest.raises(TypeError):
        ssd._workspace(s, False, dev, bytearray(need))


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 8)
    with pytest.raises(ValueError):
        ssd.fwd(x, x, x, torch.zeros(1, 1, 4), torch.zeros(1, 1, 8, 8))


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(ImportError):
        ssd.library(str(tmp_path / "missing.so"))


def test_noalloc_refuses_oversized_shapes_on_host():
    """ssd_fwd_noalloc checks the shape's workspace against its static array
    on the host and returns SSD_ERR_WORKSPACE without touching a device."""
    lib = ssd.library()
    big = ssd.ShapeArg(4, 2, 8, 8192, 128, 128)
    assert ssd.workspace_size(big, False) > ssd.NOALLOC_WORKSPACE_BYTES
    p = ctypes.c_void_p(16)
    assert lib.ssd_fwd_noalloc(ctypes.byref(big), *([p] * 6), None) == 4
    assert lib.ssd_fwd_noalloc(ctypes.byref(ssd.ShapeArg(1, 3, 4, 10, 8, 8)), *([p] * 6), None) == 2
    # the largest workload of the pages at T = 2048 fits
    assert ssd.workspace_size(ssd.ShapeArg(4, 2, 8, 2048, 128, 128), False) <= ssd.NOALLOC_WORKSPACE_BYTES


@pytest.mark.parametrize("B,G,H,T,dk,dv", [(1, 1, 2, 300, 256, 256), (2, 2, 4, 150, 200, 136),
                                           (1, 1, 1, 70, 129, 1), (1, 2, 2, 100, 1, 250)])
def test_wide_shapes_workspace(B, G, H, T, dk, dv):
    """dk or dv in 129..256 run as column-block sub-problems: the workspace
    holds the largest sub-problem's workspace plus one block of every operand
    and output; the region query refuses these shapes."""
    s = ssd.ShapeArg(B, G, H, T, dk, dv)
    lib = ssd.library()
    arr = (ctypes.c_size_t * (ssd.WS_REGIONS + 1))()
    assert lib.ssd_workspace_layout(ctypes.byref(s), 1, arr) == 3
    sub = max(ssd.workspace_size(ssd.ShapeArg(B, G, H, T, a, b), True)
              for a in ([dk] if dk <= 128 else [128, dk - 128]) for b in ([dv] if dv <= 128 else [128, dv - 128]))
    dkm, dvm = min(dk, 128), min(dv, 128)
    blocks = 4 * (2 * B * G * T * dkm + B * H * T * dvm + B * H * dkm * dvm)
    assert ssd.workspace_size(s, True) >= sub + blocks
    assert ssd.workspace_size(s, False) >= ssd.workspace_size(
        ssd.ShapeArg(B, G, H, T, dkm, dvm), False) + blocks
    # validation still happens on the host before anything else
    assert _call_fwd(s, ptr=0x1000, ws_bytes=ssd.workspace_size(s, False) - 1) == 4
    assert _call_bwd(s, ptr=0x1000, ws_bytes=ssd.workspace_size(s, True) - 1) == 4


# ---- selective (Mamba-style) scan: host-side checks, no launches


def _mamba_call(shape, ptr=0x1000, ws_bytes=0):
    lib = ssd.library()
    p = ctypes.c_void_p(ptr) if ptr else None
    return lib.mamba_fwd(ctypes.byref(shape), *([p] * 7), p, ws_bytes, None)


@pytest.mark.parametrize("shape,code", [
    (ssd.MambaShapeArg(-1, 10, 4, 16), 2),        # negative B
    (ssd.MambaShapeArg(1, -3, 4, 16), 2),         # negative L
    (ssd.MambaShapeArg(1, 10, 0, 16), 2),         # D = 0
    (ssd.MambaShapeArg(1, 10, 4, 0), 2),          # N = 0
    (ssd.MambaShapeArg(1, 10, 4, 17), 3),         # more states than a thread holds
    (ssd.MambaShapeArg(70000, 10, 4, 16), 3),     # batch beyond the grid's z extent
    (ssd.MambaShapeArg(1, 65535 * 256 + 1, 4, 16), 3),   # segments beyond the grid's y extent
])
def test_mamba_bad_shapes_rejected(shape, code):
    assert _mamba_call(shape) == code
    assert ssd.library().mamba_fwd_workspace_size(ctypes.byref(shape)) == 0


def test_mamba_validation_before_launch():
    lib = ssd.library()
    assert lib.mamba_fwd(None, *([None] * 7), None, 0, None) == 1
    s = ssd.MambaShapeArg(2, 4096, 64, 16)
    need = ssd.mamba_workspace_size(s)
    assert need > 0
    assert _mamba_call(s, ptr=0) == 1                          # null tensors
    assert _mamba_call(s, ptr=0x1002) == 5                     # misaligned
    assert _mamba_call(s, ptr=0x1000, ws_bytes=need - 1) == 4  # short workspace
    # empty problems need nothing
    assert _mamba_call(ssd.MambaShapeArg(0, 10, 4, 16), ptr=0) == 0
    assert _mamba_call(ssd.MambaShapeArg(3, 0, 4, 16), ptr=0) == 0


def test_mamba_workspace_formula():
    """Segment end states float [B][nseg][N][D] and summed deltas float
    [B][nseg][D], each 256-byte aligned; about 1024 threads per CU (256 CUs
    when no device is visible), segments of 16 to 256 steps."""
    def plan(B, L, D):
        nseg = max(1, -(-256 * 1024 // (B * D)))
        nseg = min(nseg, max(1, L // 16))
        nseg = max(nseg, -(-L // 256))
        sl = -(-L // nseg)
        return -(-L // sl)
    up = lambda x: (x + 255) // 256 * 256
    for B, L, D, N in [(4, 8192, 256, 16), (4, 512, 1024, 16), (1, 100, 3, 5), (2, 7, 64, 16), (1, 70000, 1, 1)]:
        ns = plan(B, L, D)
        want = 0 if ns == 1 else up(B * ns * N * D * 4) + up(B * ns * D * 4)
        assert ssd.mamba_workspace_size(ssd.MambaShapeArg(B, L, D, N)) == want, (B, L, D, N)


def _mamba_bwd_call(shape, ptr=0x1000, ws_bytes=0, ws=None):
    lib = ssd.library()
    p = ctypes.c_void_p(ptr) if ptr else None
    w = ctypes.c_void_p(ws) if ws else p
    return lib.mamba_bwd(ctypes.byref(shape), *([p] * 13), w, ws_bytes, None)


def test_mamba_bwd_validation_before_launch():
    lib = ssd.library()
    assert lib.mamba_bwd(None, *([None] * 13), None, 0, None) == 1
    for bad, code in [(ssd.MambaShapeArg(1, 10, 4, 17), 3), (ssd.MambaShapeArg(1, 10, 0, 16), 2),
                      (ssd.MambaShapeArg(1, 65535 * 32 + 1, 4, 16), 3)]:   # backward segments beyond the grid
        assert _mamba_bwd_call(bad) == code
        assert lib.mamba_bwd_workspace_size(ctypes.byref(bad)) == 0
    s = ssd.MambaShapeArg(2, 4096, 64, 16)
    need = ssd.mamba_workspace_size(s, backward=True)
    assert need > 0
    assert _mamba_bwd_call(s, ptr=0) == 1                          # null tensors
    assert _mamba_bwd_call(s, ptr=0x1002) == 5                     # misaligned
    assert _mamba_bwd_call(s, ptr=0x1000, ws_bytes=need - 1) == 4  # short workspace
    assert _mamba_bwd_call(s, ptr=0x1000, ws_bytes=need, ws=0x1004) == 5   # workspace not 16-byte aligned


def test_mamba_bwd_workspace_formula():
    """Segments of 32 steps; forward entering states [B][nseg][N][D], summed
    deltas [B][nseg][D], adjoints entering from the right and dA partials
    [B][nseg][D][N], dDskip partials [B][nseg][D], and with nsplit > 1 the
    dB / dC partials [nsplit][B][L][2][N]; nsplit = min(channel chunks of 64,
    ceil(2 CUs / (nseg B))), 256 CUs when no device is visible."""
    up = lambda x: (x + 255) // 256 * 256
    for B, L, D, N in [(4, 8192, 1024, 16), (4, 512, 256, 16), (1, 100, 3, 5), (2, 7, 64, 16), (1, 70000, 1, 1)]:
        ns = -(-L // 32)
        split = max(1, min(-(-D // 64), -(-2 * 256 // (ns * B))))
        want = up(B * ns * N * D * 4) + up(B * ns * D * 4) + 2 * up(B * ns * D * N * 4) + up(B * ns * D * 4)
        if split > 1:
            want += up(split * B * L * 2 * N * 4)
        assert ssd.mamba_workspace_size(ssd.MambaShapeArg(B, L, D, N), backward=True) == want, (B, L, D, N)
    assert ssd.mamba_workspace_size(ssd.MambaShapeArg(0, 10, 4, 16), backward=True) == 0


def test_mamba_fwd_bwd_validation_before_launch():
    lib = ssd.library()
    s = ssd.MambaShapeArg(2, 4096, 64, 16)
    need = ssd.mamba_workspace_size(s, backward=True)
    p = ctypes.c_void_p(0x1000)

    def call(y, ws_bytes=need):
        return lib.mamba_fwd_bwd(ctypes.byref(s), *([p] * 7), y, *([p] * 6), p, ws_bytes, None)
    assert call(None) == 1                           # y missing
    assert call(ctypes.c_void_p(0x1002)) == 5        # y misaligned
    assert call(p, need - 1) == 4                    # short workspace
    assert lib.mamba_fwd_bwd(None, *([None] * 14), None, 0, None) == 1
    # an empty problem needs no y, and still zeroes dA and dDskip (not run here)
    e = ssd.MambaShapeArg(0, 10, 4, 16)
    assert lib.mamba_fwd_bwd(ctypes.byref(e), *([None] * 8), *([None] * 2), None, None, None, None, None, 0,
                             None) == 1              # dA, dDskip are required
