// Host-only argument checks and workspace layout for the SSD scan C ABI.
// This unit makes no HIP call (the device's compute-unit count comes from
// device_cus() in the HIP unit).
#include <cstdlib>
#include <cstring>

#include "ssd_internal.h"

namespace ssd {

int check_shape(const ssd_shape *s)
{
    if (!s) return SSD_ERR_NULL;
    if (s->B < 0 || s->T < 0 || s->G < 1 || s->H < 1 || s->dk < 1 || s->dv < 1) return SSD_ERR_SHAPE;
    if (s->H % s->G != 0) return SSD_ERR_SHAPE;
    // Keep every element index comfortably inside 64-bit arithmetic and the
    // per-(b,h) sequence offsets inside 32-bit chunk counts.
    const int64_t lim = int64_t(1) << 40;
    if (s->B > lim || s->H > lim || s->T > lim) return SSD_ERR_SHAPE;
    const int64_t dmax = s->dk > s->dv ? s->dk : s->dv;
    if (dmax > kMaxApiDim) return SSD_ERR_UNSUPPORTED;
    if (s->B > lim / s->H) return SSD_ERR_SHAPE;           // B*H <= 2^40, no overflow below
    if (s->B * s->H > lim / (s->T + 1)) return SSD_ERR_SHAPE;
    if (s->B * s->H * (s->T + 1) > lim / dmax) return SSD_ERR_SHAPE;
    if ((s->T + kChunk - 1) / kChunk > (int64_t(1) << 30)) return SSD_ERR_SHAPE;
    // Every launch grid is one-dimensional: blocks must fit in 2^31 - 1.
    const int64_t nc = (s->T + kChunk - 1) / kChunk;
    const int64_t grid_lim = (int64_t(1) << 31) - 1;
    if (s->B * s->H > grid_lim / 16) return SSD_ERR_UNSUPPORTED;
    if (nc > 0 && s->B * s->H > grid_lim / nc) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

static size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

void head_split(const ssd_shape *s, int64_t NC, int cus, int *hsplit, int *hpb)
{
    const int64_t hpg = s->H / s->G, blocks = s->B * s->G * NC;
    int64_t want = 1;
    if (blocks > 0 && blocks < cus) want = (cus + blocks - 1) / blocks;
    if (want > hpg) want = hpg;
    const int64_t per = (hpg + want - 1) / want;
    *hpb = (int)per;
    *hsplit = (int)((hpg + per - 1) / per);
}

bool fwd_pairs(const ssd_shape *s, int cus)
{
    const int64_t NC = (s->T + kChunk - 1) / kChunk;
    return pad_dim(s->dv) == 128 && s->B * s->G * ((NC + 1) / 2) >= 2 * int64_t(cus);
}

int mamba_check_shape(const mamba_shape *s)
{
    if (!s) return SSD_ERR_NULL;
    if (s->B < 0 || s->L < 0 || s->D < 1 || s->N < 1) return SSD_ERR_SHAPE;
    const int64_t lim = int64_t(1) << 40;
    if (s->B > lim || s->L > lim || s->D > lim || s->N > lim) return SSD_ERR_SHAPE;
    if (s->N > MAMBA_MAX_STATE) return SSD_ERR_UNSUPPORTED;
    const int64_t w = s->D > s->N ? s->D : s->N;
    if (s->B > lim / (s->L + 1) || s->B * (s->L + 1) > lim / w) return SSD_ERR_SHAPE;
    // grid: x over 256-channel blocks, y over segments (at most 65535 of at
    // most kMambaMaxSeg steps), z over batch
    if ((s->D + 255) / 256 > (int64_t(1) << 31) - 1 || s->B > 65535) return SSD_ERR_UNSUPPORTED;
    if (s->L > 65535 * kMambaMaxSeg) return SSD_ERR_UNSUPPORTED;
    // a segment's rows of x, delta and y are one buffer resource (< 2 GiB)
    if (s->D > (int64_t(1) << 20)) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

MambaPlan mamba_plan(const mamba_shape *s, int cus)
{
    MambaPlan P;
    P.seg_len = s->L;
    if (s->B == 0 || s->L == 0) return P;
    // About 1024 threads (16 waves) per CU over all segments, segments of
    // at least 16 steps where that allows, at most kMambaMaxSeg steps, and
    // at most 65535 of them (the launch grid's y extent).  More segments
    // hide more latency in the scans but lengthen the carry pass's chain;
    // over the page's grid (batch 4, dim 256 to 1024, seq 512 to 8192) this
    // choice was the fastest or within 2% of it among 512 to 4096 threads
    // per CU and segments of 8 or 16 steps and up.
    const int64_t want = (int64_t(cus) * 1024 + s->B * s->D - 1) / (s->B * s->D);
    int64_t nseg = want < 1 ? 1 : want;
    const int64_t cap = s->L / 16 > 1 ? s->L / 16 : 1;
    if (nseg > cap) nseg = cap;
    const int64_t least = (s->L + kMambaMaxSeg - 1) / kMambaMaxSeg;
    if (nseg < least) nseg = least;
    if (nseg > 65535) nseg = 65535;
    P.seg_len = (s->L + nseg - 1) / nseg;
    P.nseg = (s->L + P.seg_len - 1) / P.seg_len;
    if (P.nseg <= 1) {
        P.nseg = 1;
        return P;   // one segment: no workspace
    }
    size_t o = 0;
    P.hend = o;
    o = round_up(o + size_t(s->B) * size_t(P.nseg) * size_t(s->N) * size_t(s->D) * sizeof(float), 256);
    P.sdl = o;
    o = round_up(o + size_t(s->B) * size_t(P.nseg) * size_t(s->D) * sizeof(float), 256);
    P.total = o;
    return P;
}

MambaBwdPlan mamba_bwd_plan(const mamba_shape *s, int cus)
{
    MambaBwdPlan P;
    if (s->B == 0 || s->L == 0) return P;
    P.nseg = (s->L + kMambaBwdSeg - 1) / kMambaBwdSeg;
    const int64_t nchunk = (s->D + kMambaBwdChans - 1) / kMambaBwdChans;
    int64_t want = (2 * int64_t(cus) + P.nseg * s->B - 1) / (P.nseg * s->B);
    if (want > nchunk) want = nchunk;
    if (want < 1) want = 1;
    P.nsplit = (int)want;
    const size_t B = size_t(s->B), ns = size_t(P.nseg), N = size_t(s->N), D = size_t(s->D), f = sizeof(float);
    size_t o = 0;
    P.hend = o;
    o = round_up(o + B * ns * N * D * f, 256);
    P.sdl = o;
    o = round_up(o + B * ns * D * f, 256);
    P.gl = o;
    o = round_up(o + B * ns * D * N * f, 256);
    P.dApart = o;
    o = round_up(o + B * ns * D * N * f, 256);
    P.dDpart = o;
    o = round_up(o + B * ns * D * f, 256);
    P.dBC = o;
    if (P.nsplit > 1) o = round_up(o + size_t(P.nsplit) * B * size_t(s->L) * 2 * N * f, 256);
    P.total = o;
    return P;
}

int fwd_chunk_setting()
{
    const char *e = std::getenv("SSD_FWD_CHUNK");
    if (!e || !*e) return 0;
    if (!std::strcmp(e, "64")) return 64;
    if (!std::strcmp(e, "128")) return 128;
    return -1;
}

// The pair kernel is built for 64- and 128-column states.
static bool pair_cols(int64_t dv) { return pad_dim(dv) >= 64; }

int fwd_pair_mode(const ssd_shape *s, int cus, bool *pair)
{
    const int c = fwd_chunk_setting();
    if (c < 0 || (c == 128 && !pair_cols(s->dv))) return SSD_ERR_UNSUPPORTED;
    *pair = c == 0 ? fwd_pairs(s, cus) : c == 128;
    return SSD_OK;
}

int fwd_chunk_check(const ssd_shape *s)
{
    const int c = fwd_chunk_setting();
    if (c < 0) return SSD_ERR_UNSUPPORTED;
    if (c != 128) return SSD_OK;
    // dv blocks: dv itself, or kMaxDim and the rest
    if (s->dv <= kMaxDim) return pair_cols(s->dv) ? SSD_OK : SSD_ERR_UNSUPPORTED;
    return pair_cols(s->dv - kMaxDim) ? SSD_OK : SSD_ERR_UNSUPPORTED;
}

ScanPlan scan_plan(const ssd_shape *s, int ndir, int cus)
{
    ScanPlan P;
    const int64_t NC = (s->T + kChunk - 1) / kChunk;
    const int64_t DKP = pad_dim(s->dk), DVP = pad_dim(s->dv);
    const int64_t tiles_k = s->B * s->H * (DKP / 32);
    const int64_t wide = ndir * tiles_k * (DVP / (DVP < 64 ? DVP : 64));
    P.narrow = DVP >= 64 && 2 * wide <= cus;
    const int64_t blocks = P.narrow ? 2 * wide : wide;
    while (blocks * P.nseg * 2 <= cus && NC >= P.nseg * 2 * kMinSegChunks && P.nseg < kMaxSegs) P.nseg *= 2;
    P.seg_len = (NC + P.nseg - 1) / P.nseg;
    // every segment holds at least one chunk (the last may be shorter)
    if (P.seg_len > 0) P.nseg = (int)((NC + P.seg_len - 1) / P.seg_len);
    P.blocks = blocks * P.nseg;
    return P;
}

Layout make_layout(const ssd_shape *s, bool backward, int cus)
{
    Layout L;
    L.NC = (s->T + kChunk - 1) / kChunk;
    L.E = s->dk * s->dv;
    L.Epad = (L.E + 63) / 64 * 64;
    head_split(s, L.NC, cus, &L.hsplit, &L.hpb);
    L.nqk_pad = (s->B * s->G * s->T * s->dk + 63) / 64 * 64;
    const size_t BH = size_t(s->B) * size_t(s->H);
    if (BH == 0 || s->T == 0) return L;   // nothing to store
    const size_t slab = BH * size_t(L.NC) * size_t(L.Epad) * sizeof(float);
    size_t o = 0;
    L.off[0] = o;
    o = round_up(o + BH * size_t(L.NC) * 2 * kChunk * sizeof(float), 256);
    L.cdec_off = o;
    o = round_up(o + BH * size_t(L.NC) * sizeof(float), 256);
    L.off[1] = o;
    o = round_up(o + slab, 256);
    L.off[2] = o;
    if (backward) o = round_up(o + slab, 256);
    L.off[3] = o;
    if (backward && L.hsplit > 1) o = round_up(o + 2 * size_t(L.hsplit) * size_t(L.nqk_pad) * sizeof(float), 256);
    // segment end states, for launches whose plan cuts the chunks into
    // segments: the forward launch (one direction); the backward runs either
    // both directions in one launch or the reverse alone
    size_t nends = 0;
    const size_t one = size_t(scan_plan(s, 1, cus).nseg);
    if (one > 1) nends = one;
    if (backward) {
        const size_t two = size_t(scan_plan(s, 2, cus).nseg);
        if (two > 1 && 2 * two > nends) nends = 2 * two;
    }
    L.ends_off = o;
    if (nends > 0) o = round_up(o + nends * BH * size_t(L.Epad) * sizeof(float), 256);
    L.segd_off = o;
    if (nends > 0) o = round_up(o + 2 * BH * size_t(L.NC) * sizeof(float), 256);
    L.off[4] = o;
    return L;
}

bool needs_split(const ssd_shape *s) { return s->dk > kMaxDim || s->dv > kMaxDim; }

ssd_shape sub_shape(const ssd_shape *s, const SplitLayout &P, int I, int J)
{
    ssd_shape t = *s;
    t.dk = P.dkb[I];
    t.dv = P.dvb[J];
    return t;
}

// Blocks of kMaxDim columns and the remainder: 200 = 128 + 72.
static int split_dim(int64_t d, int64_t *off, int64_t *w)
{
    if (d <= kMaxDim) {
        off[0] = 0;
        w[0] = d;
        return 1;
    }
    off[0] = 0;
    w[0] = kMaxDim;
    off[1] = kMaxDim;
    w[1] = d - kMaxDim;
    return 2;
}

SplitLayout make_split_layout(const ssd_shape *s, bool backward, int cus)
{
    SplitLayout P;
    P.nI = split_dim(s->dk, P.i0, P.dkb);
    P.nJ = split_dim(s->dv, P.j0, P.dvb);
    P.dkm = P.dkb[0];
    P.dvm = P.dvb[0];
    for (int I = 0; I < P.nI; ++I)
        for (int J = 0; J < P.nJ; ++J) {
            const ssd_shape t = sub_shape(s, P, I, J);
            const size_t b = make_layout(&t, backward, cus).off[SSD_WS_REGIONS];
            if (b > P.sub_bytes) P.sub_bytes = b;
        }
    const size_t f = sizeof(float);
    const size_t BG = size_t(s->B) * size_t(s->G), BH = size_t(s->B) * size_t(s->H), T = size_t(s->T);
    const size_t nq = BG * T * size_t(P.dkm), nv = BH * T * size_t(P.dvm), nh = BH * size_t(P.dkm * P.dvm);
    size_t o = 0;
    auto take = [&](size_t &at, size_t n) {
        at = o;
        o = round_up(o + n, 256);
    };
    take(P.sub, P.sub_bytes);
    take(P.qb, nq * f);
    take(P.kb, nq * f);
    take(P.vb, nv * f);
    take(P.h0b, nh * f);
    if (!backward) {
        take(P.yb, nv * f);
    } else {
        take(P.dyb, nv * f);
        take(P.dqb, nq * f);
        take(P.dkbuf, nq * f);
        take(P.dvbuf, nv * f);
        take(P.dlab, BH * T * f);
        take(P.dh0b, nh * f);
    }
    P.total = o;
    return P;
}

size_t workspace_bytes(const ssd_shape *s, bool backward, int cus)
{
    if (s->B == 0 || s->T == 0) return 0;
    if (needs_split(s)) return make_split_layout(s, backward, cus).total;
    return make_layout(s, backward, cus).off[SSD_WS_REGIONS];
}

}  // namespace ssd

extern "C" {

size_t ssd_fwd_workspace_size(const ssd_shape *shape)
{
    if (ssd::check_shape(shape) != SSD_OK) return (size_t)-1;
    return ssd::workspace_bytes(shape, false, ssd::device_cus());
}

size_t ssd_bwd_workspace_size(const ssd_shape *shape)
{
    if (ssd::check_shape(shape) != SSD_OK) return (size_t)-1;
    return ssd::workspace_bytes(shape, true, ssd::device_cus());
}

int ssd_workspace_layout(const ssd_shape *shape, int backward, size_t offsets[SSD_WS_REGIONS + 1])
{
    if (!offsets) return SSD_ERR_NULL;
    const int rc = ssd::check_shape(shape);
    if (rc != SSD_OK) return rc;
    if (ssd::needs_split(shape)) return SSD_ERR_UNSUPPORTED;   // regions of the direct path only
    const ssd::Layout L = ssd::make_layout(shape, backward != 0, ssd::device_cus());
    for (int i = 0; i <= SSD_WS_REGIONS; ++i) offsets[i] = L.off[i];
    return SSD_OK;
}

size_t mamba_fwd_workspace_size(const mamba_shape *shape)
{
    if (ssd::mamba_check_shape(shape) != SSD_OK) return 0;
    return ssd::mamba_plan(shape, ssd::device_cus()).total;
}

size_t mamba_bwd_workspace_size(const mamba_shape *shape)
{
    if (ssd::mamba_check_shape(shape) != SSD_OK || shape->L > 65535 * ssd::kMambaBwdSeg) return 0;
    return ssd::mamba_bwd_plan(shape, ssd::device_cus()).total;
}

int ssd_fwd_state_stride(const ssd_shape *shape)
{
    if (ssd::check_shape(shape) != SSD_OK || ssd::needs_split(shape)) return -1;
    bool pair = false;
    if (ssd::fwd_pair_mode(shape, ssd::device_cus(), &pair) != SSD_OK) return -1;
    return pair ? 2 : 1;
}

const char *ssd_strerror(int status)
{
    switch (status) {
    case SSD_OK: return "success";
    case SSD_ERR_NULL: return "a required pointer is NULL";
    case SSD_ERR_SHAPE: return "invalid shape (negative size, G < 1, H not a multiple of G, or too large)";
    case SSD_ERR_UNSUPPORTED:
        return "unsupported shape (dk and dv must be in 1..256) or SSD_FWD_CHUNK setting (unset, 64 or 128)";
    case SSD_ERR_WORKSPACE: return "workspace smaller than the size query requires";
    case SSD_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case SSD_ERR_DEVICE: return "HIP launch or runtime error";
    default: return "unknown status";
    }
}

int ssd_chunk_size(void) { return SSD_CHUNK; }

}  // extern "C"
