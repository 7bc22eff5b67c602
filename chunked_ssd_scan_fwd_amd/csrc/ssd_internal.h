// Internal host-side declarations shared by the validation unit and the HIP
// units.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "ssd.h"

namespace ssd {

constexpr int kChunk = SSD_CHUNK;   // steps per chunk = wavefront width
constexpr int64_t kMaxDim = 128;    // largest dk / dv the kernels take directly
constexpr int64_t kMaxApiDim = 256; // largest dk / dv of the ABI (split into <= 128 blocks)

struct Layout {
    int64_t NC = 0;      // chunks per sequence, ceil(T / 64)
    int64_t E = 0;       // dk * dv
    int64_t Epad = 0;    // E rounded up to a multiple of 64 (slab stride, floats)
    // byte offsets: decay weights, states, dstates, split partial sums, total
    size_t off[SSD_WS_REGIONS + 1] = {0, 0, 0, 0, 0};
    size_t cdec_off = 0;   // per-chunk decays, inside the decay region
    // The output and gradient kernels take one block per (b, g, chunk) and loop
    // over the group's heads.  With fewer such blocks than CUs a group's heads
    // are split over `hsplit` blocks of `hpb` heads each (the last may hold
    // fewer); the gradient kernel then writes per-split partial sums of dq and
    // dk, [2][hsplit][nqk_pad] floats at byte offset off[3], which a small
    // kernel adds up in split order.
    int hsplit = 1;
    int hpb = 1;
    int64_t nqk_pad = 0;     // B*G*T*dk rounded up to a multiple of 64
    // Segment end states of a segmented state scan (see ScanPlan), at byte
    // offset ends_off inside region 3: [ndir][nseg][B*H][Epad] floats; then at
    // segd_off, [2][B*H][NC] floats: per direction and chunk (in scan order),
    // the product of the chunk decays from its segment's start up to it.
    size_t ends_off = 0;
    size_t segd_off = 0;
};

// Launch plan of the state scan for one launch over `ndir` directions.  The
// scan walks the chunks in order, so its grid (one block per state tile)
// can leave most CUs idle on small problems.  Then the tiles are first made
// 32 wide (`narrow`), and if the grid still fills at most half the CUs the
// chunk sequence is cut into `nseg` segments of `seg_len` chunks (a power of
// two, each segment at least kMinSegChunks long) that run in parallel from a
// zero state (the first from the true initial state); a fix-up pass then
// adds each segment's decayed entering state to its chunk states.
constexpr int64_t kMinSegChunks = 8;
constexpr int kMaxSegs = 64;
struct ScanPlan {
    bool narrow = false;
    int nseg = 1;
    int64_t seg_len = 0;
    int64_t blocks = 0;   // blocks of the launch
};
ScanPlan scan_plan(const ssd_shape *s, int ndir, int cus);

// Whether the forward of a direct (dk, dv <= 128) shape runs on chunk pairs
// by the library's own choice: full 128-column states (pad(dv) = 128) and at
// least two pair units (b, g, pair of chunks) per CU.  Its state scan then
// stores the states of even chunks only.
bool fwd_pairs(const ssd_shape *s, int cus);

// The forward's chunk length as the environment variable SSD_FWD_CHUNK sets
// it, read at each call: 0 when unset or empty (the library chooses per
// shape), 64, 128, or -1 for any other value.
int fwd_chunk_setting();

// Whether the forward of a direct shape runs on chunk pairs under that
// setting (SSD_OK and *pair), or SSD_ERR_UNSUPPORTED for an invalid setting
// or for 128 where the pair kernel does not take the shape (pad(dv) must be
// 64 or 128).
int fwd_pair_mode(const ssd_shape *s, int cus, bool *pair);

// The same check for a whole forward, direct or cut into column blocks
// (every dv block must suit the pair kernel under 128), made before anything
// is enqueued.
int fwd_chunk_check(const ssd_shape *s);

// Heads per block and number of splits for a shape on a device with `cus`
// compute units (see Layout).
void head_split(const ssd_shape *s, int64_t NC, int cus, int *hsplit, int *hpb);

// SSD_OK, SSD_ERR_NULL (shape == NULL), SSD_ERR_SHAPE or SSD_ERR_UNSUPPORTED.
int check_shape(const ssd_shape *s);

// Workspace layout for a valid shape with dk, dv <= kMaxDim on a device with
// `cus` compute units.  Empty shapes give total == 0.
Layout make_layout(const ssd_shape *s, bool backward, int cus);

// Shapes with dk or dv above kMaxDim run as nI x nJ sub-problems on column
// blocks of at most kMaxDim: dk block I covers columns i0[I] .. i0[I] +
// dkb[I] of q, k (rows of h0), dv block J columns j0[J] .. j0[J] + dvb[J] of
// v, dy, y (columns of h0).  The outputs are sums of the sub-problems'
// (y over I; dq, dk over J; dv over I; dlog_alpha over both; dh0 block by
// block), so the workspace holds the largest sub-problem's workspace and
// contiguous copies of one block of each operand and output.
struct SplitLayout {
    int nI = 1, nJ = 1;
    int64_t i0[2] = {0, 0}, dkb[2] = {0, 0}, j0[2] = {0, 0}, dvb[2] = {0, 0};
    int64_t dkm = 0, dvm = 0;   // largest block widths
    // byte offsets: sub-problem workspace, q, k, v, h0, y (fwd) or dy, dq, dk,
    // dv, dlog_alpha, dh0 blocks (bwd), total
    size_t sub = 0, qb = 0, kb = 0, vb = 0, h0b = 0, yb = 0, dyb = 0, dqb = 0, dkbuf = 0, dvbuf = 0, dlab = 0,
           dh0b = 0, total = 0;
    size_t sub_bytes = 0;
};
bool needs_split(const ssd_shape *s);
ssd_shape sub_shape(const ssd_shape *s, const SplitLayout &P, int I, int J);
SplitLayout make_split_layout(const ssd_shape *s, bool backward, int cus);

// Total workspace bytes for any valid shape (direct or split).
size_t workspace_bytes(const ssd_shape *s, bool backward, int cus);

// Compute units of the current HIP device, read once per device and cached;
// 256 (MI355X) when no device can be queried.  Defined in the HIP unit.
int device_cus();

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---- selective (Mamba-style) scan
// Shape checks: SSD_ERR_NULL, SSD_ERR_SHAPE (negative B or L, D or N below
// 1, index range), SSD_ERR_UNSUPPORTED (N above MAMBA_MAX_STATE, B above
// 65535, L above 65535 * kMambaMaxSeg, D above 2^20).
int mamba_check_shape(const mamba_shape *s);
// The sequence is cut into nseg segments of seg_len steps (the last may be
// shorter) that run in parallel: one thread per (b, channel, segment).  A
// first pass forms each segment's end state from zero, a carry pass turns
// them, in place, into the state entering each segment, and the output pass
// rescans every segment from its entering state.
constexpr int64_t kMambaMaxSeg = 256;   // longest segment (its B, C rows sit in LDS)
struct MambaPlan {
    int64_t nseg = 1, seg_len = 0;
    // byte offsets in the workspace: end / entering states float [B][nseg][N][D],
    // summed delta of each segment float [B][nseg][D], total
    size_t hend = 0, sdl = 0, total = 0;
};
MambaPlan mamba_plan(const mamba_shape *s, int cus);
// The backward cuts the sequence into segments of kMambaBwdSeg steps (their
// states are held in registers) and splits each segment's channel chunks of
// kMambaBwdChans over nsplit blocks.  Byte offsets: forward end / entering states
// [B][nseg][N][D], summed deltas [B][nseg][D], adjoints entering from the
// right [B][nseg][D][N], dA partials [B][nseg][D][N], dDskip partials
// [B][nseg][D], and with nsplit > 1 the dB / dC partials [nsplit][B][L][2][N].
constexpr int kMambaBwdSeg = 32;
constexpr int kMambaBwdChans = 64;
struct MambaBwdPlan {
    int64_t nseg = 0;
    int nsplit = 1;
    size_t hend = 0, sdl = 0, gl = 0, dApart = 0, dDpart = 0, dBC = 0, total = 0;
};
MambaBwdPlan mamba_bwd_plan(const mamba_shape *s, int cus);

// Padded MFMA tile width (32, 64 or 128) for dk / dv in 1..128.
inline int pad_dim(int64_t d) { return d <= 32 ? 32 : (d <= 64 ? 64 : 128); }

}  // namespace ssd
