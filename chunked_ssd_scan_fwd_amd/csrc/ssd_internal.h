// Internal host-side declarations shared by the validation unit and the HIP
// units.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "ssd.h"

namespace ssd {

constexpr int kChunk = SSD_CHUNK;   // steps per chunk = wavefront width
constexpr int64_t kMaxDim = 128;    // largest dk / dv the kernels take directly

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
};

// Heads per block and number of splits for a shape on a device with `cus`
// compute units (see Layout).
void head_split(const ssd_shape *s, int64_t NC, int cus, int *hsplit, int *hpb);

// SSD_OK, SSD_ERR_NULL (shape == NULL), SSD_ERR_SHAPE or SSD_ERR_UNSUPPORTED.
int check_shape(const ssd_shape *s);

// Workspace layout for a valid shape on a device with `cus` compute units.
// Empty shapes give total == 0.
Layout make_layout(const ssd_shape *s, bool backward, int cus);

// Compute units of the current HIP device, read once per device and cached;
// 256 (MI355X) when no device can be queried.  Defined in the HIP unit.
int device_cus();

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Padded MFMA tile width (32, 64 or 128) for dk / dv in 1..128.
inline int pad_dim(int64_t d) { return d <= 32 ? 32 : (d <= 64 ? 64 : 128); }

}  // namespace ssd
