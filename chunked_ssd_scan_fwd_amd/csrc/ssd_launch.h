// Host-side launch plumbing shared by the kernel units: the resolved problem
// (shape, workspace regions, padded tile sizes), the caller-owned kernel
// timer, the launch helper and the compile-time dispatch over tile sizes.
// Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <stdint.h>
#include <tuple>
#include <vector>

#include "ssd.h"
#include "ssd_internal.h"

namespace ssd {

enum KernelId { KID_SCAN = 0, KID_OUTPUT, KID_SCAN2, KID_GRADS, KID_SCANR, KID_AUX, KID_COUNT };

}  // namespace ssd

// Per-kernel HIP-event timing owned by the caller (see ssd_timer_create).
struct ssd_timer {
    unsigned mask = 0;   // bit kid: time kernel kid
    std::vector<hipEvent_t> pool;
    std::vector<hipEvent_t> pending[ssd::KID_COUNT][2];
    double total[ssd::KID_COUNT] = {};
    int64_t count[ssd::KID_COUNT] = {};
};

namespace ssd {

inline hipEvent_t timer_event(ssd_timer *tm)
{
    if (!tm->pool.empty()) {
        hipEvent_t e = tm->pool.back();
        tm->pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Launches f on st.  When `tm` times kernel kid, the start and stop events
// are bound to the kernel's own dispatch through hipExtLaunchKernel, so they
// time the kernel alone and put no extra packets between kernels.
template <typename... P, typename... A>
inline void launch(ssd_timer *tm, int kid, void (*f)(P...), dim3 grid, dim3 blk, hipStream_t st, A... a)
{
    static_assert(sizeof...(P) == sizeof...(A), "argument count");
    std::tuple<P...> args{static_cast<P>(a)...};
    void *ptrs[sizeof...(P)];
    std::apply([&](auto &...x) {
        int i = 0;
        ((ptrs[i++] = static_cast<void *>(&x)), ...);
    }, args);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (tm && kid >= 0 && ((tm->mask >> kid) & 1u)) {
        e0 = timer_event(tm);
        e1 = timer_event(tm);
        if (!e0 || !e1) {
            if (e0) tm->pool.push_back(e0);
            if (e1) tm->pool.push_back(e1);
            e0 = e1 = nullptr;
        }
    }
    // A failed launch is also this thread's last HIP error, which
    // launch_status() reports; its events were never recorded and go back.
    const hipError_t rc = hipExtLaunchKernel(reinterpret_cast<const void *>(f), grid, blk, ptrs, 0, st, e0, e1, 0);
    if (e0 && e1) {
        auto &to0 = rc == hipSuccess ? tm->pending[kid][0] : tm->pool;
        auto &to1 = rc == hipSuccess ? tm->pending[kid][1] : tm->pool;
        to0.push_back(e0);
        to1.push_back(e1);
    }
}

inline int launch_status()
{
    return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_DEVICE;
}

// One instantiation per padded tile size (32, 64 or 128 for dk and dv) and
// per addressing mode: exact (dk, dv equal to their padded sizes: index
// arithmetic on constants), vec (dk, dv multiples of 4: 16-byte accesses) or
// scalar.
#define SSD_DISPATCH_DIMS(DKP_, DVP_, BODY)                                          \
    do {                                                                             \
        if (DKP_ == 32 && DVP_ == 32) { constexpr int KP = 32, VP = 32; BODY; }       \
        else if (DKP_ == 32 && DVP_ == 64) { constexpr int KP = 32, VP = 64; BODY; }  \
        else if (DKP_ == 32 && DVP_ == 128) { constexpr int KP = 32, VP = 128; BODY; } \
        else if (DKP_ == 64 && DVP_ == 32) { constexpr int KP = 64, VP = 32; BODY; }  \
        else if (DKP_ == 64 && DVP_ == 64) { constexpr int KP = 64, VP = 64; BODY; }  \
        else if (DKP_ == 64 && DVP_ == 128) { constexpr int KP = 64, VP = 128; BODY; } \
        else if (DKP_ == 128 && DVP_ == 32) { constexpr int KP = 128, VP = 32; BODY; } \
        else if (DKP_ == 128 && DVP_ == 64) { constexpr int KP = 128, VP = 64; BODY; } \
        else { constexpr int KP = 128, VP = 128; BODY; }                              \
    } while (0)

#define SSD_DISPATCH(P_, BODY)                                                     \
    do {                                                                           \
        if ((P_).exact) {                                                          \
            constexpr bool VE = true, EXD = true;                                  \
            SSD_DISPATCH_DIMS((P_).DKP, (P_).DVP, BODY);                           \
        } else if ((P_).vec) {                                                     \
            constexpr bool VE = true, EXD = false;                                 \
            SSD_DISPATCH_DIMS((P_).DKP, (P_).DVP, BODY);                           \
        } else {                                                                   \
            constexpr bool VE = false, EXD = false;                                \
            SSD_DISPATCH_DIMS((P_).DKP, (P_).DVP, BODY);                           \
        }                                                                          \
    } while (0)

// A problem whose dk and dv are at most kBlockDim, resolved for launching.
struct Problem {
    ssd_shape s;
    Layout L;
    int DKP, DVP;
    bool vec;     // dk and dv multiples of 4: 16-byte loads
    bool exact;   // dk == DKP and dv == DVP: the kernels' index arithmetic on constants
    int cus;      // compute units of the device
    float *wts, *cdec;   // per-position decay weights and per-chunk decays (scan input)
    float *states, *dstates;
    float *parts;   // split partial sums of dq, dk (backward with hsplit > 1), else null
    float *ends;    // segment end states of a segmented scan
    float *segd;    // per-chunk decay products within segments (segmented scan)
    // The forward runs on chunk pairs: its scan stores the states of even
    // chunks only and the pair output kernel takes the odd chunks' inter term
    // from them.
    bool pair;
    ssd_timer *timer;
};

// With `prep`, the per-chunk decay weights from log_alpha first; then the
// fused chunk-state + state-pass scan over the directions in `dirs`: 1 =
// forward only (fills `states` with S_in), 3 = both in one launch (also
// fills `dstates` with dS_out and writes dh0), 2 = reverse only (dstates and
// dh0; `states` is not touched, the weights must be in place).  The forward
// direction stores S_in of every chunk (kStoreAll), of even chunks only
// (kStoreEven: the forward on chunk pairs) or of odd chunks only (kStoreOdd:
// completing what such a forward left).
enum StoreSet { kStoreAll = 0, kStoreEven = 1, kStoreOdd = 2 };
int run_scan(const Problem &P, int dirs, bool prep, StoreSet store, const float *q, const float *k, const float *v,
             const float *dy, const float *la, const float *h0, float *dh0, hipStream_t st);

// Output of every chunk: y = intra-chunk term + diag(e^b) Q S_in.  With
// P.pair, from the states of even chunks (run_pair_output).
int run_output(const Problem &P, const float *q, const float *k, const float *v, const float *la, float *y,
               hipStream_t st);
int run_pair_output(const Problem &P, const float *q, const float *k, const float *v, const float *la, float *y,
                    hipStream_t st);

// Gradients of every chunk from the states and state gradients in the
// workspace; with a head split, also the fixed-order sum of the partials.
int run_grads(const Problem &P, const float *q, const float *k, const float *v, const float *dy, const float *la,
              float *dq, float *dk, float *dv, float *dla, hipStream_t st);

}  // namespace ssd
