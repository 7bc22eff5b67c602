// The C ABI of the SSD scan: argument checks, workspace resolution and the
// launch sequence of the forward and backward, and the caller-owned kernel
// timer.  The kernels live in k_scan.hip, k_output.hip and k_grads.hip.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <new>

#include "ssd.h"
#include "ssd_internal.h"
#include "ssd_launch.h"

namespace ssd {

constexpr int NTZ = 256;

// Fill n floats with zero (dh0 when T == 0).
__global__ __launch_bounds__(NTZ) void k_zero(float *__restrict__ p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * NTZ + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

constexpr int kMaxDevices = 64;
constexpr int kDefaultCUs = 256;

int device_cus()
{
    // A memo of a device property (each entry written once with the same
    // value), not state that any result depends on beyond the device itself.
    static std::atomic<int> cache[kMaxDevices];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return kDefaultCUs;
    }
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return kDefaultCUs;
    }
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Workspace of ssd_fwd_noalloc: a file-scope device array, one copy per GPU
// the library runs on, held until the process ends.  In host code its name
// stands for a host-side shadow, never for device memory: every use goes
// through the device address that hipGetSymbolAddress returns for the
// current device (static_ws_ptr), never through the name.
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_WORKSPACE_BYTES];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and cached; NULL if it cannot be had.
static void *static_ws_ptr()
{
    static std::atomic<void *> cache[kMaxDevices];
    static std::mutex mu;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    void *p = cache[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(mu);
    p = cache[dev].load(std::memory_order_acquire);
    if (p) return p;
    void *addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) {
        (void)hipGetLastError();
        return nullptr;
    }
    cache[dev].store(addr, std::memory_order_release);
    return addr;
}

static int prepare(const ssd_shape *shape, bool backward, void *ws, size_t ws_bytes, ssd_timer *tm, Problem *P)
{
    P->s = *shape;
    P->cus = device_cus();
    P->L = make_layout(shape, backward, P->cus);
    if (ws_bytes < P->L.off[SSD_WS_REGIONS]) return SSD_ERR_WORKSPACE;
    if (P->L.off[SSD_WS_REGIONS] > 0) {
        if (!ws) return SSD_ERR_NULL;
        if (!aligned16(ws)) return SSD_ERR_ALIGN;
    }
    P->DKP = pad_dim(shape->dk);
    P->DVP = pad_dim(shape->dv);
    P->vec = (shape->dk % 4) == 0 && (shape->dv % 4) == 0;
    P->exact = shape->dk == P->DKP && shape->dv == P->DVP;
    char *w = static_cast<char *>(ws);
    P->wts = reinterpret_cast<float *>(w + P->L.off[0]);
    P->cdec = reinterpret_cast<float *>(w + P->L.cdec_off);
    P->states = reinterpret_cast<float *>(w + P->L.off[1]);
    P->dstates = backward ? reinterpret_cast<float *>(w + P->L.off[2]) : nullptr;
    P->parts = backward && P->L.hsplit > 1 ? reinterpret_cast<float *>(w + P->L.off[3]) : nullptr;
    P->timer = tm;
    return SSD_OK;
}

static int fwd_impl(const ssd_shape *shape, const float *q, const float *k, const float *v, const float *log_alpha,
                    const float *h0, float *y, void *workspace, size_t workspace_bytes, void *stream, ssd_timer *tm)
{
    int rc = check_shape(shape);
    if (rc != SSD_OK) return rc;
    const ssd_shape &s = *shape;
    if (s.B == 0 || s.T == 0) return SSD_OK;   // y has no elements
    if (!q || !k || !v || !log_alpha || !h0 || !y) return SSD_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(log_alpha) || !aligned16(h0) ||
        !aligned16(y))
        return SSD_ERR_ALIGN;
    Problem P;
    rc = prepare(shape, false, workspace, workspace_bytes, tm, &P);
    if (rc != SSD_OK) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    rc = run_scan(P, 1, true, q, k, v, nullptr, log_alpha, h0, nullptr, st);
    if (rc != SSD_OK) return rc;
    return run_output(P, q, k, v, log_alpha, y, st);
}

// Backward launches.  With `reuse`, the workspace already holds the decay
// weights and S_in of every chunk as ssd_fwd wrote them for these inputs, so
// only the reverse state pass and the gradient kernel run.
static int bwd_impl(const ssd_shape *shape, const float *q, const float *k, const float *v,
                    const float *log_alpha, const float *h0, const float *dy, float *dq, float *dk, float *dv,
                    float *dlog_alpha, float *dh0, void *workspace, size_t workspace_bytes, void *stream, bool reuse,
                    ssd_timer *tm)
{
    int rc = check_shape(shape);
    if (rc != SSD_OK) return rc;
    const ssd_shape &s = *shape;
    if (s.B == 0) return SSD_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (s.T == 0) {
        // Only dh0 has elements, and it is zero.
        if (!dh0) return SSD_ERR_NULL;
        if (!aligned16(dh0)) return SSD_ERR_ALIGN;
        const int64_t n = s.B * s.H * s.dk * s.dv;
        launch(tm, KID_AUX, k_zero, dim3((unsigned)((n + NTZ - 1) / NTZ)), dim3(NTZ), st, dh0, n);
        return launch_status();
    }
    if (!q || !k || !v || !log_alpha || !h0 || !dy || !dq || !dk || !dv || !dlog_alpha || !dh0)
        return SSD_ERR_NULL;
    const void *ptrs[] = {q, k, v, log_alpha, h0, dy, dq, dk, dv, dlog_alpha, dh0};
    for (const void *p : ptrs)
        if (!aligned16(p)) return SSD_ERR_ALIGN;
    Problem P;
    rc = prepare(shape, true, workspace, workspace_bytes, tm, &P);
    if (rc != SSD_OK) return rc;
    // dS_out (reverse) of every chunk and dh0; without reuse also the decay
    // weights and S_in (forward), the latter in the same launch.
    rc = run_scan(P, reuse ? 2 : 3, !reuse, q, k, v, dy, log_alpha, h0, dh0, st);
    if (rc != SSD_OK) return rc;
    return run_grads(P, q, k, v, dy, log_alpha, dq, dk, dv, dlog_alpha, st);
}

static const char *kKernelNames[KID_COUNT] = {"state_scan", "chunk_output", "state_scan_bidir",
                                              "bwd_grads", "state_scan_rev", "aux"};

static void collect_timing(ssd_timer *tm)
{
    for (int kid = 0; kid < KID_COUNT; ++kid) {
        auto &A = tm->pending[kid][0];
        auto &B = tm->pending[kid][1];
        for (size_t i = 0; i < A.size(); ++i) {
            float ms = 0.f;
            hipEventSynchronize(B[i]);
            if (hipEventElapsedTime(&ms, A[i], B[i]) == hipSuccess) {
                tm->total[kid] += ms;
                tm->count[kid] += 1;
            }
            tm->pool.push_back(A[i]);
            tm->pool.push_back(B[i]);
        }
        A.clear();
        B.clear();
    }
}

}  // namespace ssd

using namespace ssd;

extern "C" {

int ssd_fwd(const ssd_shape *shape, const float *q, const float *k, const float *v, const float *log_alpha,
            const float *h0, float *y, void *workspace, size_t workspace_bytes, void *stream)
{
    return fwd_impl(shape, q, k, v, log_alpha, h0, y, workspace, workspace_bytes, stream, nullptr);
}

int ssd_fwd_noalloc(const ssd_shape *shape, const float *q, const float *k, const float *v, const float *log_alpha,
                    const float *h0, float *y, void *stream)
{
    // The same checks and launches as ssd_fwd; the workspace is the static
    // array.  Nothing is allocated, and the forward's workspace needs no
    // clearing (every region is written before it is read).
    int rc = check_shape(shape);
    if (rc != SSD_OK) return rc;
    const size_t need = make_layout(shape, false, device_cus()).off[SSD_WS_REGIONS];
    if (need > SSD_NOALLOC_WORKSPACE_BYTES) return SSD_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need > 0) {
        ws = static_ws_ptr();
        if (!ws) return SSD_ERR_DEVICE;
    }
    return fwd_impl(shape, q, k, v, log_alpha, h0, y, ws, SSD_NOALLOC_WORKSPACE_BYTES, stream, nullptr);
}

int ssd_bwd(const ssd_shape *shape, const float *q, const float *k, const float *v, const float *log_alpha,
            const float *h0, const float *dy, float *dq, float *dk, float *dv, float *dlog_alpha, float *dh0,
            void *workspace, size_t workspace_bytes, void *stream)
{
    return bwd_impl(shape, q, k, v, log_alpha, h0, dy, dq, dk, dv, dlog_alpha, dh0, workspace, workspace_bytes,
                    stream, false, nullptr);
}

int ssd_bwd_from_fwd(const ssd_shape *shape, const float *q, const float *k, const float *v,
                     const float *log_alpha, const float *h0, const float *dy, float *dq, float *dk, float *dv,
                     float *dlog_alpha, float *dh0, void *workspace, size_t workspace_bytes, void *stream)
{
    return bwd_impl(shape, q, k, v, log_alpha, h0, dy, dq, dk, dv, dlog_alpha, dh0, workspace, workspace_bytes,
                    stream, true, nullptr);
}

ssd_timer *ssd_timer_create(int mask)
{
    ssd_timer *tm = new (std::nothrow) ssd_timer;
    if (tm) tm->mask = static_cast<unsigned>(mask);
    return tm;
}

int ssd_timer_destroy(ssd_timer *tm)
{
    if (!tm) return SSD_ERR_NULL;
    collect_timing(tm);
    for (hipEvent_t e : tm->pool) hipEventDestroy(e);
    delete tm;
    return SSD_OK;
}

int ssd_timer_reset(ssd_timer *tm)
{
    if (!tm) return SSD_ERR_NULL;
    collect_timing(tm);
    for (int i = 0; i < KID_COUNT; ++i) {
        tm->total[i] = 0.0;
        tm->count[i] = 0;
    }
    return SSD_OK;
}

int ssd_timer_read(ssd_timer *tm, int kid, double *total_ms, int64_t *count)
{
    if (!tm || !total_ms || !count) return SSD_ERR_NULL;
    if (kid < 0 || kid >= KID_COUNT) return SSD_ERR_SHAPE;
    collect_timing(tm);
    *total_ms = tm->total[kid];
    *count = tm->count[kid];
    return SSD_OK;
}

int ssd_fwd_timed(ssd_timer *tm, const ssd_shape *shape, const float *q, const float *k, const float *v,
                  const float *log_alpha, const float *h0, float *y, void *workspace, size_t workspace_bytes,
                  void *stream)
{
    if (!tm) return SSD_ERR_NULL;
    return fwd_impl(shape, q, k, v, log_alpha, h0, y, workspace, workspace_bytes, stream, tm);
}

int ssd_bwd_timed(ssd_timer *tm, const ssd_shape *shape, const float *q, const float *k, const float *v,
                  const float *log_alpha, const float *h0, const float *dy, float *dq, float *dk, float *dv,
                  float *dlog_alpha, float *dh0, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!tm) return SSD_ERR_NULL;
    return bwd_impl(shape, q, k, v, log_alpha, h0, dy, dq, dk, dv, dlog_alpha, dh0, workspace, workspace_bytes,
                    stream, false, tm);
}

int ssd_kernel_count(void) { return KID_COUNT; }

const char *ssd_kernel_name(int kid)
{
    if (kid < 0 || kid >= KID_COUNT) return "unknown";
    return kKernelNames[kid];
}

}  // extern "C"
