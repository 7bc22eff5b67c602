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

constexpr int NTC = 256;

// dst[b][r][c] = src[b][r][c] (or += with `add`) for b < nb, r < rows,
// c < cols; batch and row strides in floats.  Moves column blocks of the
// operands and outputs of problems with dk or dv above 128.
__global__ __launch_bounds__(NTC) void k_copy_block(float *__restrict__ dst, int64_t dbs, int64_t dld,
                                                    const float *__restrict__ src, int64_t sbs, int64_t sld,
                                                    int64_t nb, int64_t rows, int64_t cols, int add)
{
    const int64_t n = nb * rows * cols;
    for (int64_t i = (int64_t)blockIdx.x * NTC + threadIdx.x; i < n; i += (int64_t)gridDim.x * NTC) {
        const int64_t c = i % cols, t = i / cols, r = t % rows, b = t / rows;
        const float x = src[b * sbs + r * sld + c];
        float *d = dst + b * dbs + r * dld + c;
        *d = add ? *d + x : x;
    }
}

static int copy_block(ssd_timer *tm, hipStream_t st, float *dst, int64_t dbs, int64_t dld, const float *src,
                      int64_t sbs, int64_t sld, int64_t nb, int64_t rows, int64_t cols, bool add)
{
    const int64_t n = nb * rows * cols;
    if (n == 0) return SSD_OK;
    const int64_t blocks = (n + NTC - 1) / NTC;
    launch(tm, KID_AUX, k_copy_block, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(NTC), st, dst, dbs,
           dld, src, sbs, sld, nb, rows, cols, (int)add);
    return launch_status();
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

// `fwd_states`: the forward's state layout matters to this call (a forward,
// or a backward that reuses what the forward stored).
static int prepare(const ssd_shape *shape, bool backward, bool fwd_states, void *ws, size_t ws_bytes,
                   ssd_timer *tm, Problem *P)
{
    P->s = *shape;
    P->cus = device_cus();
    // Chunk pairs where they measured faster: full 128-column states (the
    // pair kernel's P is formed once per two steps) and at least two pair
    // units per CU (its larger set-up, Q K^T over 128 positions, is then
    // loaded under the previous unit's MFMAs).  g2h8_d128 T8192: forward
    // 279 -> 257 us; at one unit per CU (T2048) or dv = 64 it was slower.
    // SSD_FWD_CHUNK overrides the choice.
    P->pair = false;
    if (fwd_states) {
        const int rc = fwd_pair_mode(shape, P->cus, &P->pair);
        if (rc != SSD_OK) return rc;
    }
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
    P->ends = reinterpret_cast<float *>(w + P->L.ends_off);
    P->segd = reinterpret_cast<float *>(w + P->L.segd_off);
    P->timer = tm;
    return SSD_OK;
}

static int fwd_split(const ssd_shape &s, const float *q, const float *k, const float *v, const float *log_alpha,
                     const float *h0, float *y, void *workspace, size_t ws_bytes, hipStream_t st, ssd_timer *tm);
static int bwd_split(const ssd_shape &s, const float *q, const float *k, const float *v, const float *log_alpha,
                     const float *h0, const float *dy, float *dq, float *dk, float *dv, float *dla, float *dh0,
                     void *workspace, size_t ws_bytes, hipStream_t st, ssd_timer *tm);

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
    hipStream_t st = static_cast<hipStream_t>(stream);
    rc = fwd_chunk_check(shape);
    if (rc != SSD_OK) return rc;
    if (needs_split(shape)) return fwd_split(s, q, k, v, log_alpha, h0, y, workspace, workspace_bytes, st, tm);
    Problem P;
    rc = prepare(shape, false, true, workspace, workspace_bytes, tm, &P);
    if (rc != SSD_OK) return rc;
    rc = run_scan(P, 1, true, P.pair ? kStoreEven : kStoreAll, q, k, v, nullptr, log_alpha, h0, nullptr, st);
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
    // Problems split into column blocks recompute everything (no reuse).
    if (needs_split(shape))
        return bwd_split(s, q, k, v, log_alpha, h0, dy, dq, dk, dv, dlog_alpha, dh0, workspace, workspace_bytes, st,
                         tm);
    Problem P;
    rc = prepare(shape, true, reuse, workspace, workspace_bytes, tm, &P);
    if (rc != SSD_OK) return rc;
    // dS_out (reverse) of every chunk and dh0; without reuse also the decay
    // weights and S_in (forward), the latter in the same launch.  A forward
    // on chunk pairs left S_in of even chunks only: the forward direction
    // runs again, storing the odd chunks' states.
    if (reuse && P.pair)
        rc = run_scan(P, 3, false, kStoreOdd, q, k, v, dy, log_alpha, h0, dh0, st);
    else
        rc = run_scan(P, reuse ? 2 : 3, !reuse, kStoreAll, q, k, v, dy, log_alpha, h0, dh0, st);
    if (rc != SSD_OK) return rc;
    return run_grads(P, q, k, v, dy, log_alpha, dq, dk, dv, dlog_alpha, st);
}

// Workspace regions of a split problem, resolved against a caller's workspace.
static int split_prepare(const ssd_shape &s, bool backward, void *ws, size_t ws_bytes, SplitLayout *L)
{
    *L = make_split_layout(&s, backward, device_cus());
    if (ws_bytes < L->total) return SSD_ERR_WORKSPACE;
    if (!ws) return SSD_ERR_NULL;
    if (!aligned16(ws)) return SSD_ERR_ALIGN;
    return SSD_OK;
}

// Forward of a problem with dk or dv above 128: for each dv block J and dk
// block I, the sub-problem on (q_I, k_I, v_J, log_alpha, h0[I, J]) gives y_IJ,
// and y[:, :, :, J] = sum over I of y_IJ, added in ascending I.
static int fwd_split(const ssd_shape &s, const float *q, const float *k, const float *v, const float *log_alpha,
                     const float *h0, float *y, void *workspace, size_t ws_bytes, hipStream_t st, ssd_timer *tm)
{
    SplitLayout L;
    int rc = split_prepare(s, false, workspace, ws_bytes, &L);
    if (rc != SSD_OK) return rc;
    char *w = static_cast<char *>(workspace);
    float *qb = reinterpret_cast<float *>(w + L.qb), *kb = reinterpret_cast<float *>(w + L.kb);
    float *vb = reinterpret_cast<float *>(w + L.vb), *h0b = reinterpret_cast<float *>(w + L.h0b);
    float *yb = reinterpret_cast<float *>(w + L.yb);
    const int64_t nqr = s.B * s.G * s.T, nvr = s.B * s.H * s.T, BH = s.B * s.H;
    for (int J = 0; J < L.nJ && rc == SSD_OK; ++J) {
        const int64_t j0 = L.j0[J], dvJ = L.dvb[J];
        rc = copy_block(tm, st, vb, 0, dvJ, v + j0, 0, s.dv, 1, nvr, dvJ, false);
        for (int I = 0; I < L.nI && rc == SSD_OK; ++I) {
            const int64_t i0 = L.i0[I], dkI = L.dkb[I];
            rc = copy_block(tm, st, qb, 0, dkI, q + i0, 0, s.dk, 1, nqr, dkI, false);
            if (rc == SSD_OK) rc = copy_block(tm, st, kb, 0, dkI, k + i0, 0, s.dk, 1, nqr, dkI, false);
            if (rc == SSD_OK)
                rc = copy_block(tm, st, h0b, dkI * dvJ, dvJ, h0 + i0 * s.dv + j0, s.dk * s.dv, s.dv, BH, dkI, dvJ,
                                false);
            const ssd_shape t = sub_shape(&s, L, I, J);
            if (rc == SSD_OK) rc = fwd_impl(&t, qb, kb, vb, log_alpha, h0b, yb, w + L.sub, L.sub_bytes, st, tm);
            if (rc == SSD_OK) rc = copy_block(tm, st, y + j0, 0, s.dv, yb, 0, dvJ, 1, nvr, dvJ, I > 0);
        }
    }
    return rc;
}

// Backward of a problem with dk or dv above 128: each sub-problem (I, J) of
// fwd_split gives its five gradients; dq and dk of block I are summed over J,
// dv of block J over I, dlog_alpha over all of them (in the loop order: J
// outer, I inner), and dh0 is taken block by block.
static int bwd_split(const ssd_shape &s, const float *q, const float *k, const float *v, const float *log_alpha,
                     const float *h0, const float *dy, float *dq, float *dk, float *dv, float *dla, float *dh0,
                     void *workspace, size_t ws_bytes, hipStream_t st, ssd_timer *tm)
{
    SplitLayout L;
    int rc = split_prepare(s, true, workspace, ws_bytes, &L);
    if (rc != SSD_OK) return rc;
    char *w = static_cast<char *>(workspace);
    auto at = [&](size_t off) { return reinterpret_cast<float *>(w + off); };
    float *qb = at(L.qb), *kb = at(L.kb), *vb = at(L.vb), *h0b = at(L.h0b), *dyb = at(L.dyb);
    float *dqb = at(L.dqb), *dkb = at(L.dkbuf), *dvb = at(L.dvbuf), *dlab = at(L.dlab), *dh0b = at(L.dh0b);
    const int64_t nqr = s.B * s.G * s.T, nvr = s.B * s.H * s.T, BH = s.B * s.H;
    for (int J = 0; J < L.nJ && rc == SSD_OK; ++J) {
        const int64_t j0 = L.j0[J], dvJ = L.dvb[J];
        rc = copy_block(tm, st, vb, 0, dvJ, v + j0, 0, s.dv, 1, nvr, dvJ, false);
        if (rc == SSD_OK) rc = copy_block(tm, st, dyb, 0, dvJ, dy + j0, 0, s.dv, 1, nvr, dvJ, false);
        for (int I = 0; I < L.nI && rc == SSD_OK; ++I) {
            const int64_t i0 = L.i0[I], dkI = L.dkb[I];
            rc = copy_block(tm, st, qb, 0, dkI, q + i0, 0, s.dk, 1, nqr, dkI, false);
            if (rc == SSD_OK) rc = copy_block(tm, st, kb, 0, dkI, k + i0, 0, s.dk, 1, nqr, dkI, false);
            if (rc == SSD_OK)
                rc = copy_block(tm, st, h0b, dkI * dvJ, dvJ, h0 + i0 * s.dv + j0, s.dk * s.dv, s.dv, BH, dkI, dvJ,
                                false);
            const ssd_shape t = sub_shape(&s, L, I, J);
            if (rc == SSD_OK)
                rc = bwd_impl(&t, qb, kb, vb, log_alpha, h0b, dyb, dqb, dkb, dvb, dlab, dh0b, w + L.sub, L.sub_bytes,
                              st, false, tm);
            if (rc == SSD_OK) rc = copy_block(tm, st, dq + i0, 0, s.dk, dqb, 0, dkI, 1, nqr, dkI, J > 0);
            if (rc == SSD_OK) rc = copy_block(tm, st, dk + i0, 0, s.dk, dkb, 0, dkI, 1, nqr, dkI, J > 0);
            if (rc == SSD_OK) rc = copy_block(tm, st, dv + j0, 0, s.dv, dvb, 0, dvJ, 1, nvr, dvJ, I > 0);
            if (rc == SSD_OK) rc = copy_block(tm, st, dla, 0, 1, dlab, 0, 1, 1, nvr, 1, I > 0 || J > 0);
            if (rc == SSD_OK)
                rc = copy_block(tm, st, dh0 + i0 * s.dv + j0, s.dk * s.dv, s.dv, dh0b, dkI * dvJ, dvJ, BH, dkI, dvJ,
                                false);
        }
    }
    return rc;
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
    const size_t need = workspace_bytes(shape, false, device_cus());
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
