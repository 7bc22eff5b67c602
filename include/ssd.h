/*
 * ssd.h -- C ABI of the MI355X (gfx950) chunked scalar-decay SSD scan.
 *
 * The operation.  For every batch b and head h, with g = h / (H/G) the group
 * whose q and k the head reads (heads of a group are contiguous):
 *
 *     S_{-1} = h0[b,h]                                       (dk x dv)
 *     S_t    = exp(log_alpha[b,h,t]) * S_{t-1} + k[b,g,t] v[b,h,t]^T
 *     y[b,h,t] = S_t^T q[b,g,t]
 *
 * The tensor set and layouts are those fixed by the byte counts of the
 * benchmark pages kernel_ssd_cpu.json / kernel_ssd_gpu.json (results records
 * of impl "chunked": xla_arg_mb = q + k + v + log_alpha + h0 and xla_out_mb = y
 * in float32 for mode fwd; the five input gradients for mode fwd_bwd, see
 * rel_err_grads).  No final state is returned, and the gradient path keeps no
 * residual between forward and backward (residual_mb 0.0 in every chunked
 * fwd_bwd record): ssd_bwd recomputes what it needs from its inputs.
 *
 * Layouts (all float32, dense, row-major, no strides):
 *     q, k           [B, G, T, dk]
 *     v, y, dy       [B, H, T, dv]
 *     log_alpha      [B, H, T]
 *     h0, dh0        [B, H, dk, dv]
 *     dq, dk         [B, G, T, dk]   (summed over the heads of each group)
 *     dv             [B, H, T, dv]
 *     dlog_alpha     [B, H, T]
 *
 * Method.  The sequence is cut into chunks of SSD_CHUNK = 64 steps (one
 * step per lane of a 64-wide wavefront).  Per chunk: the within-chunk
 * cumulative log-decay, the decay-masked Q K^T V product on fp32 MFMA, the
 * chunk's decayed K^T V state contribution, a sequential pass over chunks
 * that carries the state from h0, and the inter-chunk output term
 * diag(e^b) Q S.  The backward mirrors these steps.  All products and sums
 * are fp32 (no reduced-precision products); results are deterministic run
 * to run (no floating-point atomics, fixed reduction orders).
 *
 * Memory and ownership.  Every tensor pointer and the workspace pointer are
 * DEVICE pointers on the current HIP device, allocated and owned by the
 * caller; the library never allocates, frees or synchronizes.  Each must be
 * 16-byte aligned.  Outputs are overwritten, never accumulated into, and
 * must not alias inputs, each other or the workspace.  Inputs are not
 * modified.
 *
 * Asynchrony.  Work is enqueued on `stream` (a hipStream_t; NULL is the
 * null stream) and the call returns after enqueueing.  The workspace and
 * the outputs must stay allocated until that work has completed.
 *
 * Errors.  Arguments are validated on the host before anything is enqueued;
 * on any validation failure the call returns a non-zero status, enqueues
 * nothing and leaves every output untouched.  A failed kernel launch returns
 * SSD_ERR_DEVICE (work enqueued before it may have run).  Faults during
 * execution surface at the caller's next synchronization.
 *
 * Supported shapes.  B >= 0, T >= 0, G >= 1, H >= 1, H % G == 0,
 * 1 <= dk <= 128, 1 <= dv <= 128; B*H*T*max(dk,dv) < 2^40.  Other dk/dv
 * return SSD_ERR_UNSUPPORTED.  log_alpha must be finite.
 *
 * Thread safety.  Calls are reentrant; concurrent calls on different streams
 * need separate workspaces.  The optional kernel-timing facility below is
 * process-global and not thread-safe.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_CHUNK 64

typedef struct ssd_shape {
    int64_t B, G, H, T, dk, dv;
} ssd_shape;

enum ssd_status {
    SSD_OK = 0,
    SSD_ERR_NULL = 1,        /* a required pointer is NULL                       */
    SSD_ERR_SHAPE = 2,       /* negative size, G < 1, H % G != 0, size overflow   */
    SSD_ERR_UNSUPPORTED = 3, /* valid shape outside the supported dk/dv range     */
    SSD_ERR_WORKSPACE = 4,   /* workspace smaller than the size query's answer    */
    SSD_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned                  */
    SSD_ERR_DEVICE = 6       /* a HIP launch or runtime call failed               */
};

/* Bytes of device workspace ssd_fwd / ssd_bwd need for `shape` (0 when the
 * shape is empty).  Returns (size_t)-1 if the shape is invalid or
 * unsupported.  The workspace needs no initialization and holds no state
 * between calls. */
size_t ssd_fwd_workspace_size(const ssd_shape *shape);
size_t ssd_bwd_workspace_size(const ssd_shape *shape);

/* Forward: y = scan(q, k, v, log_alpha, h0).
 * After the call completes, the workspace holds (for inspection by tests;
 * callers treat it as opaque) the regions reported by ssd_workspace_layout. */
int ssd_fwd(const ssd_shape *shape,
            const float *q, const float *k, const float *v,
            const float *log_alpha, const float *h0,
            float *y,
            void *workspace, size_t workspace_bytes, void *stream);

/* Backward of L = sum(dy * y): writes dq, dk, dv, dlog_alpha, dh0.
 * Stateless: recomputes the forward quantities it needs. */
int ssd_bwd(const ssd_shape *shape,
            const float *q, const float *k, const float *v,
            const float *log_alpha, const float *h0, const float *dy,
            float *dq, float *dk, float *dv, float *dlog_alpha, float *dh0,
            void *workspace, size_t workspace_bytes, void *stream);

/* Byte offsets of the workspace regions, in this order:
 *   [0] bcum   float [B*H][NC*64]  within-chunk inclusive cumsum of log_alpha
 *                                  (positions past T hold the last valid value)
 *   [1] bl     float [B*H][NCp]    chunk totals (NCp = NC rounded up to 64)
 *   [2] states float [B*H][NC][E]  after ssd_fwd/ssd_bwd: the state entering
 *                                  each chunk, row-major dk x dv; E = dk*dv
 *                                  rounded up to a multiple of 64
 *   [3] dstates float [B*H][NC][E] (backward only) after ssd_bwd: the
 *                                  gradient of the state leaving each chunk
 *   [4] total bytes.  When B*G*ceil(T/64) is below the GPU's 256 compute
 *       units the backward layout also holds, between the end of dstates and
 *       the total, the per-block-split partial sums of dq and dk that the
 *       gradient kernel writes and a final kernel adds up (no caller use).
 * `backward` selects the backward layout.  Returns SSD_OK or an error. */
int ssd_workspace_layout(const ssd_shape *shape, int backward, size_t offsets[5]);

/* Static description of a status code (never NULL). */
const char *ssd_strerror(int status);

/* Chunk length used by the kernels (SSD_CHUNK). */
int ssd_chunk_size(void);

/* Backward that reuses the forward's residuals: the same outputs as ssd_bwd,
 * but the workspace must already hold what ssd_fwd wrote for the SAME inputs
 * (q, k, v, log_alpha, h0 and shape) into a workspace of at least
 * ssd_bwd_workspace_size(shape) bytes: the forward's regions (per-chunk
 * cumulative log-decay, chunk totals and the state entering every chunk)
 * sit at the same offsets in the forward and backward layouts.  Only the
 * reverse state pass and the gradient kernel run, which skips recomputing
 * the forward states.  This is the residual-keeping side of the trade-off
 * that the GPU benchmark page records in its residual_mb field (0 for the
 * stateless chunked backward, a few to a hundred MiB for its fused
 * variant); ssd_bwd stays the stateless path.  The library cannot check the
 * precondition: with a
 * workspace that does not hold the forward's results for these inputs the
 * outputs are wrong (but every access stays inside the workspace and the
 * tensors).  Arguments, layouts, ownership, asynchrony and return codes are
 * those of ssd_bwd; the forward work must be enqueued on the same stream
 * before this call, or be complete. */
int ssd_bwd_from_fwd(const ssd_shape *shape,
                     const float *q, const float *k, const float *v,
                     const float *log_alpha, const float *h0, const float *dy,
                     float *dq, float *dk, float *dv, float *dlog_alpha, float *dh0,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Optional per-kernel timing with HIP events, for benchmarks.
 * ssd_kernel_timing_enable(mask) times the launches of the kernels whose bit
 * (1 << kid) is set in `mask` (-1: all kernels; 0: off, the default): their
 * start and stop events are bound to the kernel's own dispatch on the launch
 * stream (hipExtLaunchKernel), so they cover the kernel alone.  A timed
 * dispatch still costs a few microseconds of stream time, so a benchmark
 * that also times whole calls should time only the kernels it needs.
 * ssd_kernel_timing_read synchronizes on the recorded events and returns,
 * for kernel id `kid` (0 <= kid < ssd_kernel_count()), the summed duration
 * in milliseconds and the number of timed launches since the last reset.
 * Process-global, not thread-safe. */
int ssd_kernel_timing_enable(int mask);
int ssd_kernel_timing_reset(void);
int ssd_kernel_timing_read(int kid, double *total_ms, int64_t *count);
int ssd_kernel_count(void);
const char *ssd_kernel_name(int kid);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
