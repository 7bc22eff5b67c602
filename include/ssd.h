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
 * Sources.  The benchmark pages kernel_ssd_cpu.json and kernel_ssd_gpu.json
 * print no formula; they fix the tensor set and the layouts through their
 * byte counts.  In every results record of impl "chunked" and mode "fwd",
 * xla_arg_mb equals q + k + v + log_alpha + h0 and xla_out_mb equals y, in
 * float32 and the layouts below.  In mode "fwd_bwd" the outputs are the five
 * input gradients named by the keys of rel_err_grads, and residual_mb is 0.0
 * (the chunked backward keeps nothing from its forward).  The config block
 * of each page lists the shapes as (batch, groups, heads, dk, dv).
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
 * caller; the library never allocates device memory, frees or synchronizes
 * (the timer calls below aside).  Each pointer must be 16-byte aligned.
 * Outputs are overwritten, never accumulated into, and must not alias
 * inputs, each other or the workspace.  Inputs are not modified.
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
 * 1 <= dk <= 256, 1 <= dv <= 256; B*H*T*max(dk,dv) < 2^40.  Other dk/dv
 * return SSD_ERR_UNSUPPORTED.  log_alpha must be finite.  The kernels take
 * dk, dv up to 128 directly; a larger dk or dv is cut into column blocks of
 * 128 and the rest, each block pair runs as its own problem, and the
 * outputs are added up in a fixed order (y is linear in the dk blocks of q
 * and k and separable in the dv blocks of v; the gradients follow).
 *
 * Thread safety.  The compute calls keep no mutable state between calls and
 * are reentrant; concurrent calls on different streams need separate
 * workspaces.  A timer (ssd_timer_create) belongs to one caller at a time.
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

/* Status codes.  Every call validates its arguments first and returns one of
 * these.  SSD_ERR_UNSUPPORTED is this library's form of the pages' declined
 * shapes: the results records of impls "scan" and "pallas" at config
 * g2h4_dk48_dv40 (kernel_ssd_cpu.json and kernel_ssd_gpu.json) carry
 * "skipped": "unsupported shape" instead of a result, i.e. a valid shape an
 * implementation does not compute is refused, never computed wrongly. */
enum ssd_status {
    SSD_OK = 0,
    SSD_ERR_NULL = 1,        /* a required pointer is NULL                       */
    SSD_ERR_SHAPE = 2,       /* negative size, G < 1, H % G != 0, size overflow   */
    SSD_ERR_UNSUPPORTED = 3, /* valid shape outside the supported dk/dv range,
                                 or an SSD_FWD_CHUNK the forward cannot take */
    SSD_ERR_WORKSPACE = 4,   /* workspace smaller than the size query's answer    */
    SSD_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned                  */
    SSD_ERR_DEVICE = 6       /* a HIP launch or runtime call failed               */
};

/* Bytes of device workspace ssd_fwd / ssd_bwd need for `shape` on the
 * current device (0 when the shape is empty; the size depends on the
 * device's compute-unit count, 256 assumed when no device is visible).
 * Returns (size_t)-1 if the shape is invalid or unsupported.  The workspace
 * needs no initialization and holds no state between calls.  The pages
 * report the chunked path's temporary device memory as xla_temp_mb and its
 * peak as peak_mb (kernel_ssd_gpu.json, results records of kind "peak");
 * this query is where this library's equivalent is stated up front. */
size_t ssd_fwd_workspace_size(const ssd_shape *shape);
size_t ssd_bwd_workspace_size(const ssd_shape *shape);

/* Forward: y = scan(q, k, v, log_alpha, h0), the operation of the "chunked"
 * "fwd" records of kernel_ssd_cpu.json / kernel_ssd_gpu.json (arguments per
 * xla_arg_mb, the single output per xla_out_mb).  After the call completes
 * the workspace holds (for inspection by tests; callers treat it as opaque)
 * the regions reported by ssd_workspace_layout. */
int ssd_fwd(const ssd_shape *shape,
            const float *q, const float *k, const float *v,
            const float *log_alpha, const float *h0,
            float *y,
            void *workspace, size_t workspace_bytes, void *stream);

/* Backward of L = sum(dy * y): writes dq, dk, dv, dlog_alpha, dh0, the five
 * gradients of the "chunked" "fwd_bwd" records (keys of rel_err_grads).
 * Stateless, as those records' residual_mb 0.0 says: it recomputes the
 * forward quantities it needs from its inputs. */
int ssd_bwd(const ssd_shape *shape,
            const float *q, const float *k, const float *v,
            const float *log_alpha, const float *h0, const float *dy,
            float *dq, float *dk, float *dv, float *dlog_alpha, float *dh0,
            void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * forward as ssd_fwd, with the same arguments less the workspace, which is
 * a file-scope device array of SSD_NOALLOC_WORKSPACE_BYTES (96 MiB) inside
 * the library: each GPU the library runs on holds its own copy until the
 * process ends.  The call allocates nothing (no hipMalloc, no library
 * allocation); the caller still passes the inputs and y.  Shapes whose
 * ssd_fwd_workspace_size exceeds the array return SSD_ERR_WORKSPACE before
 * anything is enqueued (every workload of the pages at T <= 2048 fits; the
 * largest, g2h8_d128 at T = 2048, needs 64.5 MiB).  Every call on one GPU
 * shares that GPU's array, so calls that overlap in time on one GPU (on
 * different streams or threads) race and give wrong results: serialize
 * them.  The array keeps the last call's contents; nothing in it needs to
 * start at zero.  Status codes as ssd_fwd, plus SSD_ERR_DEVICE if the
 * array's device address cannot be obtained. */
#define SSD_NOALLOC_WORKSPACE_BYTES (96u << 20)
int ssd_fwd_noalloc(const ssd_shape *shape,
                    const float *q, const float *k, const float *v,
                    const float *log_alpha, const float *h0,
                    float *y, void *stream);

/* Number of workspace regions reported by ssd_workspace_layout. */
#define SSD_WS_REGIONS 4

/* Byte offsets of the workspace regions, in this order:
 *   [0] decay   float [B*H][NC][2][64], then float [B*H][NC] at the next
 *               256-byte boundary: per position of chunk c, e^{b_L - b_t}
 *               and e^{b_t}, and per chunk e^{b_L}, where b_t is the
 *               within-chunk inclusive cumulative sum of log_alpha and b_L
 *               its value at the chunk's last position; NC = ceil(T/64)
 *   [1] states  float [B*H][NC][E]  the state entering each chunk, row-major
 *                                   dk x dv; E = dk*dv rounded up to a multiple
 *                                   of 64.  After ssd_bwd: every chunk.  After
 *                                   ssd_fwd: chunks 0, s, 2s, ... with s =
 *                                   ssd_fwd_state_stride(shape)
 *   [2] dstates float [B*H][NC][E]  (backward only; empty otherwise) after
 *                                   ssd_bwd: the gradient of the state
 *                                   leaving each chunk
 *   [3] aux     (no caller use; empty unless needed) in the backward, when
 *               B*G*ceil(T/64) is below the device's compute-unit count,
 *               the per-block-split partial sums of dq and dk that the
 *               gradient kernel writes and a final kernel adds up; then, when
 *               the state scan's grid would leave CUs idle, the end states of
 *               the chunk segments that its blocks scan in parallel and the
 *               per-chunk decay products within each segment
 *   [4] total bytes.
 * `backward` selects the backward layout.  Returns SSD_OK or an error;
 * SSD_ERR_UNSUPPORTED for shapes with dk or dv above 128, whose workspace
 * holds the column-block sub-problems instead.
 * Test support: the states are the quantity the chunked method passes
 * between chunks, checked against the oracle's state at chunk boundaries. */
int ssd_workspace_layout(const ssd_shape *shape, int backward, size_t offsets[SSD_WS_REGIONS + 1]);

/* Test support: 1 if ssd_fwd leaves the state of every chunk in the
 * workspace, 2 if only that of every even chunk (-1 for an invalid shape,
 * one with dk or dv above 128, or an SSD_FWD_CHUNK that ssd_fwd would
 * refuse).  With 2 the forward runs on chunk pairs: the odd chunk of a pair
 * takes its inter-chunk term from the even chunk's state S, as e^{b_L} S
 * plus the decayed sum of the even chunk's k v^T, which is the state-pass
 * recurrence itself; that halves the states the forward writes and reads.
 * In effect the forward's chunk is then 128 steps, its intra-chunk product
 * taken as four 64 x 64 blocks.  The pages fix no chunk length (the chunked
 * method's result does not depend on it beyond rounding).  The library
 * chooses per shape and device (128-column states and enough pairs to fill
 * every CU twice) unless the environment variable SSD_FWD_CHUNK, read at
 * each call of ssd_fwd, ssd_fwd_timed, ssd_fwd_noalloc, ssd_bwd_from_fwd
 * and this function (with getenv: do not change it while another thread
 * is inside one of these calls), fixes it:
 *     unset or empty   the library's choice
 *     "64"             every chunk's state (stride 1)
 *     "128"            chunk pairs (stride 2); a forward whose dv (or, above
 *                      128, each 128-column block of dv) is 32 or less
 *                      returns SSD_ERR_UNSUPPORTED
 *     anything else    ssd_fwd, ssd_fwd_noalloc and ssd_bwd_from_fwd return
 *                      SSD_ERR_UNSUPPORTED
 * It exists for the chunk-length invariance tests.  ssd_bwd_from_fwd must
 * see the same setting as the ssd_fwd whose workspace it reuses; ssd_bwd
 * ignores it (its chunk is 64). */
int ssd_fwd_state_stride(const ssd_shape *shape);

/* Static description of a status code (never NULL). */
const char *ssd_strerror(int status);

/* Chunk length used by the kernels (SSD_CHUNK).  The SSD pages state no
 * chunk length; results do not depend on it beyond rounding. */
int ssd_chunk_size(void);

/* Backward that reuses the forward's residuals: the same outputs as ssd_bwd,
 * but the workspace must already hold what ssd_fwd wrote for the SAME inputs
 * (q, k, v, log_alpha, h0 and shape) into a workspace of at least
 * ssd_bwd_workspace_size(shape) bytes: the forward's regions (the decay
 * weights and the chunk states) sit at the same offsets in the forward and
 * backward layouts.  When ssd_fwd left the state of every chunk
 * (ssd_fwd_state_stride 1), only the reverse state pass and the gradient
 * kernel run, which skips recomputing the forward states; when it left
 * every even chunk's (stride 2), the forward state pass runs again beside
 * the reverse one and stores only the odd chunks' states, and the decay
 * weights are reused.  This is the residual-keeping side
 * of the trade-off that kernel_ssd_gpu.json records in residual_mb (0.0 for
 * the stateless chunked backward; 8 to 128 MiB for its pallas variant in
 * the g2h8_d128 fwd_bwd records); ssd_bwd stays the stateless path.  The
 * library cannot check the precondition: with a workspace that does not
 * hold the forward's results for these inputs the outputs are wrong (but
 * every access stays inside the workspace and the tensors).  Arguments,
 * layouts, ownership, asynchrony and return codes are those of ssd_bwd;
 * the forward work must be enqueued on the same stream before this call,
 * or be complete.  For dk or dv above 128 it recomputes, exactly as ssd_bwd
 * (the column-block sub-problems keep no residual between calls). */
int ssd_bwd_from_fwd(const ssd_shape *shape,
                     const float *q, const float *k, const float *v,
                     const float *log_alpha, const float *h0, const float *dy,
                     float *dq, float *dk, float *dv, float *dlog_alpha, float *dh0,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Per-kernel timing with HIP events, for benchmarks: the pages time whole
 * calls (median_ms, q1_ms, q3_ms of every results record); these calls
 * time the kernels inside a call.  A timer is a caller-owned object; the
 * plain compute calls never read it.
 *
 * ssd_timer_create(mask) returns a timer (NULL if out of host memory) that
 * times the launches of the kernels whose bit (1 << kid) is set in `mask`
 * (-1: all kernels).  ssd_fwd_timed / ssd_bwd_timed are ssd_fwd / ssd_bwd
 * with the timer: the start and stop events of each timed kernel are bound
 * to the kernel's own dispatch on the launch stream (hipExtLaunchKernel),
 * so they cover the kernel alone; a timed dispatch still costs a few
 * microseconds of stream time.  ssd_timer_read synchronizes on the recorded
 * events and returns, for kernel id `kid` (0 <= kid < ssd_kernel_count()),
 * the summed duration in milliseconds and the number of timed launches
 * since the last reset.  ssd_timer_destroy waits for the timer's events and
 * frees it.  One timer must not be used by two threads at once. */
typedef struct ssd_timer ssd_timer;
ssd_timer *ssd_timer_create(int mask);
int ssd_timer_destroy(ssd_timer *timer);
int ssd_timer_reset(ssd_timer *timer);
int ssd_timer_read(ssd_timer *timer, int kid, double *total_ms, int64_t *count);
int ssd_fwd_timed(ssd_timer *timer, const ssd_shape *shape,
                  const float *q, const float *k, const float *v,
                  const float *log_alpha, const float *h0,
                  float *y,
                  void *workspace, size_t workspace_bytes, void *stream);
int ssd_bwd_timed(ssd_timer *timer, const ssd_shape *shape,
                  const float *q, const float *k, const float *v,
                  const float *log_alpha, const float *h0, const float *dy,
                  float *dq, float *dk, float *dv, float *dlog_alpha, float *dh0,
                  void *workspace, size_t workspace_bytes, void *stream);
int ssd_kernel_count(void);
const char *ssd_kernel_name(int kid);

/* ---------------------------------------------------------------------------
 * Selective (Mamba-style) scan, the second workload of the benchmark pages
 * (kernel_mamba_cpu.json, results: impls scan, assoc and chunked at batch 4,
 * state 16, dim 256/512/1024, seq 512/2048/8192, modes fwd and fwd_bwd).
 *
 * That page prints no formula.  Its byte counts fix the tensor set: every
 * fwd record's xla_arg_mb is x[B,L,D] + delta[B,L,D] + A[D,N] + B[B,L,N] +
 * C[B,L,N] + Dskip[D] in float32 (4.27 MiB at B=4, L=512, D=256, N=16) and
 * its xla_out_mb is y[B,L,D] (2.0 MiB).  The library computes the plain
 * reading of that argument set, for every batch b, channel d and state n,
 * with h_{-1} = 0:
 *     h_t[d,n] = exp(delta[b,t,d] A[d,n]) h_{t-1}[d,n] + delta[b,t,d] B[b,t,n] x[b,t,d]
 *     y[b,t,d] = sum_n C[b,t,n] h_t[d,n] + Dskip[d] x[b,t,d]
 * (delta is used as given: no softplus, no gating input).  All arithmetic
 * is fp32; results are deterministic run to run.
 *
 * Shapes: B >= 0, L >= 0, D >= 1, 1 <= N <= MAMBA_MAX_STATE (larger N:
 * SSD_ERR_UNSUPPORTED); B*L*max(D,N) < 2^40.  Layouts are dense row-major
 * as written above; pointers are device pointers on the current device,
 * 4-byte aligned, owned by the caller; outputs are overwritten and must not
 * alias anything else.  Arguments are checked on the host before anything
 * is enqueued (status codes as for ssd_fwd); work is enqueued on `stream`.
 * The workspace (mamba_fwd_workspace_size bytes, 16-byte aligned; none when
 * the size is 0) holds each sequence segment's end state and summed delta;
 * it need not be initialised and is not read after the call. */
#define MAMBA_MAX_STATE 16

typedef struct mamba_shape {
    int64_t B, L, D, N;
} mamba_shape;

/* Workspace bytes mamba_fwd needs on the current device (0 for an invalid
 * shape, and when the sequence runs as one segment). */
size_t mamba_fwd_workspace_size(const mamba_shape *shape);

/* y = the selective scan of (x, delta, A, B, C, Dskip); see above. */
int mamba_fwd(const mamba_shape *shape,
              const float *x, const float *delta, const float *A,
              const float *B, const float *C, const float *Dskip,
              float *y,
              void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes mamba_bwd needs (0 for an invalid shape or one it
 * refuses, and when B or L is 0). */
size_t mamba_bwd_workspace_size(const mamba_shape *shape);

/* The gradients of L = sum dy . y with respect to every argument, the six
 * outputs of the page's fwd_bwd records: dx, ddelta [B,L,D], dA [D,N],
 * dB, dC [B,L,N], dDskip [D], all overwritten (dA and dDskip are zero when
 * B or L is 0; they are the sums over batch and steps, taken in a fixed
 * order).  Stateless: the forward's states are recomputed.  L above
 * 65535 * 32 returns SSD_ERR_UNSUPPORTED.  Arguments, checks, ownership and
 * asynchrony as for mamba_fwd; the workspace is mamba_bwd_workspace_size
 * bytes. */
int mamba_bwd(const mamba_shape *shape,
              const float *x, const float *delta, const float *A,
              const float *B, const float *C, const float *Dskip, const float *dy,
              float *dx, float *ddelta, float *dA, float *dB, float *dC, float *dDskip,
              void *workspace, size_t workspace_bytes, void *stream);

/* y and the six gradients in one call: the value and the gradients that the
 * page's fwd_bwd records compute together.  y is mamba_fwd's output (to
 * rounding: its segments are the backward's), the gradients are mamba_bwd's
 * bit for bit.  y is formed from the states the backward recomputes anyway,
 * so no forward pass runs.  Arguments, checks and the workspace as for mamba_bwd,
 * plus y [B,L,D] (device, 4-byte aligned, overwritten; NULL only when B or
 * L is 0). */
int mamba_fwd_bwd(const mamba_shape *shape,
                  const float *x, const float *delta, const float *A,
                  const float *B, const float *C, const float *Dskip, const float *dy,
                  float *y, float *dx, float *ddelta, float *dA, float *dB, float *dC, float *dDskip,
                  void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
