// HIP kernels (gfx950) and the launch sequence behind the SSD scan C ABI.
//
// Chunked form of the scalar-decay scan.  With chunk length C = 64, within
// chunk c let b_t be the inclusive cumulative sum of log_alpha over the
// chunk's positions up to t, b_L its value at the chunk's last position, and
// D[i][j] = exp(b_i - b_j) for j <= i (0 otherwise).  Then
//
//   Y_c      = (Q K^T o D) V + diag(e^b) Q S_in(c)               (output)
//   X_c      = K^T diag(e^{b_L - b}) V                          (chunk state)
//   S_in(0)  = h0,  S_in(c+1) = e^{b_L(c)} S_in(c) + X_c         (state pass)
//
// which equals the per-step recurrence exactly up to rounding.  The backward
// mirrors it with dS_out(c), the gradient of the state leaving chunk c:
//
//   Z_c           = Q^T diag(e^b) dY
//   dS_out(NC-1)  = 0,  dS_out(c-1) = e^{b_L(c)} dS_out(c) + Z_c,
//   dh0           = e^{b_L(0)} dS_out(0) + Z_0
//   dP = (dY V^T) o D
//   dQ = dP K + diag(e^b) dY S_in^T
//   dK = dP^T Q + diag(e^{b_L - b}) V dS_out^T
//   dV = (Q K^T o D)^T dY + diag(e^{b_L - b}) K dS_out
//   dlog_alpha_r = sum_{i >= r, j < r} M_ij                    (intra)
//                + sum_{i >= r} e^{b_i} q_i . (dY S_in^T)_i        (output via S_in)
//                + sum_{j < r} e^{b_L - b_j} k_j . (V dS_out^T)_j  (outgoing state)
//                + e^{b_L} <dS_out, S_in>_F
//   with M = (Q K^T) o D o (dY V^T).
//
// The last formula differentiates each decay factor directly: D_ij depends
// on log_alpha_r exactly when j < r <= i, e^{b_i} when r <= i, e^{b_L - b_j}
// when r > j, and e^{b_L} always.  It equals the suffix sum of
// q_t.dq_t - k_t.dk_t plus the boundary term, but it has no cancelling O(1)
// terms (the diagonal of M and the last position's state term cancel
// exactly in that form), so its error scales with dlog_alpha itself.
//
// All contractions run on v_mfma_f32_32x32x2f32 (fp32 in, fp32 accumulate).
// For that instruction, lane l supplies A[l%32][l/32] and B[l/32][l%32] of a
// 32x2 by 2x32 product, and accumulator register r of lane l holds row
// 8*(r/4) + 4*(l/32) + r%4, column l%32 of the 32x32 result.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <stdint.h>
#include <tuple>
#include <vector>

#include "ssd.h"
#include "ssd_internal.h"

namespace ssd {

constexpr int CH = kChunk;   // 64
constexpr int NTH = 256;     // 4 waves per block

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x4f32: lane l supplies A[l%16][l/16] and B[l/16][l%16];
// accumulator register r of lane l holds row 4*(l/16) + r, column l%16.
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Row (within the 32x32 tile) of accumulator register r in lane `lane`.
__device__ __forceinline__ int acc_row(int r, int lane)
{
    return ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3);
}

__device__ __forceinline__ f32x16 zero16()
{
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// Cross-lane sums and scans with DPP (VALU data-parallel primitives, no LDS
// traffic).  dpp_add<C, R>(x) adds the value of the lane that DPP control C
// selects, or 0 where it selects none or the row (16 lanes) is not in mask R.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_add(float x)
{
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xf, true));
}
constexpr int kRowShr = 0x110, kRowRor = 0x120, kRowBcast15 = 0x142, kRowBcast31 = 0x143, kWaveShr1 = 0x138;

// Sum of each 32-lane half: the result is in lanes 31 (lanes 0-31) and 63
// (lanes 32-63).
__device__ __forceinline__ float sum32_hi(float x)
{
    x = dpp_add<kRowRor + 8>(x);
    x = dpp_add<kRowRor + 4>(x);
    x = dpp_add<kRowRor + 2>(x);
    x = dpp_add<kRowRor + 1>(x);          // every lane: the sum of its row
    return dpp_add<kRowBcast15, 0xa>(x);  // rows 1 and 3 add rows 0 and 2
}

// Sum of all 64 lanes, in lane 63.
__device__ __forceinline__ float sum64_hi(float x)
{
    x = sum32_hi(x);
    return dpp_add<kRowBcast31, 0xc>(x);  // rows 2 and 3 add lane 31
}

// Inclusive prefix sum over the 64 lanes (lane l: x_0 + ... + x_l).
__device__ __forceinline__ float scan64(float x)
{
    x = dpp_add<kRowShr + 1>(x);
    x = dpp_add<kRowShr + 2>(x);
    x = dpp_add<kRowShr + 4>(x);
    x = dpp_add<kRowShr + 8>(x);          // prefix within each row
    x = dpp_add<kRowBcast15, 0xa>(x);
    return dpp_add<kRowBcast31, 0xc>(x);
}

// The value of lane l - 1 (0 in lane 0).
__device__ __forceinline__ float shift_up1(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kWaveShr1, 0xf, 0xf, true));
}

__device__ __forceinline__ float readlane_f(float x, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// ---------------------------------------------------------------------------
// K1: within-chunk inclusive cumulative log-decay.  One wave per (b,h,chunk),
// lane t holds position c*64 + t.  Positions past T read log_alpha = 0, so
// they repeat the last valid cumulative value and the chunk total (lane 63)
// is the sum over the valid positions.
__global__ __launch_bounds__(NTH) void k_chunk_cumsum(const float *__restrict__ la, float *__restrict__ bcum,
                                                      float *__restrict__ bl, int64_t T, int64_t NC,
                                                      int64_t NCp, int64_t nwaves)
{
    const int64_t wv = (int64_t)blockIdx.x * (NTH / 64) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (wv >= nwaves) return;   // whole waves only
    const int64_t bh = wv / NC, c = wv - bh * NC;
    const int64_t t = c * CH + lane;
    float x = (t < T) ? la[bh * T + t] : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    bcum[bh * NC * CH + t] = x;
    if (lane == 63) bl[bh * NCp + c] = x;
}

// ---------------------------------------------------------------------------
// Helpers for the 8-wave kernels.

constexpr int NTW = 512;   // 8 waves per block

template <bool B>
struct BoolC {
    static constexpr bool value = B;
};

// Workgroup barrier across which the compiler may move no memory access.
// __syncthreads() alone is a fence pair around s_barrier, and this compiler
// has been seen to sink LDS reads below it into a region that other waves
// overwrite after the barrier; the empty asm statements with a memory
// clobber pin every access on its side.
__device__ __forceinline__ void block_sync()
{
    asm volatile("" ::: "memory");
    __syncthreads();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ float4 zero4() { return make_float4(0.f, 0.f, 0.f, 0.f); }

// Global memory goes through buffer resources: a resource covers `bytes`
// bytes from a base address, and a lane whose byte offset is at or past the
// end (kOOB is always past it) reads 0 and has its store dropped by the
// hardware.  Tile edges are masked that way, without branches, so the loads
// of a tile issue back to back and the compiler's count of memory operations
// in flight stays exact.  Every resource covers one tile, slab or row, far
// below 2 GiB.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ float4 gload4(rsrc_t r, uint32_t off)
{
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_float4(__int_as_float(x[0]), __int_as_float(x[1]), __int_as_float(x[2]), __int_as_float(x[3]));
}

__device__ __forceinline__ float gload1(rsrc_t r, uint32_t off)
{
    return __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

__device__ __forceinline__ void gstore1(rsrc_t r, uint32_t off, float x)
{
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(x), r, off, 0, 0);
}
// Store that is not read again by this kernel: non-temporal, so it does not
// displace reusable lines from L2.
__device__ __forceinline__ void gstore1_nt(rsrc_t r, uint32_t off, float x)
{
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(x), r, off, 0, 2);
}
// The same for N = 2 or 4 consecutive floats.  A non-temporal store that
// covers only part of a cache line goes out as a partial line, so stores of
// one line are best made by one instruction.
template <int N>
__device__ __forceinline__ void gstoreN_nt(rsrc_t r, uint32_t off, const float *x)
{
    if constexpr (N == 1) {
        gstore1_nt(r, off, x[0]);
    } else if constexpr (N == 2) {
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, make_float2(x[0], x[1])), r, off, 0, 2);
    } else {
        static_assert(N == 4, "1, 2 or 4 floats");
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, make_float4(x[0], x[1], x[2], x[3])), r, off,
                                               0, 2);
    }
}

// Elements c4 .. c4+3 of the row that starts at element `rowoff` of resource
// r; the row has `lim` elements (the rest read as 0), and nothing is read
// when `ok` is false.  vec: one 16-byte load (lim % 4 == 0, rows 16-byte
// aligned).
__device__ __forceinline__ float4 load4(rsrc_t r, uint32_t rowoff, int c4, int lim, bool ok, bool vec)
{
    if (vec) return gload4(r, (ok && c4 < lim) ? (rowoff + (uint32_t)c4) * 4u : kOOB);
    float e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = gload1(r, (ok && c4 + i < lim) ? (rowoff + (uint32_t)(c4 + i)) * 4u : kOOB);
    return make_float4(e[0], e[1], e[2], e[3]);
}

// Float4 number tid + u NT of a row-major tile with Q4 float4 per row, for
// NT a multiple of Q4 (0 <= tid < NT): its row and its first column.
// Unsigned, so the division is a shift; the rows of one thread step by a
// constant.
template <int Q4, int NT>
__device__ __forceinline__ int f4_row(int tid, int u)
{
    static_assert(NT % Q4 == 0, "a thread's float4 share their column");
    return (int)((unsigned)tid / Q4) + u * (NT / Q4);
}
template <int Q4>
__device__ __forceinline__ int f4_col(int tid)
{
    return (int)((unsigned)tid % Q4) * 4;
}

// Load a ROWS x DP tile into registers, PER float4 per thread, zero padded:
// row-major with row stride d and d valid columns, from resource r, which
// covers exactly the valid rows (rows past them read as 0).
template <int ROWS, int DP, int NT, int PER>
__device__ __forceinline__ void tile_to_regs(int tid, float4 (&buf)[PER], rsrc_t r, int d, bool vec)
{
    constexpr int Q4 = DP / 4;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int row = f4_row<Q4, NT>(tid, u), c4 = f4_col<Q4>(tid);
        buf[u] = load4(r, (uint32_t)(row * d), c4, d, (ROWS * Q4) % NT == 0 || row < ROWS, vec);
    }
}

// Store a register tile (see tile_to_regs) into LDS dst[ROWS][LD].
template <int ROWS, int DP, int NT, int PER, int LD>
__device__ __forceinline__ void regs_to_lds(int tid, const float4 (&buf)[PER], float *dst)
{
    constexpr int Q4 = DP / 4;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int r = f4_row<Q4, NT>(tid, u), c4 = f4_col<Q4>(tid);
        if ((ROWS * Q4) % NT == 0 || r < ROWS) {
            if (LD % 4 == 0) {
                *reinterpret_cast<float4 *>(dst + r * LD + c4) = buf[u];
            } else {
                float *pp = dst + r * LD + c4;
                pp[0] = buf[u].x;
                pp[1] = buf[u].y;
                pp[2] = buf[u].z;
                pp[3] = buf[u].w;
            }
        }
    }
}

// acc += A B^T over k in [k0, k1) (a multiple of 8 long): A and B are the
// 32-row blocks starting at A and B (row-major in LDS, row strides LDA and
// LDB).  Lane (kh, r) reads k0 + 4kh .. k0 + 4kh + 3 of its rows with one
// 16-byte load and feeds them to four MFMAs; MFMA s contracts over the k
// pair (k0 + s, k0 + 4 + s).
template <int LDA, int LDB>
__device__ __forceinline__ void mma_abt(f32x16 &acc, const float *A, const float *B, int k0, int k1, int lane)
{
    const int cl = lane & 31, kh = lane >> 5;
    const float *a = A + cl * LDA + 4 * kh;
    const float *b = B + cl * LDB + 4 * kh;
#pragma unroll 2
    for (int kk = k0; kk < k1; kk += 8) {
        const float4 x = *reinterpret_cast<const float4 *>(a + kk);
        const float4 y = *reinterpret_cast<const float4 *>(b + kk);
        acc = mfma32(x.x, y.x, acc);
        acc = mfma32(x.y, y.y, acc);
        acc = mfma32(x.z, y.z, acc);
        acc = mfma32(x.w, y.w, acc);
    }
}

// acc += A B^T for the 16-row blocks starting at A and B (row-major in LDS,
// row strides LDA and LDB) over k in [k0, k1) (a multiple of 16 long), on
// v_mfma_f32_16x16x4f32.  Lane (q, r) reads k0 + 4q .. k0 + 4q + 3 of its
// rows with one 16-byte load; MFMA s contracts over k0 + s + {0, 4, 8, 12}.
template <int LDA, int LDB>
__device__ __forceinline__ void mma16_abt(f32x4 &acc, const float *A, const float *B, int k0, int k1, int lane)
{
    const int l16 = lane & 15, lq = lane >> 4;
    const float *a = A + l16 * LDA + 4 * lq;
    const float *b = B + l16 * LDB + 4 * lq;
#pragma unroll 2
    for (int kk = k0; kk < k1; kk += 16) {
        const float4 x = *reinterpret_cast<const float4 *>(a + kk);
        const float4 y = *reinterpret_cast<const float4 *>(b + kk);
        acc = mfma16(x.x, y.x, acc);
        acc = mfma16(x.y, y.y, acc);
        acc = mfma16(x.z, y.z, acc);
        acc = mfma16(x.w, y.w, acc);
    }
}

// The C x C tiles of Q K^T, dY V^T, P and dP are handled as a 4 x 4 grid of
// 16x16 tiles, two per wave (tiles w and 15 - w of wave w, row-major), so
// every wave forms the same number of elements and no partial sums cross
// waves.  Tiles above the diagonal are zero.
__device__ __forceinline__ int cc_tile(int wave, int u) { return u == 0 ? wave : 15 - wave; }

// ---------------------------------------------------------------------------
// K3 + K4 fused: sequential scan over chunks with the state held in MFMA
// accumulators (v_mfma_f32_16x16x4f32: lane l supplies A[l%16][l/16] and
// B[l/16][l%16]; accumulator r of lane l is row 4*(l/16) + r, column l%16).
//
//   forward (dir 0):  S = h0;  for c = 0 .. NC-1:
//                       slab[c] = S;  S = e^{b_L(c)} S + K_c^T diag(e^{b_L - b}) V_c
//   reverse (dir 1):  S = 0;   for c = NC-1 .. 0:
//                       slab[c] = S;  S = e^{b_L(c)} S + Q_c^T diag(e^{b}) dY_c
//                     dh0 = S
//
// so the forward slabs hold S_in(c), the state entering chunk c, and the
// reverse slabs hold dS_out(c), the gradient of the state leaving chunk c.
// The chunk's own contribution is formed on the fly and never stored.
//
// One block owns a 32 x TJ tile of one head's dk x dv state and has two
// kinds of waves, one of each per SIMD:
//   * four compute waves hold the state (each a 16 x TJ/2 slice) and per
//     chunk read their operands from LDS, store the state and run the MFMAs;
//   * four loader waves keep the operand tiles of the next PD steps in flight
//     in registers and per step write the next step's tiles, their rows scaled
//     by the decay weights, into the other half of the double-buffered LDS
//     tiles.
// A step covers CPS consecutive chunks, so the per-step synchronisation is
// paid once per CPS chunks.  A loader wave's memory and exp work runs on its
// SIMD while the compute wave's MFMAs do, and no compute wave waits on a
// global load.  The number of steps is rounded up to a multiple of PD with
// no-op chunks (zero operands, decay 1, stores dropped), so no load or store
// is conditional and the compiler's count of loads in flight is exact.
// A compute wave owns NU = TJ/32 16x16 accumulator tiles whose columns
// interleave (tile u holds the wave's columns NU j + u), so one LDS read of
// NU consecutive floats gives a lane all its B operands.  Blocks of one
// (b, g) are placed on one XCD so that the group's q/k and each head's v/dy
// tiles are shared through that XCD's L2.
constexpr int TI = 32;
constexpr int NTS = 512;        // 4 compute + 4 loader waves

template <int DKP, int DVP, bool VEC, int TJ, int CPS, bool EXD>
__global__ __launch_bounds__(NTS) void k_state_scan(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ dy, const float *__restrict__ h0, const float *__restrict__ bcum,
    const float *__restrict__ bl, float *__restrict__ states, float *__restrict__ dstates,
    float *__restrict__ dh0, int G, int H, int64_t T, int dk, int dv, int64_t NC, int64_t NCp, int64_t Epad,
    int64_t per_dir, int dir0)
{
    static_assert(TJ <= DVP && DVP % TJ == 0 && (TJ == 32 || TJ == 64 || TJ == 128), "tile width");
    if constexpr (EXD) {   // dk == DKP, dv == DVP: index arithmetic on constants
        dk = DKP;
        dv = DVP;
        Epad = (int64_t)DKP * DVP;
    }
    constexpr int NTJ = DVP / TJ;
    constexpr int NTILE = (DKP / TI) * NTJ;
    constexpr int NU = TJ / 32;                       // accumulator tiles per compute wave
    constexpr int WC = TJ / 2;                        // columns per compute wave
    constexpr int LDA = TI + 16;                      // A reads: rows 16 banks apart
    // B reads of NU floats per lane: rows 16 (b32) or 32 (b64) banks apart;
    // b128 reads cover 256 contiguous bytes per 16 lanes
    constexpr int LDB = (NU == 1) ? TJ + 16 : (NU == 2) ? TJ + 32 : TJ + 4;
    constexpr int NLT = 256;                          // loader threads
    constexpr int A4 = CH * TI / 4, B4 = CH * TJ / 4;
    constexpr int APER = (A4 + NLT - 1) / NLT, BPER = (B4 + NLT - 1) / NLT;
    constexpr int PD = 2;                             // steps loaded ahead (3 and 4 measured slower)
    __shared__ __attribute__((aligned(16))) float As[2][CPS][CH * LDA];
    __shared__ __attribute__((aligned(16))) float Bs[2][CPS][CH * LDB];
    __shared__ float decs[2][CPS];                    // e^{b_L} of each staged chunk

    // XCD-aware order: consecutive logical blocks share blockIdx % 8.
    const int64_t nblk = gridDim.x;
    int64_t L = blockIdx.x;
    if ((nblk & 7) == 0) L = (int64_t)(blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
    const int64_t dl = L / per_dir;                   // direction index within this launch
    const int dir = dir0 + (int)dl;                   // 0: forward states, 1: reverse
    const int64_t rem = L - dl * per_dir;
    const int64_t bh = rem / NTILE;
    const int tile = (int)(rem - bh * NTILE);
    const int i0 = (tile / NTJ) * TI, j0 = (tile % NTJ) * TJ;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const int g = h / (H / G);
    const int64_t E = (int64_t)dk * dv;
    const int64_t NSC = (NC + CPS - 1) / CPS;        // steps holding real chunks
    const int64_t NS = (NSC + PD - 1) / PD * PD;      // steps, rounded up
    const int wave = threadIdx.x >> 6;

    if (wave >= 4) {
        // ---------------- loader waves
        const int lt = threadIdx.x - 256;
        const float *Asrc = (dir == 0 ? k : q) + (b * G + g) * T * dk;   // row 0, column 0
        const float *Bsrc = (dir == 0 ? v : dy) + bh * T * dv;
        const float *bcb = bcum + bh * NC * CH;
        const rsrc_t blr = make_rsrc(bl + bh * NCp, NC * 4);
        const int lima = dk - i0, limb = dv - j0;
        struct Stage {
            float4 a[APER], b[BPER];
            float at[APER], blc;
        };
        Stage stg[PD][CPS];
        // operands of chunk n of the scan order; chunks past the end load zeros
        auto prefetch = [&](Stage &S, int64_t n) {
            const bool live = n < NC;
            const int64_t c = live ? (dir == 0 ? n : NC - 1 - n) : 0;
            const int rows = (int)((T - c * CH) < CH ? (T - c * CH) : CH);
            const rsrc_t ab = make_rsrc(Asrc + c * CH * dk, live ? (int64_t)rows * dk * 4 : 0);
            const rsrc_t bb = make_rsrc(Bsrc + c * CH * dv, live ? (int64_t)rows * dv * 4 : 0);
            const rsrc_t br = make_rsrc(bcb + c * CH, live ? CH * 4 : 0);
#pragma unroll
            for (int u = 0; u < APER; ++u) {
                const int r = f4_row<TI / 4, NLT>(lt, u), c4 = f4_col<TI / 4>(lt);
                const bool ok = A4 % NLT == 0 || r < CH;
                S.a[u] = load4(ab, (uint32_t)(r * dk + i0), c4, lima, ok, VEC);
                S.at[u] = gload1(br, ok ? (uint32_t)r * 4u : kOOB);
            }
#pragma unroll
            for (int u = 0; u < BPER; ++u) {
                const int r = f4_row<TJ / 4, NLT>(lt, u), c4 = f4_col<TJ / 4>(lt);
                S.b[u] = load4(bb, (uint32_t)(r * dv + j0), c4, limb, B4 % NLT == 0 || r < CH, VEC);
            }
            // a vector load: a scalar one would be waited for right here
            S.blc = gload1(blr, live ? (uint32_t)c * 4u : kOOB);
        };
        // stage S into LDS half `buf`, slot cc; the rows of the A tile (TI
        // wide, the narrower one) are scaled by the decay weights
        auto stage = [&](const Stage &S, int buf, int cc) {
#pragma unroll
            for (int u = 0; u < APER; ++u) {
                const int r = f4_row<TI / 4, NLT>(lt, u), c4 = f4_col<TI / 4>(lt);
                if (A4 % NLT == 0 || r < CH) {
                    const float w = (dir == 0) ? __expf(S.blc - S.at[u]) : __expf(S.at[u]);
                    float4 x = S.a[u];
                    x.x *= w;
                    x.y *= w;
                    x.z *= w;
                    x.w *= w;
                    *reinterpret_cast<float4 *>(&As[buf][cc][r * LDA + c4]) = x;
                }
            }
#pragma unroll
            for (int u = 0; u < BPER; ++u) {
                const int r = f4_row<TJ / 4, NLT>(lt, u), c4 = f4_col<TJ / 4>(lt);
                if (B4 % NLT == 0 || r < CH) {
                    *reinterpret_cast<float4 *>(&Bs[buf][cc][r * LDB + c4]) = S.b[u];
                }
            }
            if (lt == 0) decs[buf][cc] = expf(S.blc);
        };
        // step s: its chunks are published by the barrier; stage step s + 1
        // into the other half and refill its registers with step s + 1 + PD
        auto step = [&](int64_t s, int u) {
            block_sync();
            const int un = (u + 1) % PD;
#pragma unroll
            for (int cc = 0; cc < CPS; ++cc) {
                stage(stg[un][cc], (int)((s + 1) & 1), cc);
                prefetch(stg[un][cc], (s + 1 + PD) * CPS + cc);
            }
        };
#pragma unroll
        for (int u = 0; u < PD; ++u) {
#pragma unroll
            for (int cc = 0; cc < CPS; ++cc) prefetch(stg[u][cc], (int64_t)u * CPS + cc);
        }
#pragma unroll
        for (int cc = 0; cc < CPS; ++cc) {
            stage(stg[0][cc], 0, cc);
            prefetch(stg[0][cc], (int64_t)PD * CPS + cc);
        }
        // the first PD steps are peeled so that the loop is entered with the
        // loads in flight that it repeats with
#pragma unroll
        for (int u = 0; u < PD; ++u) step(u, u);
        for (int64_t s0 = PD; s0 < NS; s0 += PD) {
#pragma unroll
            for (int u = 0; u < PD; ++u) step(s0 + u, u);
        }
        return;
    }

    // ---------------- compute waves
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int rblk = wave & 1;              // 16-row block of the tile
    const int wc0 = (wave >> 1) * WC;       // first column of this wave within the tile
    float *slab = (dir == 0 ? states : dstates) + bh * NC * Epad;

    // byte offset of accumulator (u, r) in a dk x dv state, kOOB outside it
    auto soff = [&](int u, int r) -> uint32_t {
        const int row = i0 + rblk * 16 + 4 * q4 + r, col = j0 + wc0 + NU * l16 + u;
        return (row < dk && col < dv) ? (uint32_t)(row * dv + col) * 4u : kOOB;
    };
    f32x4 acc[NU];
    {
        const rsrc_t hr = make_rsrc(h0 + bh * E, dir == 0 ? E * 4 : 0);   // the reverse pass starts at 0
#pragma unroll
        for (int u = 0; u < NU; ++u) {
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[u][r] = gload1(hr, soff(u, r));
            // Wait for the h0 loads here: otherwise every state store in the
            // loop waits on the stores before it.
            asm volatile("" : "+v"(acc[u]));
        }
    }
    for (int64_t s = 0; s < NS; ++s) {
        const int buf = (int)(s & 1);
        block_sync();   // step s staged in half `buf`
#pragma unroll
        for (int cc = 0; cc < CPS; ++cc) {
            float av[CH / 4];
            float bv[CH / 4][NU];
            const float *Ab = &As[buf][cc][q4 * LDA + rblk * 16 + l16];
            const float *Bb = &Bs[buf][cc][q4 * LDB + wc0 + NU * l16];
#pragma unroll
            for (int kk = 0; kk < CH / 4; ++kk) {
                av[kk] = Ab[4 * kk * LDA];
                if constexpr (NU == 4) {
                    const float4 t4 = *reinterpret_cast<const float4 *>(Bb + 4 * kk * LDB);
                    bv[kk][0] = t4.x;
                    bv[kk][1] = t4.y;
                    bv[kk][2] = t4.z;
                    bv[kk][3] = t4.w;
                } else if constexpr (NU == 2) {
                    const float2 t2 = *reinterpret_cast<const float2 *>(Bb + 4 * kk * LDB);
                    bv[kk][0] = t2.x;
                    bv[kk][1] = t2.y;
                } else {
                    bv[kk][0] = Bb[4 * kk * LDB];
                }
            }
            const float decay = decs[buf][cc];
            // slab[c] = S (state entering the chunk in this direction); no-op chunks store nothing
            const int64_t n = s * CPS + cc;
            const bool live = n < NC;
            const rsrc_t dst =
                make_rsrc(slab + (live ? (dir == 0 ? n : NC - 1 - n) : 0) * Epad, live ? E * 4 : 0);
            if constexpr (VEC) {
                // the lane's NU columns of a row are consecutive (dv % 4 == 0,
                // so they are inside the state when the first one is)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float sv[NU];
#pragma unroll
                    for (int u = 0; u < NU; ++u) sv[u] = acc[u][r];
                    gstoreN_nt<NU>(dst, soff(0, r), sv);
                }
            } else {
#pragma unroll
                for (int u = 0; u < NU; ++u) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) gstore1_nt(dst, soff(u, r), acc[u][r]);
                }
            }
#pragma unroll
            for (int u = 0; u < NU; ++u) {
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[u][r] *= decay;
            }
            // S += A^T B over the chunk's 64 positions
#pragma unroll
            for (int kk = 0; kk < CH / 4; ++kk) {
#pragma unroll
                for (int u = 0; u < NU; ++u) acc[u] = mfma16(av[kk], bv[kk][u], acc[u]);
            }
        }
    }
    if (dir == 1) {
        const rsrc_t hr = make_rsrc(dh0 + bh * E, E * 4);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
#pragma unroll
            for (int r = 0; r < 4; ++r) gstore1(hr, soff(u, r), acc[u][r]);
        }
    }
}

// ---------------------------------------------------------------------------
// K2 + K5: output of one chunk for every head of one group.
//
// One block of 8 waves per (b, g, chunk).  Wave w owns the 32 positions
// rt = w / 4 of the chunk and, for one head at a time, one 32-column block
// of Y, all on v_mfma_f32_32x32x2f32.  A step covers HPS = 128 / DVP heads
// (one for dv = 128): slot w % 4 picks head hs = slot / NCT of the step and
// column block ct = slot % NCT.
//
//   Y[rows rt, cols ct] = diag(e^b) Q[rt] S_in[:, ct] + P[rt, :] V[:, ct]
//
// MFMA s of a contraction over d takes the index pair (8m + s, 8m + 4 + s)
// for s < 4, so a lane (kh, i) holds the four consecutive elements
// 8m + 4kh .. 8m + 4kh + 3 of its row in one float4.  Only the B operands of
// the two products are read from LDS, with 4-byte reads, so the LDS traffic
// per MFMA is a quarter of that of 16x16 tiles with both operands in LDS:
//   * Q[rt], the A operand of Q S_in, is the same for the group's heads and
//     stays in registers for the whole block;
//   * P[rt, :] is the A operand of P V.  Accumulator register r of the
//     transposed product K Q^T holds, in lane (kh, i), the element of row
//     8 (r / 4) + 4 kh + r % 4, which is exactly the index lane (kh, i)
//     supplies to MFMA r of a 32-deep contraction; so K Q^T is formed once
//     per block and kept in registers, and per head only its decay factors
//     exp(b_i - b_j) are applied.  The four waves of a row block each sum
//     a quarter of dk and exchange the partial sums through LDS;
//   * the step's S_in and V tiles are staged in LDS.  Their row stride
//     DVP + 8 puts the rows 4 apart that the two lane halves read into
//     different banks.
// The next step's tiles are loaded into registers meanwhile, their loads
// spread over the Q S_in MFMAs: a CU's load path moves about 16 bytes per
// clock, so issued together they would hold up the issuing waves for
// thousands of cycles.  LDS operands are read one MFMA group ahead.
template <int DKP, int DVP>
struct OutCfg {
    static constexpr int NCT = DVP / 32;          // 32-column blocks of Y per head
    static constexpr int HPS = 4 / NCT;           // heads per step
    static constexpr int LS = DVP + 8;            // S_in and V row stride
    static constexpr int LDK = DKP + 4;           // Q and K row stride (set-up)
    static constexpr int SN = HPS * DKP * LS;     // S_in tiles (floats)
    static constexpr int XN = 3 * 4 * 4 * 256;    // partial sums of K Q^T
    static constexpr int QKN = 2 * CH * LDK;      // Q and K tiles
    static constexpr int SXN = SN > XN ? (SN > QKN ? SN : QKN) : (XN > QKN ? XN : QKN);
    static constexpr int VN = HPS * CH * LS;
    static constexpr int SPH = (DKP * DVP / 4 + NTW - 1) / NTW;   // float4 / thread, one S_in
    static constexpr int VPH = CH * DVP / 4 / NTW;                // float4 / thread, one V tile
    static constexpr int NL = HPS * (SPH + VPH) + 1;              // loads / thread / step
    static constexpr int NQ = DKP / 8;                            // float4 of a Q row per lane
    static constexpr int NQQ = DKP / 32;                          // the same, per quarter of dk
    static constexpr int QPER = (CH * DKP / 4 + NTW - 1) / NTW;   // float4 / thread, one C x dk tile
    // With more than one column block per head, the NCT waves of a row block
    // need the same P: each forms 4 / NCT of its register groups into LDS
    // (per head, the three causal 32 x 32 tiles in MFMA A-operand order).
    static constexpr bool SHP = NCT > 1;
    static constexpr int APW = 4 / NCT;
    static constexpr int PN = SHP ? HPS * 3 * 16 * 64 : 4;
    static_assert(NTW % (DVP / 4) == 0, "a thread's float4 of a tile share their column");
};

template <int DKP, int DVP, bool VEC, bool EXD>
__global__ __launch_bounds__(NTW) void k_chunk_output(const float *__restrict__ q, const float *__restrict__ k,
                                                      const float *__restrict__ v, const float *__restrict__ bcum,
                                                      const float *__restrict__ states, float *__restrict__ y,
                                                      int G, int H, int64_t T, int dk, int dv, int64_t NC,
                                                      int64_t Epad, int hpb)
{
    using Cfg = OutCfg<DKP, DVP>;
    if constexpr (EXD) {   // dk == DKP, dv == DVP: index arithmetic on constants
        dk = DKP;
        dv = DVP;
        Epad = (int64_t)DKP * DVP;
    }
    constexpr int NCT = Cfg::NCT, HPS = Cfg::HPS, LS = Cfg::LS, LDK = Cfg::LDK;
    constexpr int SPH = Cfg::SPH, VPH = Cfg::VPH, NL = Cfg::NL, NQ = Cfg::NQ, NQQ = Cfg::NQQ;
    // S_in tiles; Q, K and then the K Q^T partial sums at set-up
    __shared__ __attribute__((aligned(16))) float SX[Cfg::SXN];
    __shared__ __attribute__((aligned(16))) float VS[Cfg::VN];
    __shared__ __attribute__((aligned(16))) float bs[HPS * CH];
    __shared__ __attribute__((aligned(16))) float eb[HPS * CH];
    __shared__ __attribute__((aligned(16))) float PS[Cfg::PN];   // [head][tile rt + jt][r][lane]

    // block ((b G + g) nsplit + split) NC + c takes heads [split hpb, split hpb + hpg) of group g
    const int hpg_all = H / G, nsplit = (hpg_all + hpb - 1) / hpb;
    const int64_t c = blockIdx.x % NC;
    const int64_t bgs = blockIdx.x / NC;
    const int split = (int)(bgs % nsplit);
    const int64_t bg = bgs / nsplit;
    const int g = (int)(bg % G);
    const int64_t b = bg / G;
    const int hpg = min(hpb, hpg_all - split * hpb);   // heads of this block
    const int64_t bh0 = b * H + (int64_t)g * hpg_all + (int64_t)split * hpb;
    const int rows = (int)((T - c * CH) < CH ? (T - c * CH) : CH);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int rt = wave >> 2, slot = wave & 3;
    const int hs = slot / NCT, ct = slot % NCT;
    const int64_t E = (int64_t)dk * dv;

    // Next step's S_in and V tiles and cumulative decays, in registers.
    // Heads past the group's last load zeros, so no load is conditional and
    // the compiler's count of loads in flight stays exact.  issue<U>() issues
    // load U of the NL loads of a step.
    float4 sbuf[HPS][SPH], vbuf[HPS][VPH];
    float bpre = 0.f;
    auto issue = [&](int step, int tid, int u) {
        if (u < NL - 1) {
            const bool isv = u >= HPS * SPH;
            const int uu = isv ? u - HPS * SPH : u;
            const int h2 = isv ? uu / VPH : uu / SPH, e = isv ? uu % VPH : uu % SPH;
            const int hh = step * HPS + h2;
            const bool live = hh < hpg;
            const int64_t bh = bh0 + (live ? hh : 0);
            // float4 tid + e NTW of the tile: row tid / (DVP/4) + e NTW / (DVP/4)
            const int r = (int)((unsigned)tid / (DVP / 4)) + e * (NTW / (DVP / 4));
            const int c4 = (int)((unsigned)tid % (DVP / 4)) * 4;
            if (!isv) {
                const rsrc_t sr = make_rsrc(states + (bh * NC + c) * Epad, live ? E * 4 : 0);
                sbuf[h2][e] = load4(sr, (uint32_t)(r * dv), c4, dv, (DKP * DVP / 4) % NTW == 0 || r < DKP, VEC);
            } else {
                const rsrc_t vr = make_rsrc(v + (bh * T + c * CH) * dv, live ? (int64_t)rows * dv * 4 : 0);
                vbuf[h2][e] = load4(vr, (uint32_t)(r * dv), c4, dv, true, VEC);
            }
        } else {
            // wave w < HPS loads head w's 64 cumulative decays
            const int hh = step * HPS + (wave < HPS ? wave : 0);
            const bool live = hh < hpg && wave < HPS;
            bpre = gload1(make_rsrc(bcum + (bh0 + (live ? hh : 0)) * NC * CH + c * CH, live ? CH * 4 : 0),
                          (uint32_t)(tid & 63) * 4u);
        }
    };
    auto stage = [&](int tid) {
#pragma unroll
        for (int h2 = 0; h2 < HPS; ++h2) {
#pragma unroll
            for (int u = 0; u < SPH; ++u) {
                const int r = (int)((unsigned)tid / (DVP / 4)) + u * (NTW / (DVP / 4));
                const int c4 = (int)((unsigned)tid % (DVP / 4)) * 4;
                if ((DKP * DVP / 4) % NTW == 0 || r < DKP)
                    *reinterpret_cast<float4 *>(SX + (h2 * DKP + r) * LS + c4) = sbuf[h2][u];
            }
#pragma unroll
            for (int u = 0; u < VPH; ++u) {
                const int r = (int)((unsigned)tid / (DVP / 4)) + u * (NTW / (DVP / 4));
                const int c4 = (int)((unsigned)tid % (DVP / 4)) * 4;
                *reinterpret_cast<float4 *>(VS + (h2 * CH + r) * LS + c4) = vbuf[h2][u];
            }
        }
        if (wave < HPS) {
            bs[wave * CH + (tid & 63)] = bpre;
            eb[wave * CH + (tid & 63)] = expf(bpre);
        }
    };

    // ---- block set-up: Q rows in registers, K Q^T, the first step staged.
    float4 qa[NQ];   // Q[32 rt + i][8m + 4kh .. 8m + 4kh + 3] in lane (kh, i)
    f32x16 kqt[2];   // (K Q^T)[32 jt + row(r)][32 rt + i], jt <= rt
    {
        const int tid = threadIdx.x, lane = tid & 63, cl = lane & 31, kh = lane >> 5;
        {
            float4 qb[Cfg::QPER], kb[Cfg::QPER];
            const int64_t tb = (int64_t)rows * dk * 4;
            tile_to_regs<CH, DKP, NTW, Cfg::QPER>(tid, qb, make_rsrc(q + (bg * T + c * CH) * dk, tb), dk, VEC);
            tile_to_regs<CH, DKP, NTW, Cfg::QPER>(tid, kb, make_rsrc(k + (bg * T + c * CH) * dk, tb), dk, VEC);
            regs_to_lds<CH, DKP, NTW, Cfg::QPER, LDK>(tid, qb, SX);
            regs_to_lds<CH, DKP, NTW, Cfg::QPER, LDK>(tid, kb, SX + CH * LDK);
        }
        block_sync();
#pragma unroll
        for (int u = 0; u < NL; ++u) issue(0, tid, u);
#pragma unroll
        for (int m = 0; m < NQ; ++m)
            qa[m] = *reinterpret_cast<const float4 *>(SX + (32 * rt + cl) * LDK + 8 * m + 4 * kh);
        // this wave's quarter of dk: m in [slot NQQ, slot NQQ + NQQ)
        float4 ka[2][NQQ];
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
            for (int mm = 0; mm < NQQ; ++mm)
                ka[jt][mm] = *reinterpret_cast<const float4 *>(SX + (CH + 32 * jt + cl) * LDK +
                                                               8 * (slot * NQQ + mm) + 4 * kh);
        }
        block_sync();   // Q and K read before the partial sums overwrite them
        f32x16 part[2] = {zero16(), zero16()};
#pragma unroll
        for (int m = 0; m < NQ; ++m) {
            if (m / NQQ == slot) {
#pragma unroll
                for (int jt = 0; jt < 2; ++jt) {
                    if (jt <= rt) {
                        const float4 x = ka[jt][m % NQQ], yq = qa[m];
                        part[jt] = mfma32(x.x, yq.x, part[jt]);
                        part[jt] = mfma32(x.y, yq.y, part[jt]);
                        part[jt] = mfma32(x.z, yq.z, part[jt]);
                        part[jt] = mfma32(x.w, yq.w, part[jt]);
                    }
                }
            }
        }
        // partial sums: tile rt + jt (0: rows 0-31 x cols 0-31, 1: 32-63 x 0-31,
        // 2: 32-63 x 32-63 of Q K^T), quarter slot, register group a
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
            if (jt <= rt) {
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    *reinterpret_cast<float4 *>(SX + ((((rt + jt) * 4 + slot) * 4 + a) * 64 + lane) * 4) =
                        make_float4(part[jt][4 * a], part[jt][4 * a + 1], part[jt][4 * a + 2], part[jt][4 * a + 3]);
            }
        }
        block_sync();
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
            kqt[jt] = zero16();
            if (jt <= rt) {
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const float4 x =
                            *reinterpret_cast<const float4 *>(SX + ((((rt + jt) * 4 + qq) * 4 + a) * 64 + lane) * 4);
                        kqt[jt][4 * a] += x.x;
                        kqt[jt][4 * a + 1] += x.y;
                        kqt[jt][4 * a + 2] += x.z;
                        kqt[jt][4 * a + 3] += x.w;
                    }
                }
            }
        }
        block_sync();   // partial sums read before S_in overwrites them
        stage(tid);
        block_sync();
    }

    const int nstep = (hpg + HPS - 1) / HPS;
    // The step loop is instantiated per row block: with rt a constant the
    // causal tests of P fold (the tile below the diagonal needs none) and
    // the P V loop has no branch.
    auto steps = [&](auto rt_c) {
        constexpr int rt = decltype(rt_c)::value ? 1 : 0;
        for (int st = 0; st < nstep; ++st) {
            // per-lane index arithmetic stays inside the loop (see k_bwd_grads)
            int tid = threadIdx.x;
            asm volatile("" : "+v"(tid));
            const int lane = tid & 63, cl = lane & 31, kh = lane >> 5;
            const int hh = st * HPS + hs;
            const bool live = hh < hpg;
            const int64_t bh = bh0 + (live ? hh : 0);
            const float *bsh = bs + hs * CH, *ebh = eb + hs * CH;
            const int i = 32 * rt + cl;
            const int dl = cl - 4 * kh;

            // p_ij = (Q K^T)_ij exp(b_i - b_j) for j <= i, exp(-inf) = 0 above the
            // diagonal.  j = 32 jt + 8a + 4kh + e and i = 32 rt + cl, so j <= i
            // compares the constant 8a + e with a per-lane bound.  The exponent
            // is the difference b_i - b_j, taken before any scaling: b log2(e)
            // stored per position would add a rounding of |b| to every exponent.
            auto pgroup = [&](int jt, int a, float out[4]) {
                const float bi = bsh[i];
                const float4 bj = *reinterpret_cast<const float4 *>(bsh + 32 * jt + 8 * a + 4 * kh);
                const float bjs[4] = {bj.x, bj.y, bj.z, bj.w};
                const int lim = dl + 32 * (rt - jt);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x = bi - bjs[e];
                    out[e] = kqt[jt][4 * a + e] * __expf(8 * a + e <= lim ? x : -INFINITY);
                }
            };
            if constexpr (Cfg::SHP) {
                // this wave's register groups a of P (ct is wave-uniform)
                float *pw = PS + (hs * 3 + rt) * 1024 + lane;
#pragma unroll
                for (int jt = 0; jt < 2; ++jt) {
                    if (jt <= rt) {
#pragma unroll
                        for (int a = 0; a < 4; ++a) {
                            if (a / Cfg::APW == ct) {
                                float o[4];
                                pgroup(jt, a, o);
#pragma unroll
                                for (int e = 0; e < 4; ++e) pw[jt * 1024 + (4 * a + e) * 64] = o[e];
                            }
                        }
                    }
                }
            }

            // Q S_in; MFMA group m issues the next step's loads [m NL / NQ, (m + 1) NL / NQ).
            // One accumulator chain: the other wave of the SIMD issues its
            // MFMAs meanwhile (two chains measured slower by the adds they need).
            f32x16 acc = zero16();
            {
                const float *sb = SX + (hs * DKP + 4 * kh) * LS + 32 * ct + cl;
                float bq[2][4];
#pragma unroll
                for (int s = 0; s < 4; ++s) bq[0][s] = sb[s * LS];
#pragma unroll
                for (int m = 0; m < NQ; ++m) {
                    if (m + 1 < NQ) {
#pragma unroll
                        for (int s = 0; s < 4; ++s) bq[(m + 1) & 1][s] = sb[(8 * (m + 1) + s) * LS];
                    }
#pragma unroll
                    for (int u = m * NL / NQ; u < (m + 1) * NL / NQ; ++u) issue(st + 1, tid, u);
                    acc = mfma32(qa[m].x, bq[m & 1][0], acc);
                    acc = mfma32(qa[m].y, bq[m & 1][1], acc);
                    acc = mfma32(qa[m].z, bq[m & 1][2], acc);
                    acc = mfma32(qa[m].w, bq[m & 1][3], acc);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if constexpr (Cfg::SHP) block_sync();   // every wave's part of P written
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const float4 e = *reinterpret_cast<const float4 *>(ebh + 32 * rt + 8 * a + 4 * kh);
                acc[4 * a] *= e.x;
                acc[4 * a + 1] *= e.y;
                acc[4 * a + 2] *= e.z;
                acc[4 * a + 3] *= e.w;
            }
            // P V; the row group's V operands and P (or decays) are read ahead.
            {
                const float *vb = VS + (hs * CH + 4 * kh) * LS + 32 * ct + cl;
                const float *pr = PS + (hs * 3 + rt) * 1024 + lane;
#pragma unroll
                for (int jt = 0; jt < 2; ++jt) {
                    if (jt <= rt) {
                        float bv[16], p[16];
#pragma unroll
                        for (int a = 0; a < 4; ++a) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                bv[4 * a + e] = vb[(32 * jt + 8 * a + e) * LS];
                                if constexpr (Cfg::SHP) p[4 * a + e] = pr[jt * 1024 + (4 * a + e) * 64];
                            }
                        }
                        if constexpr (!Cfg::SHP) {
                            __builtin_amdgcn_sched_barrier(0);   // all reads issued before the MFMAs
#pragma unroll
                            for (int a = 0; a < 4; ++a) pgroup(jt, a, p + 4 * a);
                        }
                        __builtin_amdgcn_sched_barrier(0);   // operands before the MFMAs
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc = mfma32(p[r], bv[r], acc);
                    }
                }
            }
            {
                const rsrc_t yb = make_rsrc(y + (bh * T + c * CH) * dv, live ? (int64_t)rows * dv * 4 : 0);
                const int n = 32 * ct + cl;
                // row 32 rt + acc_row(r, lane): the lane's offset plus a uniform
                // one per register (rows past the sequence end fall outside yb)
                const uint32_t base = n < dv ? (uint32_t)((32 * rt + 4 * kh) * dv + n) * 4u : kOOB;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    gstore1_nt(yb, base + (uint32_t)(8 * (r / 4) + r % 4) * (uint32_t)(dv * 4), acc[r]);
            }
            block_sync();   // S_in, V and decay reads done before the next step's writes
            stage(tid);
            block_sync();
        }
    };
    if (rt) steps(BoolC<true>{});
    else steps(BoolC<false>{});
}

// ---------------------------------------------------------------------------
// B3 + B4: gradients of one chunk for every head of one group.
//
// One block of 4 waves (one per SIMD, so a wave may hold up to 512 registers,
// the MFMA accumulators in AGPRs) per (b, g, chunk); the group's heads are
// taken in ascending order and dq, dk are summed over them in registers.  All
// products run on v_mfma_f32_32x32x2f32.  Wave w has side grp = w / 2 (0: dQ,
// 1: dK) and row block rt = w % 2 (positions 32 rt .. 32 rt + 31).  Per head:
//
//   pass 1 (state)  S_in and dS_out stream through LDS in double-buffered
//                   slabs of 32 state rows k.  Each wave keeps its 32 rows of
//                   dY (dQ side) or V (dK side) over all of dv in registers
//                   and accumulates, for every 32-row block of dk, the
//                   transposed tile
//                       dQ^T[k, rt] += e^b     x (S_in dY^T)[k, rt]
//                       dK^T[k, rt] += e^{b_L-b} x (dS_out V^T)[k, rt]
//                   (the scale is per position, i.e. per lane), together with
//                   the rows' dlog_alpha dot products, summed in-lane; and
//                       Gv[rt, cv] += K[rt, k] dS_out[k, cv]
//                   for its dv column blocks cv.  Each thread adds up
//                   <dS_out, S_in> over the elements it stages.
//   pass 2 (intra)  dY and V go to LDS.  With P = (Q K^T) o D and
//                   dP = (dY V^T) o D:
//                       dV = diag(e^{b_L - b}) Gv + P^T dY    (stored per head)
//                       dQ^T += K^T dP^T,  dK^T += Q^T dP
//                   and dlog_alpha for the chunk's positions.
//
// Q K^T is formed once per block and kept in LDS in the accumulator layout of
// Q K^T tiles (register r of lane (kh, j): row 8 (r / 4) + 4 kh + r % 4,
// column j), which is the operand layout of P^T in P^T dY and matches the
// accumulators of the dY V^T tiles, so P, dP and M = (Q K^T) o D o (dY V^T)
// need no data movement.  dP goes to LDS once for the two intra products.
//
// The rectangle sums R_r = sum_{i >= r, j < r} M_ij of dlog_alpha use that
// only the strictly lower triangle of M enters, and an element M_ij (j < i)
// is counted for r in (j, i]:
//     R_r = sum_{t < r} (c_t - w_t),  c_t = sum_{i > t} M_it,  w_t = sum_{j < t} M_tj,
// so the chunk needs the row and column sums of M's strictly lower part and
// one exclusive prefix sum, all from registers.
constexpr int NTB = 256;   // 4 waves, one per SIMD

template <int DKP, int DVP>
struct BwdCfg {
    static constexpr int cmax(int a, int b) { return a > b ? a : b; }
    static constexpr int NKS = DKP / 32;      // 32-row slabs of the states
    static constexpr int NCT = DVP / 32;      // 32-column blocks of dv
    static constexpr int NCW = NCT >= 2 ? NCT / 2 : 1;   // dV column blocks per wave
    static constexpr int NA = DVP / 8;        // float4 of a dY / V row per lane
    static constexpr int LDQ = DKP + 4;       // Q rows (column reads pair rows i, i + 8)
    static constexpr int LDK = DKP + 8;       // K rows (column reads pair rows j, j + 4)
    static constexpr int LSL = DVP + 4;       // slab rows (column reads pair rows k, k + 8)
    static constexpr int LDY = DVP + 8;       // dY, V rows (column reads pair rows i, i + 4)
    static constexpr int LDP = CH + 4;        // dP rows (column reads pair rows i, i + 8)
    static constexpr int SLN = 32 * LSL;      // one slab of one state
    static constexpr int XN = cmax(cmax(cmax(4 * SLN, 2 * CH * LDY), 2 * CH * LDQ),
                                   cmax(12 * 1024, 1024 + CH * LDP));
    static constexpr int SPER = (32 * DVP / 4 + NTB - 1) / NTB;   // float4 / thread, one slab of one state
    static constexpr int QPER = (CH * DKP / 4 + NTB - 1) / NTB;   // float4 / thread, one C x dk tile
    static constexpr int NQQ = DKP / 32;                          // float4 per lane, a quarter of dk
};

template <int DKP, int DVP, bool VEC, bool EXD>
__global__ __launch_bounds__(NTB) void k_bwd_grads(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ dy, const float *__restrict__ bcum, const float *__restrict__ bl,
    const float *__restrict__ states, const float *__restrict__ dstates, float *__restrict__ dq,
    float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ dla, int G, int H, int64_t T, int dk_,
    int dv_, int64_t NC, int64_t NCp, int64_t Epad, int hpb, int64_t pstride)
{
    using Cfg = BwdCfg<DKP, DVP>;
    if constexpr (EXD) {   // dk == DKP, dv == DVP: index arithmetic on constants
        dk_ = DKP;
        dv_ = DVP;
        Epad = (int64_t)DKP * DVP;
    }
    constexpr int NKS = Cfg::NKS, NCT = Cfg::NCT, NCW = Cfg::NCW, NA = Cfg::NA;
    constexpr int LDQ = Cfg::LDQ, LDK = Cfg::LDK, LSL = Cfg::LSL, LDY = Cfg::LDY, LDP = Cfg::LDP;
    constexpr int SLN = Cfg::SLN, SPER = Cfg::SPER, QPER = Cfg::QPER, NQQ = Cfg::NQQ;
    __shared__ __attribute__((aligned(16))) float QL[CH * LDQ];
    __shared__ __attribute__((aligned(16))) float KL[CH * LDK];
    // slabs (pass 1); dY, V and then dP (pass 2); partial sums (set-up, end)
    __shared__ __attribute__((aligned(16))) float X[Cfg::XN];
    __shared__ __attribute__((aligned(16))) float QKT[3 * 1024];   // Q K^T tiles, accumulator layout
    __shared__ __attribute__((aligned(16))) float bs[CH], eb[CH], el[CH];
    __shared__ float redq[CH], redk[CH], rsm[3][32], csm[3][32], redf[NTB / 64], sfx[CH];

    // block ((b G + g) nsplit + split) NC + c takes heads [split hpb, split hpb + hpg) of group g
    const int hpg_all = H / G, nsplit = (hpg_all + hpb - 1) / hpb;
    const int64_t c = blockIdx.x % NC;
    const int64_t bgs = blockIdx.x / NC;
    const int split = (int)(bgs % nsplit);
    const int64_t bg = bgs / nsplit;
    const int g = (int)(bg % G);
    const int64_t b = bg / G;
    const int hpg = min(hpb, hpg_all - split * hpb);   // heads of this block
    const int64_t bh0 = b * H + (int64_t)g * hpg_all + (int64_t)split * hpb;
    // dq and dk: the split's partial sums over its heads (pstride = 0 without a split)
    dq += split * pstride;
    dk += split * pstride;
    const int rows = (int)((T - c * CH) < CH ? (T - c * CH) : CH);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int grp = wave >> 1, rt = wave & 1;
    // owns dV tiles (rt, grp NCW + u); every wave does when dv > 32, and a
    // compile-time true spares the accumulators a zero fill for the other path
    const bool gvw = NCT >= 2 || grp * NCW < NCT;
    const int64_t E = (int64_t)dk_ * dv_;

    struct Slab { float4 s[SPER], d[SPER]; };
    float4 ar[NA];             // dY (dQ side) or V (dK side): row 32 rt + i, columns 8m + 4kh .. + 3
    // QKT[t][a][lane][e] = register 4a + e of lane `lane` of Q K^T tile t
    // (t = 0: rows 0-31 x cols 0-31, 1: rows 32-63 x cols 0-31, 2: rows 32-63 x cols 32-63)
    auto qkt4 = [&](int t, int a, int lane) {
        return *reinterpret_cast<const float4 *>(QKT + t * 1024 + (a * 64 + lane) * 4);
    };
    Slab p0, pn;               // the next head's slabs 0 and 1; in pass 1, the next slab to stage
    float bpre = 0.f, blpre = 0.f;

    auto load_a1 = [&](int hh, int tid, int m) {   // float4 m of the wave's A rows of head hh
        const bool live = hh < hpg;
        const int64_t bh = bh0 + (live ? hh : 0);
        const float *src = (grp ? v : dy) + (bh * T + c * CH) * dv_;
        const rsrc_t r = make_rsrc(src, live ? (int64_t)rows * dv_ * 4 : 0);
        const int lane = tid & 63, cl = lane & 31, kh = lane >> 5;
        ar[m] = load4(r, (uint32_t)((32 * rt + cl) * dv_), 8 * m + 4 * kh, dv_, true, VEC);
    };
    // float4 u of one slab of S_in and of dS_out
    auto load_slab1 = [&](Slab &p, int hh, int ks, int tid, int u) {
        const bool live = hh < hpg;
        const int64_t off = ((bh0 + (live ? hh : 0)) * NC + c) * Epad;
        const rsrc_t sr = make_rsrc(states + off, live ? E * 4 : 0), dr = make_rsrc(dstates + off, live ? E * 4 : 0);
        const int r = f4_row<DVP / 4, NTB>(tid, u), c4 = f4_col<DVP / 4>(tid);
        const bool ok = (32 * DVP / 4) % NTB == 0 || r < 32;
        p.s[u] = load4(sr, (uint32_t)((32 * ks + r) * dv_), c4, dv_, ok, VEC);
        p.d[u] = load4(dr, (uint32_t)((32 * ks + r) * dv_), c4, dv_, ok, VEC);
    };
    // The next head's slabs 0 and 1 are loaded during the intra products, one
    // float4 of each state per MFMA step (step s: slab 0's float4 s, then slab
    // 1's), so that the loads of the four waves do not queue up in one burst.
    static_assert(2 * SPER <= 16, "the shortest intra loop has 16 steps");
    auto spread_ld = [&](int hh, int tid, int s) {
        if (s < SPER) load_slab1(p0, hh, 0, tid, s);
        else if (NKS > 1 && s < 2 * SPER) load_slab1(pn, hh, 1, tid, s - SPER);
    };
    auto load_slab = [&](Slab &p, int hh, int ks, int tid) {
#pragma unroll
        for (int u = 0; u < SPER; ++u) load_slab1(p, hh, ks, tid, u);
    };
    // Stage float4 u of a slab into buffer buf; returns this thread's part of
    // <dS_out, S_in> over it.
    auto store_piece = [&](const Slab &p, int buf, int tid, int u) -> float {
        const int idx = tid + u * NTB;
        if (idx >= 32 * DVP / 4) return 0.f;
        float *ds = X + buf * 2 * SLN;
        const int r = idx / (DVP / 4), c4 = (idx % (DVP / 4)) * 4;
        *reinterpret_cast<float4 *>(ds + r * LSL + c4) = p.s[u];
        *reinterpret_cast<float4 *>(ds + SLN + r * LSL + c4) = p.d[u];
        return p.s[u].x * p.d[u].x + p.s[u].y * p.d[u].y + p.s[u].z * p.d[u].z + p.s[u].w * p.d[u].w;
    };
    // Stage a slab into buffer buf; returns this thread's part of <dS_out, S_in>.
    auto store_slab = [&](const Slab &p, int buf, int tid) -> float {
        float f = 0.f;
        float *ds = X + buf * 2 * SLN;
#pragma unroll
        for (int u = 0; u < SPER; ++u) {
            const int r = f4_row<DVP / 4, NTB>(tid, u), c4 = f4_col<DVP / 4>(tid);
            if ((32 * DVP / 4) % NTB == 0 || r < 32) {
                *reinterpret_cast<float4 *>(ds + r * LSL + c4) = p.s[u];
                *reinterpret_cast<float4 *>(ds + SLN + r * LSL + c4) = p.d[u];
                f += p.s[u].x * p.d[u].x + p.s[u].y * p.d[u].y + p.s[u].z * p.d[u].z + p.s[u].w * p.d[u].w;
            }
        }
        return f;
    };
    auto load_b = [&](int hh, int tid) {
        const bool live = hh < hpg;
        const int64_t bh = bh0 + (live ? hh : 0);
        bpre = gload1(make_rsrc(bcum + bh * NC * CH + c * CH, live ? CH * 4 : 0), (uint32_t)(tid & 63) * 4u);
        blpre = gload1(make_rsrc(bl + bh * NCp + c, live ? 4 : 0), 0u);
    };
    auto stage_b = [&](int tid) {
        if (tid < CH) {
            bs[tid] = bpre;
            eb[tid] = expf(bpre);
            el[tid] = (tid < rows) ? expf(blpre - bpre) : 0.f;
        }
    };

    // ---- block set-up: Q, K in LDS; Q K^T; the first head's operands.
    float fro_next;
    {
        const int tid = threadIdx.x, lane = tid & 63, cl = lane & 31, kh = lane >> 5;
        {
            float4 qb[QPER], kb[QPER];
            const int64_t tb = (int64_t)rows * dk_ * 4;
            tile_to_regs<CH, DKP, NTB, QPER>(tid, qb, make_rsrc(q + (bg * T + c * CH) * dk_, tb), dk_, VEC);
            tile_to_regs<CH, DKP, NTB, QPER>(tid, kb, make_rsrc(k + (bg * T + c * CH) * dk_, tb), dk_, VEC);
#pragma unroll
            for (int m = 0; m < NA; ++m) load_a1(0, tid, m);
            load_slab(p0, 0, 0, tid);
            if (NKS > 1) load_slab(pn, 0, 1, tid);
            load_b(0, tid);
            regs_to_lds<CH, DKP, NTB, QPER, LDQ>(tid, qb, QL);
            regs_to_lds<CH, DKP, NTB, QPER, LDK>(tid, kb, KL);
        }
        block_sync();
        // 12 units (tile t, quarter of dk); wave w takes units w, w + 4, w + 8
#pragma unroll
        for (int uu = 0; uu < 3; ++uu) {
            const int u = wave + 4 * uu;
            const int t = u >> 2, qt = u & 3, it = t > 0, jt = t == 2;
            f32x16 acc = zero16();
#pragma unroll
            for (int mm = 0; mm < NQQ; ++mm) {
                const int col = 8 * (qt * NQQ + mm) + 4 * kh;
                const float4 x = *reinterpret_cast<const float4 *>(QL + (32 * it + cl) * LDQ + col);
                const float4 y = *reinterpret_cast<const float4 *>(KL + (32 * jt + cl) * LDK + col);
                acc = mfma32(x.x, y.x, acc);
                acc = mfma32(x.y, y.y, acc);
                acc = mfma32(x.z, y.z, acc);
                acc = mfma32(x.w, y.w, acc);
            }
#pragma unroll
            for (int a = 0; a < 4; ++a)
                *reinterpret_cast<float4 *>(X + ((u * 4 + a) * 64 + lane) * 4) =
                    make_float4(acc[4 * a], acc[4 * a + 1], acc[4 * a + 2], acc[4 * a + 3]);
        }
        block_sync();
        // sum the four quarters of each tile
        for (int f = tid; f < 3 * 256; f += NTB) {
            const int t = f >> 8, o = (f & 255) * 4;
            float4 acc4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int qt = 0; qt < 4; ++qt) {
                const float4 x = *reinterpret_cast<const float4 *>(X + (t * 4 + qt) * 1024 + o);
                acc4.x += x.x;
                acc4.y += x.y;
                acc4.z += x.z;
                acc4.w += x.w;
            }
            *reinterpret_cast<float4 *>(QKT + t * 1024 + o) = acc4;
        }
        block_sync();   // partial sums read before the slabs overwrite them
        fro_next = store_slab(p0, 0, tid);
        if (NKS > 1) fro_next += store_slab(pn, 1, tid);
        stage_b(tid);
        block_sync();
    }

    f32x16 dacc[NKS];   // dQ^T (dQ side) or dK^T (dK side): state rows 32 ks + row(r), positions 32 rt + i
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) dacc[ks] = zero16();
    // wave 0: dQ^T rows 32 (NKS - 1) .., positions 32 ..; wave 3: dK^T rows
    // 32 (NKS - 1) .., positions 0 .. (intra parts taken over from waves 1, 2)
    constexpr bool OFF = NKS > 1;
    f32x16 xacc = zero16();

    for (int hh = 0; hh < hpg; ++hh) {
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, cl = lane & 31, kh = lane >> 5;
        const int64_t bh = bh0 + hh;
        const float blh = blpre;
        float fro = fro_next;
        f32x16 gv[NCW];
#pragma unroll
        for (int u = 0; u < NCW; ++u) gv[u] = zero16();

        // ---- pass 1: state slabs
        const float *W = grp ? KL : QL;
        const int ldw = grp ? LDK : LDQ;
        // Fold one slab's tile, held transposed (register r of lane (kh, i): state
        // row 32 ks + row(r), position 32 rt + i): dQ^T (dK^T) += tile x the
        // position's scale, and the lane adds the position's dot product with its
        // Q (K) row over those state rows.
        const float sa = (grp ? el : eb)[32 * rt + cl];   // e^b (dQ) or e^{b_L - b} (dK)
        float rd = 0.f;
        auto fold = [&](const f32x16 &gt, const int ks) {
            const float *wr = W + (32 * rt + cl) * ldw + 32 * ks + 4 * kh;
            float t = 0.f;
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const float4 w4 = *reinterpret_cast<const float4 *>(wr + 8 * a);
                const float ws[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * a + e;
                    dacc[ks][r] += sa * gt[r];
                    t += gt[r] * ws[e];
                }
            }
            rd += sa * t;
        };
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if (ks > 0) block_sync();   // slab ks visible, slab ks - 1 read
            const float *sS = X + (ks & 1) * 2 * SLN, *sD = sS + SLN;
            // Gv operands (MFMA group g2 contracts slab rows (16 (g2 / 2) + 4 (g2 % 2) + e, + 8))
            const float *kp = KL + (32 * rt + cl) * LDK + 32 * ks + 8 * kh;
            const float *bd = sD + 8 * kh * LSL + 32 * grp * NCW + cl;
            float4 xk[2];
            float bv[2][NCW][4];
            auto ldv = [&](int g2, int buf) {
                const int o = 16 * (g2 >> 1) + 4 * (g2 & 1);
                xk[buf] = *reinterpret_cast<const float4 *>(kp + o);
#pragma unroll
                for (int u = 0; u < NCW; ++u) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) bv[buf][u][e] = bd[(o + e) * LSL + 32 * u];
                }
            };
            // Gq / Gk: A = slab rows (row i of the slab in lane i), B = the wave's rows;
            // operands read one MFMA group ahead.  Spread over the first groups: the
            // next slab goes from registers to the free buffer and the one after it
            // is loaded, one float4 of each state per two groups, so that neither
            // the LDS writes nor the global loads arrive in a burst; the last group
            // reads the first Gv operands.
            f32x16 gt = zero16();
            {
                const float *bp = (grp ? sD : sS) + cl * LSL + 4 * kh;
                float4 yb[2];
                yb[0] = *reinterpret_cast<const float4 *>(bp);
#pragma unroll
                for (int m = 0; m < NA; ++m) {
                    if (m + 1 < NA) yb[(m + 1) & 1] = *reinterpret_cast<const float4 *>(bp + 8 * (m + 1));
                    const float4 y = yb[m & 1];
                    gt = mfma32(y.x, ar[m].x, gt);
                    gt = mfma32(y.y, ar[m].y, gt);
                    gt = mfma32(y.z, ar[m].z, gt);
                    gt = mfma32(y.w, ar[m].w, gt);
                    if ((m & 1) && (m >> 1) < SPER) {
                        if (ks >= 1 && ks + 1 < NKS) fro += store_piece(pn, (ks + 1) & 1, tid, m >> 1);
                        if (ks + 2 < NKS) load_slab1(pn, hh, ks + 2, tid, m >> 1);
                    }
                    if (m == NA - 1 && gvw) ldv(0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if (gvw) {
#pragma unroll
                for (int g2 = 0; g2 < 4; ++g2) {
                    if (g2 + 1 < 4) ldv(g2 + 1, (g2 + 1) & 1);
                    const float4 x = xk[g2 & 1];
                    const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
#pragma unroll
                        for (int u = 0; u < NCW; ++u) gv[u] = mfma32(xs[e], bv[g2 & 1][u][e], gv[u]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            fold(gt, ks);
        }
        // the two lane halves hold the dot products over different state rows
        rd += __shfl_xor(rd, 32);
        if (kh == 0) (grp ? redk : redq)[32 * rt + cl] = rd;
        fro = sum64_hi(fro);
        if (lane == 63) redf[wave] = fro;
        block_sync();   // slabs read
        {
            float *dst = X + (grp ? CH * LDY : 0) + (32 * rt + cl) * LDY + 4 * kh;
#pragma unroll
            for (int m = 0; m < NA; ++m) *reinterpret_cast<float4 *>(dst + 8 * m) = ar[m];
        }
        block_sync();   // dY and V in LDS

        // ---- pass 2
        const float *RY = X, *RV = X + CH * LDY;
        // dV tiles (rows 32 rt + row(r), columns 32 (grp NCW + u) + i) =
        // diag(e^{b_L - b}) Gv + P^T dY.  P is formed per row block of positions,
        // then the MFMAs run.
        if (gvw) {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const float4 e4 = *reinterpret_cast<const float4 *>(el + 32 * rt + 8 * a + 4 * kh);
#pragma unroll
                for (int u = 0; u < NCW; ++u) {
                    gv[u][4 * a] *= e4.x;
                    gv[u][4 * a + 1] *= e4.y;
                    gv[u][4 * a + 2] *= e4.z;
                    gv[u][4 * a + 3] *= e4.w;
                }
            }
            // j = 32 rt + cl, i = 32 it + 8a + 4kh + e: j <= i is 8a + e >= lim
            const int j = 32 * rt + cl;
            const float bj = bs[j];
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                if (it >= rt) {
                    float p[16];
                    const int lim = cl - 4 * kh + 32 * (rt - it);
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const float4 k4 = qkt4(it + rt, a, lane);
                        const float4 b4 = *reinterpret_cast<const float4 *>(bs + 32 * it + 8 * a + 4 * kh);
                        const float ks4[4] = {k4.x, k4.y, k4.z, k4.w}, bis[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            p[4 * a + e] = ks4[e] * __expf(8 * a + e >= lim ? bis[e] - bj : -INFINITY);
                    }
                    // dY operands four registers (one group) ahead of their MFMAs,
                    // so no MFMA waits on the LDS read just issued before it
                    float yb[2][4][NCW];
                    auto ldy = [&](int g4, int buf) {
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) {
                            const int i = 32 * it + acc_row(4 * g4 + rr, lane);
#pragma unroll
                            for (int u = 0; u < NCW; ++u) yb[buf][rr][u] = RY[i * LDY + 32 * (grp * NCW + u) + cl];
                        }
                    };
                    ldy(0, 0);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        if (g4 + 1 < 4) ldy(g4 + 1, (g4 + 1) & 1);
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) {
#pragma unroll
                            for (int u = 0; u < NCW; ++u) gv[u] = mfma32(p[4 * g4 + rr], yb[g4 & 1][rr][u], gv[u]);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
            const rsrc_t dvb = make_rsrc(dv + (bh * T + c * CH) * dv_, (int64_t)rows * dv_ * 4);
#pragma unroll
            for (int u = 0; u < NCW; ++u) {
                const int n = 32 * (grp * NCW + u) + cl;
                // row 32 rt + acc_row(r, lane): the lane's offset plus a uniform
                // one per register (rows past the sequence end fall outside dvb)
                const uint32_t base = n < dv_ ? (uint32_t)((32 * rt + 4 * kh) * dv_ + n) * 4u : kOOB;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    gstore1_nt(dvb, base + (uint32_t)(8 * (r / 4) + r % 4) * (uint32_t)(dv_ * 4), gv[u][r]);
            }
        }
        // dY V^T tiles: tile 0 (rows 0-31 x cols 0-31) split over dv halves between
        // waves 0 and 2, tile 1 (32-63 x 0-31) on wave 1, tile 2 (32-63 x 32-63) on
        // wave 3, so that with the dV tiles every wave runs the same number of
        // MFMAs.  The next head's A rows are loaded LPG per MFMA group.
        f32x16 ad = zero16();
        auto dyvt = [&](f32x16 &acc, int it, int jt, int m0, int m1, int LPG) {
            const float *xa = RY + (32 * it + cl) * LDY + 4 * kh, *ya = RV + (32 * jt + cl) * LDY + 4 * kh;
            float4 xb[2], yb[2];
            xb[m0 & 1] = *reinterpret_cast<const float4 *>(xa + 8 * m0);
            yb[m0 & 1] = *reinterpret_cast<const float4 *>(ya + 8 * m0);
#pragma unroll
            for (int m = 0; m < NA; ++m) {
                if (m >= m0 && m < m1) {
                    if (m + 1 < m1) {
                        xb[(m + 1) & 1] = *reinterpret_cast<const float4 *>(xa + 8 * (m + 1));
                        yb[(m + 1) & 1] = *reinterpret_cast<const float4 *>(ya + 8 * (m + 1));
                    }
                    const float4 x = xb[m & 1], y = yb[m & 1];
                    acc = mfma32(x.x, y.x, acc);
                    acc = mfma32(x.y, y.y, acc);
                    acc = mfma32(x.z, y.z, acc);
                    acc = mfma32(x.w, y.w, acc);
#pragma unroll
                    for (int l = 0; l < LPG; ++l) load_a1(hh + 1, tid, (m - m0) * LPG + l);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        if (wave == 0) {
            dyvt(ad, 0, 0, 0, NA / 2, 2);
        } else if (wave == 1) {
            dyvt(ad, 1, 0, 0, NA, 1);
        } else if (wave == 2) {
            dyvt(ad, 0, 0, NA / 2, NA, 2);
        } else {
            dyvt(ad, 1, 1, 0, NA, 1);
        }
        load_b(hh + 1, tid);
        block_sync();   // dY and V read
        if (wave == 2) {
#pragma unroll
            for (int a = 0; a < 4; ++a)
                *reinterpret_cast<float4 *>(X + (a * 64 + lane) * 4) =
                    make_float4(ad[4 * a], ad[4 * a + 1], ad[4 * a + 2], ad[4 * a + 3]);
        }
        block_sync();   // wave 2's half of tile 0 visible
        float *const DP = X + 1024;   // dP [CH][LDP]

        if (wave != 2) {
            // dP = (dY V^T) o D to LDS, and the row and column sums of the strictly
            // lower part of M = (Q K^T) o D o (dY V^T)
            const int td = wave == 0 ? 0 : wave == 1 ? 1 : 2;
            const int it = td > 0, jt = td == 2;
            if (wave == 0) {
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const float4 x = *reinterpret_cast<const float4 *>(X + (a * 64 + lane) * 4);
                    ad[4 * a] += x.x;
                    ad[4 * a + 1] += x.y;
                    ad[4 * a + 2] += x.z;
                    ad[4 * a + 3] += x.w;
                }
            }
            const int j = 32 * jt + cl;
            const float bj = bs[j];
            const int lim = cl - 4 * kh + 32 * (jt - it);   // j <= i is 8a + e >= lim
            float ms[16], csum = 0.f;
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const float4 k4 = qkt4(td, a, lane);
                const float4 b4 = *reinterpret_cast<const float4 *>(bs + 32 * it + 8 * a + 4 * kh);
                const float ks4[4] = {k4.x, k4.y, k4.z, k4.w}, bis[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * a + e, i = 32 * it + 8 * a + 4 * kh + e;
                    const float d = __expf(8 * a + e >= lim ? bis[e] - bj : -INFINITY);
                    const float dp = ad[r] * d;
                    DP[i * LDP + j] = dp;
                    ms[r] = (8 * a + e > lim) ? ks4[e] * dp : 0.f;   // (Q K^T) o D o (dY V^T), j < i
                    csum += ms[r];
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) ms[r] = dpp_add<kRowRor + 8>(ms[r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) ms[r] = dpp_add<kRowRor + 4>(ms[r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) ms[r] = dpp_add<kRowRor + 2>(ms[r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) ms[r] = dpp_add<kRowRor + 1>(ms[r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) ms[r] = dpp_add<kRowBcast15, 0xa>(ms[r]);
            if (cl == 31) {
#pragma unroll
                for (int r = 0; r < 16; ++r) rsm[td][acc_row(r, lane)] = ms[r];
            }
            csum += __shfl_xor(csum, 32);
            if (kh == 0) csm[td][cl] = csum;
        }
        block_sync();   // dP and the reductions visible

        // Intra products.  The row blocks rt = 1 (dQ) and rt = 0 (dK) have twice
        // the work of the others, so with dk > 32 their last 32 state rows are
        // taken by the other wave of the side (wave 0 for wave 1, wave 3 for wave
        // 2), summed over heads in xacc and added at the end.
        // (the shedding waves are 1 and 2: rt = 1 on the dQ side, rt = 0 on the dK side)
        if (grp == 0) {
            // dQ^T[ct, rt] += K[:, ct]^T dP[rt, :]^T over j < 32 (rt + 1); all tiles
            // interleaved on independent chains
            const float *ap = DP + (32 * rt + cl) * LDP + 4 * kh;
            const float *bk = KL + 4 * kh * LDK + cl;
            // operands of step (a, e) are read one step ahead: x for the next a,
            // the K column values for the next e
            float4 xq[2];
            float kq[2][NKS];
            auto ldk = [&](int a, int e, int buf) {
#pragma unroll
                for (int ct = 0; ct < NKS; ++ct) kq[buf][ct] = bk[(8 * a + e) * LDK + 32 * ct];
            };
            // the loop is instantiated per row block (which also fixes whether
            // the wave sheds), so that no branch splits its MFMA stream
            auto dq_intra = [&](auto rt_c) {
                constexpr int RT = decltype(rt_c)::value ? 1 : 0;
                constexpr bool SH = OFF && RT == 1;   // sheds its last state block
                constexpr int na = 4 * (RT + 1);
                xq[0] = *reinterpret_cast<const float4 *>(ap);
                ldk(0, 0, 0);
#pragma unroll
                for (int a = 0; a < 8; ++a) {
                    if (a < na) {
                        if (a + 1 < na) xq[(a + 1) & 1] = *reinterpret_cast<const float4 *>(ap + 8 * (a + 1));
                        const float4 x = xq[a & 1];
                        const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int f = 4 * a + e;
                            if (e < 3) ldk(a, e + 1, (f + 1) & 1);
                            else if (a + 1 < na) ldk(a + 1, 0, (f + 1) & 1);
#pragma unroll
                            for (int ct = 0; ct < NKS; ++ct) {
                                if (ct < NKS - 1 || !SH) dacc[ct] = mfma32(kq[f & 1][ct], xs[e], dacc[ct]);
                            }
                            spread_ld(hh + 1, tid, f);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                }
            };
            if (rt) dq_intra(BoolC<true>{});
            else dq_intra(BoolC<false>{});
            if (OFF && wave == 0) {
                // dQ^T[NKS - 1, 1] for wave 1
                const float *ap1 = DP + (32 + cl) * LDP + 4 * kh;
                const float *bk1 = bk + 32 * (NKS - 1);
#pragma unroll
                for (int a = 0; a < 8; ++a) {
                    const float4 x = *reinterpret_cast<const float4 *>(ap1 + 8 * a);
                    xacc = mfma32(bk1[(8 * a + 0) * LDK], x.x, xacc);
                    xacc = mfma32(bk1[(8 * a + 1) * LDK], x.y, xacc);
                    xacc = mfma32(bk1[(8 * a + 2) * LDK], x.z, xacc);
                    xacc = mfma32(bk1[(8 * a + 3) * LDK], x.w, xacc);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
            // dK^T[ct, rt] += Q[:, ct]^T dP[:, rt] over i >= 32 rt; MFMA s = 8 g2 + e
            // contracts rows (i0 + 16 g2 + e, + 8)
            const float *ap = DP + 8 * kh * LDP + 32 * rt + cl;
            const float *bq = QL + 8 * kh * LDQ + cl;
            // step f = 16 it + 8 g2 + e contracts rows (32 it + 16 g2 + e, + 8); its
            // operands are read one step ahead
            float xd[2], qv[2][NKS];
            auto ldq = [&](int f, int buf) {
                const int i = 32 * (f >> 4) + 16 * ((f >> 3) & 1) + (f & 7);
                xd[buf] = ap[i * LDP];
#pragma unroll
                for (int ct = 0; ct < NKS; ++ct) qv[buf][ct] = bq[i * LDQ + 32 * ct];
            };
            auto dk_intra = [&](auto rt_c) {   // instantiated per row block
                constexpr int RT = decltype(rt_c)::value ? 1 : 0;
                constexpr bool SH = OFF && RT == 0;   // sheds its last state block
                ldq(16 * RT, 0);
#pragma unroll
                for (int f = 0; f < 32; ++f) {
                    if (f >= 16 * RT) {
                        if (f + 1 < 32) ldq(f + 1, (f + 1) & 1);
#pragma unroll
                        for (int ct = 0; ct < NKS; ++ct) {
                            if (ct < NKS - 1 || !SH) dacc[ct] = mfma32(qv[f & 1][ct], xd[f & 1], dacc[ct]);
                        }
                        spread_ld(hh + 1, tid, f - 16 * RT);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            };
            if (rt) dk_intra(BoolC<true>{});
            else dk_intra(BoolC<false>{});
            if (OFF && wave == 3) {
                // dK^T[NKS - 1, 0] for wave 2
                const float *ap0 = DP + 8 * kh * LDP + cl;
                const float *bq1 = bq + 32 * (NKS - 1);
#pragma unroll
                for (int it = 0; it < 2; ++it) {
#pragma unroll
                    for (int g2 = 0; g2 < 2; ++g2) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int i = 32 * it + 16 * g2 + e;
                            xacc = mfma32(bq1[i * LDQ], ap0[i * LDP], xacc);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
        }
        if (wave == 2) {
            // dlog_alpha_r = R_r + sum_{i >= r} iq_i + sum_{j < r} ik_j + e^{b_L} <dS_out, S_in>
            const int t = lane;
            const float ik = redk[t];
            const float rw = t < 32 ? rsm[0][t] : rsm[1][t - 32] + rsm[2][t - 32];
            const float cs = t < 32 ? csm[0][t] + csm[1][t] : csm[2][t - 32];
            float frob = 0.f;
#pragma unroll
            for (int w = 0; w < NTB / 64; ++w) frob += redf[w];
            // suffix sum of iq: prefix sum over the reversed rows
            sfx[63 - t] = scan64(redq[63 - t]);
            const float rr = shift_up1(scan64(cs - rw)), pk = shift_up1(scan64(ik));
            // lanes exchange through sfx: order the write before the read
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const float sq = sfx[t];
            gstore1(make_rsrc(dla + bh * T + c * CH, (int64_t)rows * 4), (uint32_t)t * 4u,
                    rr + sq + pk + expf(blh) * frob);
        }
        block_sync();   // dP, dY V^T sums and reductions read; the slab buffers are free
        fro_next = store_slab(p0, 0, tid);
        if (NKS > 1) fro_next += store_slab(pn, 1, tid);
        stage_b(tid);
        block_sync();
    }

    // ---- dq, dk: transposed through LDS into [position][dk] rows, stored with
    // 16-byte writes
    {
        const int tid = threadIdx.x, lane = tid & 63, cl = lane & 31, kh = lane >> 5;
        float *o = X + grp * CH * LDQ + (32 * rt + cl) * LDQ + 4 * kh;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
            for (int a = 0; a < 4; ++a)
                *reinterpret_cast<float4 *>(o + 32 * ks + 8 * a) =
                    make_float4(dacc[ks][4 * a], dacc[ks][4 * a + 1], dacc[ks][4 * a + 2], dacc[ks][4 * a + 3]);
        }
        block_sync();
        if (OFF && (wave == 0 || wave == 3)) {
            // add the tiles taken over from waves 1 (dQ, positions 32 ..) and 2 (dK, positions 0 ..)
            float *ox = X + grp * CH * LDQ + (32 * (1 - rt) + cl) * LDQ + 4 * kh + 32 * (NKS - 1);
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                float4 y = *reinterpret_cast<const float4 *>(ox + 8 * a);
                y.x += xacc[4 * a];
                y.y += xacc[4 * a + 1];
                y.z += xacc[4 * a + 2];
                y.w += xacc[4 * a + 3];
                *reinterpret_cast<float4 *>(ox + 8 * a) = y;
            }
        }
        block_sync();
        const int64_t tb = (int64_t)rows * dk_ * 4;
        const rsrc_t rq = make_rsrc(dq + (bg * T + c * CH) * dk_, tb), rk = make_rsrc(dk + (bg * T + c * CH) * dk_, tb);
        constexpr int Q4 = DKP / 4;
        for (int idx = tid; idx < 2 * CH * Q4; idx += NTB) {
            const int gg = idx / (CH * Q4), rem = idx - gg * CH * Q4;
            const int row = rem / Q4, c4 = (rem - row * Q4) * 4;
            const float4 x = *reinterpret_cast<const float4 *>(X + gg * CH * LDQ + row * LDQ + c4);
            const rsrc_t r = gg ? rk : rq;
            if (VEC) {
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(__attribute__((ext_vector_type(4))) int, x), r,
                    c4 < dk_ ? (uint32_t)(row * dk_ + c4) * 4u : kOOB, 0, 0);
            } else {
                const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    gstore1(r, c4 + e < dk_ ? (uint32_t)(row * dk_ + c4 + e) * 4u : kOOB, xs[e]);
            }
        }
    }
}

// Fill n floats with zero (used for dh0 when T == 0).
__global__ __launch_bounds__(NTH) void k_zero(float *__restrict__ p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * NTH + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

// dq or dk of a split gradient launch: out[i] = sum over the ns splits of
// parts[j * stride + i], added in split order.
__global__ __launch_bounds__(NTH) void k_sum_splits(float *__restrict__ out, const float *__restrict__ parts, int ns,
                                                    int64_t stride, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * NTH + threadIdx.x; i < n; i += (int64_t)gridDim.x * NTH) {
        float acc = parts[i];
        for (int j = 1; j < ns; ++j) acc += parts[j * stride + i];
        out[i] = acc;
    }
}

// ---------------------------------------------------------------------------
// Kernel timing (optional, process-global).

enum KernelId { KID_CUMSUM = 0, KID_SCAN, KID_OUTPUT, KID_SCAN2, KID_GRADS, KID_SCANR, KID_COUNT };
static const char *kKernelNames[KID_COUNT] = {"chunk_cumsum", "state_scan", "chunk_output", "state_scan_bidir",
                                              "bwd_grads", "state_scan_rev"};

struct Timing {
    unsigned mask = 0;   // bit kid: time kernel kid
    std::vector<hipEvent_t> pool;
    std::vector<hipEvent_t> pending[KID_COUNT][2];
    double total[KID_COUNT] = {};
    int64_t count[KID_COUNT] = {};
};
static Timing g_timing;

static hipEvent_t get_event()
{
    if (!g_timing.pool.empty()) {
        hipEvent_t e = g_timing.pool.back();
        g_timing.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Launches f on st.  When kernel kid is timed, the start and stop events are
// bound to the kernel's own dispatch through hipExtLaunchKernel, so they time
// the kernel alone and put no extra packets between kernels on the stream.
template <typename... P, typename... A>
static void launch(int kid, void (*f)(P...), dim3 grid, dim3 blk, hipStream_t st, A... a)
{
    static_assert(sizeof...(P) == sizeof...(A), "argument count");
    std::tuple<P...> args{static_cast<P>(a)...};
    void *ptrs[sizeof...(P)];
    std::apply([&](auto &...x) {
        int i = 0;
        ((ptrs[i++] = static_cast<void *>(&x)), ...);
    }, args);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (kid >= 0 && ((g_timing.mask >> kid) & 1u)) {
        e0 = get_event();
        e1 = get_event();
        if (!e0 || !e1) {
            if (e0) g_timing.pool.push_back(e0);
            if (e1) g_timing.pool.push_back(e1);
            e0 = e1 = nullptr;
        }
    }
    hipExtLaunchKernel(reinterpret_cast<const void *>(f), grid, blk, ptrs, 0, st, e0, e1, 0);
    if (e0 && e1) {
        g_timing.pending[kid][0].push_back(e0);
        g_timing.pending[kid][1].push_back(e1);
    }
}

static void collect_timing()
{
    for (int kid = 0; kid < KID_COUNT; ++kid) {
        auto &A = g_timing.pending[kid][0];
        auto &B = g_timing.pending[kid][1];
        for (size_t i = 0; i < A.size(); ++i) {
            float ms = 0.f;
            hipEventSynchronize(B[i]);
            if (hipEventElapsedTime(&ms, A[i], B[i]) == hipSuccess) {
                g_timing.total[kid] += ms;
                g_timing.count[kid] += 1;
            }
            g_timing.pool.push_back(A[i]);
            g_timing.pool.push_back(B[i]);
        }
        A.clear();
        B.clear();
    }
}

// ---------------------------------------------------------------------------
// Launch helpers.

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

struct Problem {
    ssd_shape s;
    Layout L;
    int DKP, DVP;
    bool vec;     // dk and dv multiples of 4: 16-byte loads
    bool exact;   // dk == DKP and dv == DVP: the kernels' index arithmetic on constants
    float *bcum, *bl, *states, *dstates;
    float *parts;   // split partial sums of dq, dk (backward with hsplit > 1), else null
};

static int launch_status()
{
    return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_DEVICE;
}

// Chunk cumsum (when `cumsum`), then the fused state scan over the
// directions in `dirs`: 1 = forward only (fills `states` with S_in), 3 = both
// in one launch (also fills `dstates` with dS_out and writes dh0), 2 = reverse
// only (dstates and dh0; bcum and bl must already hold the cumsum).
static int run_scan(const Problem &P, int dirs, bool cumsum, const float *q, const float *k, const float *v,
                    const float *dy, const float *la, const float *h0, float *dh0, hipStream_t st)
{
    const ssd_shape &s = P.s;
    const int64_t BH = s.B * s.H;
    if (cumsum) {
        const int64_t nw = BH * P.L.NC;
        const int64_t grid = (nw + 3) / 4;
        launch(KID_CUMSUM, k_chunk_cumsum, dim3((unsigned)grid), dim3(NTH), st, la, P.bcum, P.bl, s.T, P.L.NC,
               P.L.NCp, nw);
        if (launch_status() != SSD_OK) return SSD_ERR_DEVICE;
    }
    {
        // Two chunks per step when there is at most one block per CU (the
        // paired tiles fill most of a CU's LDS); otherwise one.  State tiles
        // are 32 x 64 (32 x dv for dv < 64): wider tiles re-read fewer operand
        // tiles but halve the number of independent sequential chains per CU,
        // which measured slower.
        const int ndir = dirs == 3 ? 2 : 1, dir0 = dirs == 2 ? 1 : 0;
        const int64_t tiles_k = BH * (P.DKP / TI);
        const int64_t wide = ndir * tiles_k * (P.DVP / (P.DVP < 64 ? P.DVP : 64));
        // With at most half a block per CU, 32-wide tiles: twice the
        // independent chains, each step half the work.
        const bool narrow = P.DVP >= 64 && 2 * wide <= kNumCUs;
        const bool pair = (narrow ? 2 * wide : wide) <= kNumCUs;
        const int kid = dirs == 1 ? KID_SCAN : dirs == 2 ? KID_SCANR : KID_SCAN2;
        auto run = [&](auto tj_c) {
            SSD_DISPATCH(P, ({
                constexpr int TJ = decltype(tj_c)::value ? 32 : (VP < 64 ? VP : 64);
                const int64_t per_dir = tiles_k * (VP / TJ);
                const dim3 grid((unsigned)(ndir * per_dir)), blk(NTS);
                if (pair)
                    launch(kid, k_state_scan<KP, VP, VE, TJ, 2, EXD>, grid, blk, st, q, k, v, dy, h0, P.bcum,
                           P.bl, P.states, P.dstates, dh0, (int)s.G, (int)s.H, s.T, (int)s.dk, (int)s.dv, P.L.NC,
                           P.L.NCp, P.L.Epad, per_dir, dir0);
                else
                    launch(kid, k_state_scan<KP, VP, VE, TJ, 1, EXD>, grid, blk, st, q, k, v, dy, h0, P.bcum,
                           P.bl, P.states, P.dstates, dh0, (int)s.G, (int)s.H, s.T, (int)s.dk, (int)s.dv, P.L.NC,
                           P.L.NCp, P.L.Epad, per_dir, dir0);
            }));
        };
        if (narrow) run(BoolC<true>{});
        else run(BoolC<false>{});
    }
    return launch_status();
}

static int prepare(const ssd_shape *shape, bool backward, void *ws, size_t ws_bytes, Problem *P)
{
    P->s = *shape;
    P->L = make_layout(shape, backward);
    if (ws_bytes < P->L.off[4]) return SSD_ERR_WORKSPACE;
    if (P->L.off[4] > 0) {
        if (!ws) return SSD_ERR_NULL;
        if (!aligned16(ws)) return SSD_ERR_ALIGN;
    }
    P->DKP = pad_dim(shape->dk);
    P->DVP = pad_dim(shape->dv);
    P->vec = (shape->dk % 4) == 0 && (shape->dv % 4) == 0;
    P->exact = shape->dk == P->DKP && shape->dv == P->DVP;
    char *w = static_cast<char *>(ws);
    P->bcum = reinterpret_cast<float *>(w + P->L.off[0]);
    P->bl = reinterpret_cast<float *>(w + P->L.off[1]);
    P->states = reinterpret_cast<float *>(w + P->L.off[2]);
    P->dstates = backward ? reinterpret_cast<float *>(w + P->L.off[3]) : nullptr;
    P->parts = backward && P->L.hsplit > 1 ? reinterpret_cast<float *>(w + P->L.part_off) : nullptr;
    return SSD_OK;
}

}  // namespace ssd

using namespace ssd;

extern "C" {

int ssd_fwd(const ssd_shape *shape, const float *q, const float *k, const float *v, const float *log_alpha,
            const float *h0, float *y, void *workspace, size_t workspace_bytes, void *stream)
{
    int rc = check_shape(shape);
    if (rc != SSD_OK) return rc;
    const ssd_shape &s = *shape;
    const bool empty = (s.B == 0 || s.T == 0);
    if (empty) return SSD_OK;   // y has no elements
    if (!q || !k || !v || !log_alpha || !h0 || !y) return SSD_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(log_alpha) || !aligned16(h0) ||
        !aligned16(y))
        return SSD_ERR_ALIGN;
    Problem P;
    rc = prepare(shape, false, workspace, workspace_bytes, &P);
    if (rc != SSD_OK) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);

    rc = run_scan(P, 1, true, q, k, v, nullptr, log_alpha, h0, nullptr, st);
    if (rc != SSD_OK) return rc;
    SSD_DISPATCH(P, launch(KID_OUTPUT, k_chunk_output<KP, VP, VE, EXD>,
                           dim3((unsigned)(s.B * s.G * P.L.hsplit * P.L.NC)), dim3(NTW), st, q, k, v, P.bcum,
                           P.states, y, (int)s.G, (int)s.H, s.T, (int)s.dk, (int)s.dv, P.L.NC, P.L.Epad, P.L.hpb));
    return launch_status();
}

}  // extern "C"

namespace ssd {
// Backward launches.  With `reuse`, the workspace already holds what ssd_fwd
// wrote for these inputs (the chunk cumsum, its totals and S_in of every
// chunk), so only the reverse state pass and the gradient kernel run.
static int bwd_impl(const ssd_shape *shape, const float *q, const float *k, const float *v,
                    const float *log_alpha, const float *h0, const float *dy, float *dq, float *dk, float *dv,
                    float *dlog_alpha, float *dh0, void *workspace, size_t workspace_bytes, void *stream, bool reuse)
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
        launch(-1, k_zero, dim3((unsigned)((n + NTH - 1) / NTH)), dim3(NTH), st, dh0, n);
        return launch_status();
    }
    if (!q || !k || !v || !log_alpha || !h0 || !dy || !dq || !dk || !dv || !dlog_alpha || !dh0)
        return SSD_ERR_NULL;
    const void *ptrs[] = {q, k, v, log_alpha, h0, dy, dq, dk, dv, dlog_alpha, dh0};
    for (const void *p : ptrs)
        if (!aligned16(p)) return SSD_ERR_ALIGN;
    Problem P;
    rc = prepare(shape, true, workspace, workspace_bytes, &P);
    if (rc != SSD_OK) return rc;

    // dS_out (reverse) of every chunk and dh0; without reuse also the cumsum
    // and S_in (forward), in the same launch.
    rc = run_scan(P, reuse ? 2 : 3, !reuse, q, k, v, dy, log_alpha, h0, dh0, st);
    if (rc != SSD_OK) return rc;
    // With a head split the gradient kernel writes each split's dq and dk
    // partial sums to the workspace, and k_sum_splits adds them up.
    const int hs = P.L.hsplit;
    const int64_t nqk = s.B * s.G * s.T * s.dk;
    float *pq = hs > 1 ? P.parts : dq, *pk = hs > 1 ? P.parts + hs * P.L.nqk_pad : dk;
    const int64_t pstride = hs > 1 ? P.L.nqk_pad : 0;
    SSD_DISPATCH(P, launch(KID_GRADS, k_bwd_grads<KP, VP, VE, EXD>, dim3((unsigned)(s.B * s.G * hs * P.L.NC)),
                           dim3(NTB), st, q, k, v, dy, P.bcum, P.bl, P.states, P.dstates, pq, pk, dv, dlog_alpha,
                           (int)s.G, (int)s.H, s.T, (int)s.dk, (int)s.dv, P.L.NC, P.L.NCp, P.L.Epad, P.L.hpb,
                           pstride));
    if (hs > 1) {
        if (launch_status() != SSD_OK) return SSD_ERR_DEVICE;
        const int64_t nb = (nqk + NTH - 1) / NTH;
        const dim3 grid((unsigned)(nb < 4096 ? nb : 4096));
        launch(-1, k_sum_splits, grid, dim3(NTH), st, dq, (const float *)pq, hs, pstride, nqk);
        launch(-1, k_sum_splits, grid, dim3(NTH), st, dk, (const float *)pk, hs, pstride, nqk);
    }
    return launch_status();
}
}  // namespace ssd

extern "C" {

int ssd_bwd(const ssd_shape *shape, const float *q, const float *k, const float *v, const float *log_alpha,
            const float *h0, const float *dy, float *dq, float *dk, float *dv, float *dlog_alpha, float *dh0,
            void *workspace, size_t workspace_bytes, void *stream)
{
    return bwd_impl(shape, q, k, v, log_alpha, h0, dy, dq, dk, dv, dlog_alpha, dh0, workspace, workspace_bytes,
                    stream, false);
}

int ssd_bwd_from_fwd(const ssd_shape *shape, const float *q, const float *k, const float *v,
                     const float *log_alpha, const float *h0, const float *dy, float *dq, float *dk, float *dv,
                     float *dlog_alpha, float *dh0, void *workspace, size_t workspace_bytes, void *stream)
{
    return bwd_impl(shape, q, k, v, log_alpha, h0, dy, dq, dk, dv, dlog_alpha, dh0, workspace, workspace_bytes,
                    stream, true);
}

int ssd_kernel_timing_enable(int mask)
{
    g_timing.mask = static_cast<unsigned>(mask);
    return SSD_OK;
}

int ssd_kernel_timing_reset(void)
{
    collect_timing();
    for (int i = 0; i < KID_COUNT; ++i) {
        g_timing.total[i] = 0.0;
        g_timing.count[i] = 0;
    }
    return SSD_OK;
}

int ssd_kernel_timing_read(int kid, double *total_ms, int64_t *count)
{
    if (kid < 0 || kid >= KID_COUNT) return SSD_ERR_SHAPE;
    if (!total_ms || !count) return SSD_ERR_NULL;
    collect_timing();
    *total_ms = g_timing.total[kid];
    *count = g_timing.count[kid];
    return SSD_OK;
}

int ssd_kernel_count(void) { return KID_COUNT; }

const char *ssd_kernel_name(int kid)
{
    if (kid < 0 || kid >= KID_COUNT) return "unknown";
    return kKernelNames[kid];
}

}  // extern "C"
