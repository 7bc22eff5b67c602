// Device-side helpers shared by the gfx950 kernels of the SSD scan: MFMA
// wrappers, DPP cross-lane sums and scans, buffer-resource loads and stores,
// register/LDS tile movement and the pinned block barrier.
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
// All contractions run on fp32 MFMA (fp32 in, fp32 accumulate).  For
// v_mfma_f32_32x32x2f32, lane l supplies A[l%32][l/32] and B[l/32][l%32] of a
// 32x2 by 2x32 product, and accumulator register r of lane l holds row
// 8*(r/4) + 4*(l/32) + r%4, column l%32 of the 32x32 result.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

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

// The within-chunk inclusive cumulative log-decay b of the chunk whose 64
// log_alpha values the wave holds, one per lane (positions past the sequence
// end hold 0, so they repeat the last valid b and lane 63 holds the chunk
// total b_L).  Every kernel forms b with this one scan, so all of them see
// bitwise the same b.  Needs all 64 lanes active.
__device__ __forceinline__ float chunk_cumsum(float la) { return scan64(la); }

// ---------------------------------------------------------------------------
// Helpers for the 8-wave kernels.

constexpr int NTW = 512;   // 8 waves per block

template <bool B>
struct BoolC {
    static constexpr bool value = B;
};
template <int N>
struct IntC {
    static constexpr int value = N;
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
// Store that is not read again by this kernel: non-temporal at device scope
// (cache policy nt + sc1), so it does not displace reusable lines from L2.
// Measured against nt alone on the fwd + bwd step: 922 against 930 us (the
// state scans' chunk states, y and dv go out this way).
constexpr int kStoreNT = 2 | 16;
__device__ __forceinline__ void gstore1_nt(rsrc_t r, uint32_t off, float x)
{
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(x), r, off, 0, kStoreNT);
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
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, make_float2(x[0], x[1])), r, off, 0,
                                              kStoreNT);
    } else {
        static_assert(N == 4, "1, 2 or 4 floats");
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, make_float4(x[0], x[1], x[2], x[3])), r, off,
                                               0, kStoreNT);
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

}  // namespace ssd
