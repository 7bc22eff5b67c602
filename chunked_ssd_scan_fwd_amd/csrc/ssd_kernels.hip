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

#include <stdint.h>
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

// Sum over the 32 lanes that share lane/32 (fixed butterfly order).
__device__ __forceinline__ float sum32(float x)
{
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 8);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 1);
    return x;
}

__device__ __forceinline__ float sum64(float x)
{
    x += __shfl_xor(x, 32);
    return sum32(x);
}

__device__ __forceinline__ float readlane_f(float x, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Copy rows [0, rows) x cols [0, d) of a row-major global tile with row
// stride d into LDS dst[CH][LD]; columns d..DP-1 and rows >= rows become 0.
// Each row is optionally scaled by w[row] (LDS).
template <int DP, int LD, bool SCALE, int NT = NTH>
__device__ __forceinline__ void stage_rows(float *dst, const float *__restrict__ src, int rows, int d,
                                           bool vec, const float *w)
{
    if (vec) {
        constexpr int Q4 = DP / 4;
        for (int idx = threadIdx.x; idx < CH * Q4; idx += NT) {
            const int t = idx / Q4, c4 = (idx - t * Q4) * 4;
            float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
            if (t < rows && c4 < d) val = *reinterpret_cast<const float4 *>(src + (size_t)t * d + c4);
            if (SCALE) {
                const float s = w[t];
                val.x *= s;
                val.y *= s;
                val.z *= s;
                val.w *= s;
            }
            float *p = dst + t * LD + c4;
            p[0] = val.x;
            p[1] = val.y;
            p[2] = val.z;
            p[3] = val.w;
        }
    } else {
        for (int idx = threadIdx.x; idx < CH * DP; idx += NT) {
            const int t = idx / DP, cc = idx - t * DP;
            float val = (t < rows && cc < d) ? src[(size_t)t * d + cc] : 0.f;
            if (SCALE) val *= w[t];
            dst[t * LD + cc] = val;
        }
    }
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

__device__ __forceinline__ float4 zero4() { return make_float4(0.f, 0.f, 0.f, 0.f); }

// row[c4 .. c4+3] of the row starting at base + rowoff, which has `lim`
// valid entries (the rest read as 0).  `base` is uniform across the wave and
// the per-lane offset is 32-bit, so the load addresses from a scalar base.
// vec: one aligned 16-byte load (requires lim % 4 == 0 and an aligned row).
__device__ __forceinline__ float4 load4(const float *__restrict__ base, uint32_t rowoff, int c4, int lim, bool vec)
{
    const float *p = base + (rowoff + (uint32_t)c4);
    if (vec) return (c4 < lim) ? *reinterpret_cast<const float4 *>(p) : zero4();
    float4 r;
    r.x = (c4 + 0 < lim) ? p[0] : 0.f;
    r.y = (c4 + 1 < lim) ? p[1] : 0.f;
    r.z = (c4 + 2 < lim) ? p[2] : 0.f;
    r.w = (c4 + 3 < lim) ? p[3] : 0.f;
    return r;
}

// Load a ROWS x DP tile (row-major, row stride d, `nrows` valid rows, d valid
// columns) into registers, PER float4 per thread, zero padded.
template <int ROWS, int DP, int NT, int PER>
__device__ __forceinline__ void tile_to_regs(int tid, float4 (&buf)[PER], const float *__restrict__ src, int nrows,
                                             int d, bool vec)
{
    constexpr int Q4 = DP / 4;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int idx = tid + u * NT;
        const int r = idx / Q4, c4 = (idx - r * Q4) * 4;
        buf[u] = (idx < ROWS * Q4 && r < nrows) ? load4(src, (uint32_t)(r * d), c4, d, vec) : zero4();
    }
}

// Store a register tile (see tile_to_regs) into LDS dst[ROWS][LD].
template <int ROWS, int DP, int NT, int PER, int LD>
__device__ __forceinline__ void regs_to_lds(int tid, const float4 (&buf)[PER], float *dst)
{
    constexpr int Q4 = DP / 4;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int idx = tid + u * NT;
        if (idx < ROWS * Q4) {
            const int r = idx / Q4, c4 = (idx - r * Q4) * 4;
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

// Q K^T tiles of a chunk (causal 32x32 tiles (0,0), (1,0), (1,1)), the dk
// contraction split over six waves: waves 0-2 end up holding the full tile
// (w % 3), the partial sums of waves 3-5 pass through `scratch` (3 x 1024).
template <int DKP, int LDQ, int LDK>
__device__ __forceinline__ f32x16 qk_tiles(const float *Qs, const float *Ks, float *scratch, int wave, int lane)
{
    const int cl = lane & 31, kh = lane >> 5;
    const int tile = wave % 3, half = wave / 3;
    const int ib = (tile == 0) ? 0 : 1, jb = (tile == 2) ? 1 : 0;
    f32x16 acc = zero16();
    if (wave < 6) {
        const int k0 = half * (DKP / 2);
#pragma unroll 8
        for (int kk = k0; kk < k0 + DKP / 2; kk += 2)
            acc = mfma32(Qs[(ib * 32 + cl) * LDQ + kk + kh], Ks[(jb * 32 + cl) * LDK + kk + kh], acc);
        if (wave >= 3) {
#pragma unroll
            for (int r = 0; r < 16; ++r) scratch[tile * 1024 + r * 64 + lane] = acc[r];
        }
    }
    __syncthreads();
    if (wave < 3) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] += scratch[tile * 1024 + r * 64 + lane];
    }
    __syncthreads();
    return acc;
}

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
// One block of 4 waves owns a 32 x TJ tile of one head's dk x dv state; the
// next chunk's operand tiles are prefetched into registers while the current
// chunk's MFMAs run, then written to the other half of a double-buffered LDS
// tile.  Blocks of one (b, g) are placed on one XCD so that the group's q/k
// and each head's v/dy tiles are shared through that XCD's L2.
constexpr int TI = 32;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int DKP, int DVP>
__global__ __launch_bounds__(NTH) void k_state_scan(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ dy, const float *__restrict__ h0, const float *__restrict__ bcum,
    const float *__restrict__ bl, float *__restrict__ states, float *__restrict__ dstates,
    float *__restrict__ dh0, int G, int H, int64_t T, int dk, int dv, int64_t NC, int64_t NCp, int64_t Epad,
    int64_t per_dir, int vecK, int vecV)
{
    constexpr int TJ = DVP < 64 ? DVP : 64;
    constexpr int NTJ = DVP / TJ;
    constexpr int NTILE = (DKP / TI) * NTJ;
    constexpr int LDA = TI + 16, LDB = TJ + 16;
    constexpr int A4 = CH * TI / 4, B4 = CH * TJ / 4;
    constexpr int APER = (A4 + NTH - 1) / NTH, BPER = (B4 + NTH - 1) / NTH;
    constexpr int NB16 = (2 * (TJ / 16)) / 4;   // 16x16 accumulator tiles per wave
    __shared__ __attribute__((aligned(16))) float As[2][CH * LDA];
    __shared__ __attribute__((aligned(16))) float Bs[2][CH * LDB];

    // XCD-aware order: consecutive logical blocks share blockIdx % 8.
    const int64_t nblk = gridDim.x;
    int64_t L = blockIdx.x;
    if ((nblk & 7) == 0) L = (int64_t)(blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
    const int dir = (int)(L / per_dir);
    const int64_t rem = L - dir * per_dir;
    const int64_t bh = rem / NTILE;
    const int tile = (int)(rem - bh * NTILE);
    const int i0 = (tile / NTJ) * TI, j0 = (tile % NTJ) * TJ;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const int g = h / (H / G);
    const float *Asrc = (dir == 0 ? k : q) + (b * G + g) * T * dk + i0;
    const float *Bsrc = (dir == 0 ? v : dy) + bh * T * dv + j0;
    float *slab = (dir == 0 ? states : dstates) + bh * NC * Epad;
    const float *bcb = bcum + bh * NC * CH;
    const int lima = dk - i0, limb = dv - j0;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int rblk = wave & 1;                 // 16-row block of the tile
    const int cblk0 = (wave >> 1) * NB16;      // first 16-column block

    // operand prefetch for one chunk
    float4 abuf[APER], bbuf[BPER];
    float bt[BPER], blc = 0.f;
    auto prefetch = [&](int64_t c) {
        const int rows = (int)((T - c * CH) < CH ? (T - c * CH) : CH);
#pragma unroll
        for (int u = 0; u < APER; ++u) {
            const int idx = threadIdx.x + u * NTH;
            const int r = idx / (TI / 4), c4 = (idx - r * (TI / 4)) * 4;
            abuf[u] = (idx < A4 && r < rows) ? load4(Asrc + c * CH * dk, (uint32_t)(r * dk), c4, lima, vecK != 0) : zero4();
        }
#pragma unroll
        for (int u = 0; u < BPER; ++u) {
            const int idx = threadIdx.x + u * NTH;
            const int r = idx / (TJ / 4), c4 = (idx - r * (TJ / 4)) * 4;
            bbuf[u] = (idx < B4 && r < rows) ? load4(Bsrc + c * CH * dv, (uint32_t)(r * dv), c4, limb, vecV != 0) : zero4();
            bt[u] = (idx < B4) ? bcb[c * CH + r] : 0.f;
        }
        blc = bl[bh * NCp + c];
    };

    f32x4 acc[NB16];
#pragma unroll
    for (int u = 0; u < NB16; ++u) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = i0 + rblk * 16 + 4 * q4 + r, col = j0 + (cblk0 + u) * 16 + l16;
            acc[u][r] = (dir == 0 && row < dk && col < dv) ? h0[bh * (int64_t)dk * dv + (int64_t)row * dv + col] : 0.f;
        }
    }

    prefetch(dir == 0 ? 0 : NC - 1);
    for (int64_t s = 0; s < NC; ++s) {
        const int64_t c = (dir == 0) ? s : NC - 1 - s;
        const int buf = (int)(s & 1);
        // stage this chunk's operands; scale B rows by the decay weights
#pragma unroll
        for (int u = 0; u < APER; ++u) {
            const int idx = threadIdx.x + u * NTH;
            if (idx < A4) {
                const int r = idx / (TI / 4), c4 = (idx - r * (TI / 4)) * 4;
                *reinterpret_cast<float4 *>(&As[buf][r * LDA + c4]) = abuf[u];
            }
        }
#pragma unroll
        for (int u = 0; u < BPER; ++u) {
            const int idx = threadIdx.x + u * NTH;
            if (idx < B4) {
                const int r = idx / (TJ / 4), c4 = (idx - r * (TJ / 4)) * 4;
                const float w = (dir == 0) ? expf(blc - bt[u]) : expf(bt[u]);
                float4 x = bbuf[u];
                x.x *= w;
                x.y *= w;
                x.z *= w;
                x.w *= w;
                *reinterpret_cast<float4 *>(&Bs[buf][r * LDB + c4]) = x;
            }
        }
        const float decay = expf(blc);
        if (s + 1 < NC) prefetch(dir == 0 ? c + 1 : c - 1);
        __syncthreads();

        // slab[c] = S (state entering the chunk in this direction)
        float *dst = slab + c * Epad;
#pragma unroll
        for (int u = 0; u < NB16; ++u) {
            const int col = j0 + (cblk0 + u) * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = i0 + rblk * 16 + 4 * q4 + r;
                if (row < dk && col < dv) dst[row * dv + col] = acc[u][r];
                acc[u][r] *= decay;
            }
        }
        // S += A^T B over the chunk's 64 positions
        const float *Ab = &As[buf][q4 * LDA + rblk * 16 + l16];
        const float *Bb = &Bs[buf][q4 * LDB + cblk0 * 16 + l16];
#pragma unroll 4
        for (int kk = 0; kk < CH; kk += 4) {
            const float a = Ab[kk * LDA];
#pragma unroll
            for (int u = 0; u < NB16; ++u) acc[u] = mfma16(a, Bb[kk * LDB + u * 16], acc[u]);
        }
    }
    if (dir == 1) {
#pragma unroll
        for (int u = 0; u < NB16; ++u) {
            const int col = j0 + (cblk0 + u) * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = i0 + rblk * 16 + 4 * q4 + r;
                if (row < dk && col < dv) dh0[bh * (int64_t)dk * dv + (int64_t)row * dv + col] = acc[u][r];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// K2 + K5: output of one chunk for every head of one group.
// One block of 8 waves per (b,g,chunk).  Q K^T (causal 32x32 tiles) is
// formed once and kept in registers.  Per head: the next head's V tile and
// incoming state S_in are prefetched into registers while this head runs;
// P = (Q K^T) o D goes to LDS; then each wave computes one 32x32 tile of
// Y = P V + diag(e^b) (Q S_in) with every operand read from LDS.  For dv < 128
// the Q S_in contraction is split over the spare waves and summed in a fixed
// order.
template <int DKP, int DVP>
__global__ __launch_bounds__(NTW) void k_chunk_output(const float *__restrict__ q, const float *__restrict__ k,
                                                      const float *__restrict__ v, const float *__restrict__ bcum,
                                                      const float *__restrict__ states, float *__restrict__ y,
                                                      int G, int H, int64_t T, int dk, int dv, int64_t NC,
                                                      int64_t Epad, int vecK, int vecV)
{
    constexpr int LDQ = DKP + 1;
    constexpr int LDKV = (DKP > DVP ? DKP : DVP) + 1;
    constexpr int LDP = CH + 1;
    constexpr int NCB = DVP / 32, NOB = 2 * NCB, KS = 8 / NOB;
    constexpr int VPER = (CH * DVP / 4 + NTW - 1) / NTW;
    constexpr int SPER = (DKP * DVP / 4 + NTW - 1) / NTW;
    __shared__ float Qs[CH * LDQ];
    __shared__ float KVs[CH * LDKV];
    __shared__ __attribute__((aligned(16))) float Ss[DKP * DVP];
    __shared__ float Ps[CH * LDP];
    __shared__ float Red[KS > 1 ? (KS - 1) * NOB * 1024 : 1];
    __shared__ float bs[CH], eb[CH];

    const int64_t c = blockIdx.x % NC;
    const int64_t bg = blockIdx.x / NC;
    const int g = (int)(bg % G);
    const int64_t b = bg / G;
    const int hpg = H / G;
    const int64_t bh0 = b * H + (int64_t)g * hpg;
    const int rows = (int)((T - c * CH) < CH ? (T - c * CH) : CH);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cl = lane & 31, kh = lane >> 5;

    float4 vbuf[VPER], sbuf[SPER];
    float bpre = 0.f;
    auto prefetch = [&](int hh) {
        const int64_t bh = bh0 + hh;
        tile_to_regs<CH, DVP, NTW, VPER>(threadIdx.x, vbuf, v + (bh * T + c * CH) * dv, rows, dv, vecV != 0);
        tile_to_regs<DKP, DVP, NTW, SPER>(threadIdx.x, sbuf, states + (bh * NC + c) * Epad, dk, dv, vecV != 0);
        if (threadIdx.x < CH) bpre = bcum[bh * NC * CH + c * CH + threadIdx.x];
    };
    prefetch(0);

    stage_rows<DKP, LDQ, false, NTW>(Qs, q + (bg * T + c * CH) * dk, rows, dk, vecK != 0, nullptr);
    stage_rows<DKP, LDKV, false, NTW>(KVs, k + (bg * T + c * CH) * dk, rows, dk, vecK != 0, nullptr);
    __syncthreads();
    const f32x16 accA = qk_tiles<DKP, LDQ, LDKV>(Qs, KVs, Ps, wave, lane);
    const int ib = (wave == 0) ? 0 : 1, jb = (wave == 2) ? 1 : 0;

    const int ob = wave % NOB, ks = wave / NOB;
    const int rb = ob / NCB, cb = ob % NCB;
    const int n = cb * 32 + cl;
    for (int hh = 0; hh < hpg; ++hh) {
        const int64_t bh = bh0 + hh;
        regs_to_lds<CH, DVP, NTW, VPER, LDKV>(threadIdx.x, vbuf, KVs);
        regs_to_lds<DKP, DVP, NTW, SPER, DVP>(threadIdx.x, sbuf, Ss);
        if (threadIdx.x < CH) {
            bs[threadIdx.x] = bpre;
            eb[threadIdx.x] = expf(bpre);
        }
        if (hh + 1 < hpg) prefetch(hh + 1);
        __syncthreads();
        if (wave < 3) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = ib * 32 + acc_row(r, lane), j = jb * 32 + cl;
                Ps[i * LDP + j] = (j <= i) ? accA[r] * expf(bs[i] - bs[j]) : 0.f;
            }
        }
        __syncthreads();

        f32x16 ay = zero16(), ai = zero16();
        if (ks == 0) {
            const int kend = (rb + 1) * 32;
            for (int kk = 0; kk < kend; kk += 2)
                ay = mfma32(Ps[(rb * 32 + cl) * LDP + kk + kh], KVs[(kk + kh) * LDKV + n], ay);
        }
        {
            constexpr int KL = DKP / KS;
            const int i0 = ks * KL;
#pragma unroll 8
            for (int i = i0; i < i0 + KL; i += 2)
                ai = mfma32(Qs[(rb * 32 + cl) * LDQ + i + kh], Ss[(i + kh) * DVP + n], ai);
        }
        if (KS > 1) {
            if (ks > 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r) Red[((ks - 1) * NOB + ob) * 1024 + r * 64 + lane] = ai[r];
            }
            __syncthreads();
            if (ks == 0) {
                for (int kk2 = 1; kk2 < KS; ++kk2) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) ai[r] += Red[((kk2 - 1) * NOB + ob) * 1024 + r * 64 + lane];
                }
            }
        }
        if (ks == 0 && n < dv) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = rb * 32 + acc_row(r, lane);
                if (row < rows) y[(bh * T + c * CH + row) * dv + n] = ay[r] + eb[row] * ai[r];
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// B3 + B4: gradients of one chunk for every head of one group.
//
// One block of 8 waves per (b, g, chunk).  The group's heads are taken in
// ascending order; dq and dk are summed over them in registers.  Per head:
//
//   state phase  S_in and dS_out are streamed through LDS in slabs of 32
//                state columns (all dk rows of both).  With the slab's 32
//                columns n of dY and V:
//                    Gq += dY[:, n] S_in[:, n]^T      (C x dk, 32x32 tiles)
//                    Gk += V[:, n] dS_out[:, n]^T     (C x dk, 32x32 tiles)
//                    Gv[:, n] = K dS_out[:, n]        (C x 32, 16x16 tiles)
//                and every thread adds the products of the state elements
//                it staged to <dS_out, S_in>.
//   intra phase  dP = (dY V^T) o D and P = (Q K^T) o D, then
//                    dQ += diag(e^b) Gq + dP K
//                    dK += diag(e^{b_L - b}) Gk + dP^T Q
//                    dV  = diag(e^{b_L - b}) Gv + P^T dY
//                and dlog_alpha for the chunk's positions.
//
// Every MFMA operand is read from LDS.  The LDS regions are Q / slabs (the
// two share memory in time; Q is staged again for every head), K, dY,
// V / ((dY V^T) partial sums + P) and dP / M.  The next head's V, dY and
// first slab, and each next slab, are loaded into registers while the
// current ones are in use.  Row strides keep the 16-byte row reads and the
// column reads free of LDS bank conflicts.
template <int DKP, int DVP>
struct BwdCfg {
    static constexpr int LDK = DKP + 4;   // Q, K
    static constexpr int LDV = DVP + 4;   // dY, V
    static constexpr int LDP = CH + 4;    // dP, M, P
    static constexpr int LSL = 36;        // slab rows: 32 state columns + 4
    static constexpr int NKB = DKP / 32;  // 32-column blocks of dk
    static constexpr int NTK = 2 * NKB;   // 32x32 tiles of a C x dk result
    static constexpr int NSL = DVP / 32;  // slabs per state
    static constexpr int SCR = 3 * 1024;  // (dY V^T) partial sums, start of the V region
    static constexpr int QN = (CH * LDK > 2 * DKP * LSL) ? CH * LDK : 2 * DKP * LSL;
    static constexpr int VN = (CH * LDV > SCR + CH * LDP) ? CH * LDV : SCR + CH * LDP;
    static constexpr int PN = (CH * LDP > SCR) ? CH * LDP : SCR;
    static constexpr int TPER = (CH * DVP / 4 + NTW - 1) / NTW;   // float4 / thread, C x dv tile
    static constexpr int QPER = (CH * DKP / 4 + NTW - 1) / NTW;   // float4 / thread, C x dk tile
    static constexpr int SPER = (DKP * 8 + NTW - 1) / NTW;        // float4 / thread, one state slab
};

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

template <int DKP, int DVP>
__global__ __launch_bounds__(NTW) void k_bwd_grads(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ dy, const float *__restrict__ bcum, const float *__restrict__ bl,
    const float *__restrict__ states, const float *__restrict__ dstates, float *__restrict__ dq,
    float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ dla, int G, int H, int64_t T, int dk_,
    int dv_, int64_t NC, int64_t NCp, int64_t Epad, int vecK, int vecV)
{
    using Cfg = BwdCfg<DKP, DVP>;
    constexpr int LDK = Cfg::LDK, LDV = Cfg::LDV, LDP = Cfg::LDP, LSL = Cfg::LSL;
    constexpr int NKB = Cfg::NKB, NTK = Cfg::NTK, NSL = Cfg::NSL, SCR = Cfg::SCR;
    constexpr int TPER = Cfg::TPER, QPER = Cfg::QPER, SPER = Cfg::SPER;
    __shared__ __attribute__((aligned(16))) float RQ[Cfg::QN];
    __shared__ __attribute__((aligned(16))) float RK[CH * LDK];
    __shared__ __attribute__((aligned(16))) float RY[CH * LDV];
    __shared__ __attribute__((aligned(16))) float RV[Cfg::VN];
    __shared__ __attribute__((aligned(16))) float RP[Cfg::PN];
    __shared__ float bs[CH], eb[CH], el[CH];
    __shared__ float redQ[NKB][CH], redK[NKB][CH];
    __shared__ float redR[NTW / 64][CH];
    __shared__ float redB[NTW / 64];
    float *const slS = RQ;               // S_in slab   [DKP][LSL]
    float *const slD = RQ + DKP * LSL;   // dS_out slab [DKP][LSL]
    float *const Pm = RV + SCR;          // P           [CH][LDP]

    const int64_t c = blockIdx.x % NC;
    const int64_t bg = blockIdx.x / NC;
    const int g = (int)(bg % G);
    const int64_t b = bg / G;
    const int hpg = H / G;
    const int64_t bh0 = b * H + (int64_t)g * hpg;
    const int rows = (int)((T - c * CH) < CH ? (T - c * CH) : CH);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cl = lane & 31;
    const int l16 = lane & 15, lq = lane >> 4;
    const bool vk = vecK != 0, vv = vecV != 0;
    const float *qsrc = q + (bg * T + c * CH) * dk_;

    float4 vbuf[TPER], ybuf[TPER];   // a head's V and dY
    float4 sbuf[SPER], dbuf[SPER];   // a slab of S_in and of dS_out
    float4 qbuf[QPER];               // Q
    float bpre = 0.f, blpre = 0.f;   // a head's b (thread t < 64: position t) and b_L

    auto load_vy = [&](int hh, int tid) {
        const int64_t bh = bh0 + hh;
        tile_to_regs<CH, DVP, NTW, TPER>(tid, vbuf, v + (bh * T + c * CH) * dv_, rows, dv_, vv);
        tile_to_regs<CH, DVP, NTW, TPER>(tid, ybuf, dy + (bh * T + c * CH) * dv_, rows, dv_, vv);
        if (tid < CH) {
            bpre = bcum[bh * NC * CH + c * CH + tid];
            blpre = bl[bh * NCp + c];
        }
    };
    auto load_slab = [&](int hh, int m, int tid) {
        const int64_t off = ((bh0 + hh) * NC + c) * Epad + 32 * m;
        const int lim = dv_ - 32 * m;
#pragma unroll
        for (int u = 0; u < SPER; ++u) {
            const int idx = tid + u * NTW;
            const int r = idx >> 3, c4 = (idx & 7) * 4;
            const bool ok = idx < DKP * 8 && r < dk_;
            sbuf[u] = ok ? load4(states + off, (uint32_t)(r * dv_), c4, lim, vv) : zero4();
            dbuf[u] = ok ? load4(dstates + off, (uint32_t)(r * dv_), c4, lim, vv) : zero4();
        }
    };
    // Write the staged slab to LDS; returns this thread's part of <dS_out, S_in>.
    auto store_slab = [&](int tid) -> float {
        float f = 0.f;
#pragma unroll
        for (int u = 0; u < SPER; ++u) {
            const int idx = tid + u * NTW;
            if (idx < DKP * 8) {
                const int r = idx >> 3, c4 = (idx & 7) * 4;
                *reinterpret_cast<float4 *>(slS + r * LSL + c4) = sbuf[u];
                *reinterpret_cast<float4 *>(slD + r * LSL + c4) = dbuf[u];
                f += sbuf[u].x * dbuf[u].x + sbuf[u].y * dbuf[u].y + sbuf[u].z * dbuf[u].z +
                     sbuf[u].w * dbuf[u].w;
            }
        }
        return f;
    };

    // ---- block set-up: K, Q, A = Q K^T, the first head's V, dY and slab.
    load_vy(0, tid);
    tile_to_regs<CH, DKP, NTW, QPER>(tid, qbuf, qsrc, rows, dk_, vk);
    regs_to_lds<CH, DKP, NTW, QPER, LDK>(tid, qbuf, RQ);
    tile_to_regs<CH, DKP, NTW, QPER>(tid, qbuf, k + (bg * T + c * CH) * dk_, rows, dk_, vk);
    regs_to_lds<CH, DKP, NTW, QPER, LDK>(tid, qbuf, RK);
    load_slab(0, 0, tid);
    __syncthreads();
    // causal 32x32 tiles (0,0), (1,0), (1,1) of Q K^T; waves w and w + 3 split dk
    const int at = wave % 3, ah = wave / 3;
    const int aib = (at == 0) ? 0 : 1, ajb = (at == 2) ? 1 : 0;
    f32x16 accA = zero16();
    if (wave < 6)
        mma_abt<LDK, LDK>(accA, RQ + aib * 32 * LDK, RK + ajb * 32 * LDK, ah * (DKP / 2), (ah + 1) * (DKP / 2),
                          lane);
    if (wave >= 3 && wave < 6) {
#pragma unroll
        for (int r = 0; r < 16; ++r) RP[at * 1024 + r * 64 + lane] = accA[r];
    }
    __syncthreads();
    if (wave < 3) {
#pragma unroll
        for (int r = 0; r < 16; ++r) accA[r] += RP[at * 1024 + r * 64 + lane];
    }
    regs_to_lds<CH, DVP, NTW, TPER, LDV>(tid, vbuf, RV);
    regs_to_lds<CH, DVP, NTW, TPER, LDV>(tid, ybuf, RY);
    float fro_next = store_slab(tid);
    __syncthreads();

    const int rbk = wave / NKB, cbk = wave % NKB;   // this wave's dq / dk tile (waves < NTK)
    const bool hasK = wave < NTK;
    f32x16 dQacc = zero16(), dKacc = zero16();

    for (int hh = 0; hh < hpg; ++hh) {
        // Per-lane index arithmetic is redone inside the loop (the asm hides
        // that tid is loop-invariant): hoisting it would exceed the register
        // budget.
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, cl = lane & 31, l16 = lane & 15, lq = lane >> 4;
        const int64_t bh = bh0 + hh;
        const float bcur = bpre, blh = blpre;
        float fro = fro_next;

        // ---- state phase
        f32x16 gq = zero16(), gk = zero16();
        f32x4 gv[NSL];
#pragma unroll
        for (int m = 0; m < NSL; ++m) {
            if (m > 0) {
                __syncthreads();   // slab m - 1 fully read
                fro += store_slab(tid);
            }
            if (m + 1 < NSL)
                load_slab(hh, m + 1, tid);
            else
                tile_to_regs<CH, DKP, NTW, QPER>(tid, qbuf, qsrc, rows, dk_, vk);
            if (m > 0) __syncthreads();
            if (hasK) {
                mma_abt<LDV, LSL>(gq, RY + rbk * 32 * LDV + 32 * m, slS + cbk * 32 * LSL, 0, 32, lane);
                mma_abt<LDV, LSL>(gk, RV + rbk * 32 * LDV + 32 * m, slD + cbk * 32 * LSL, 0, 32, lane);
            }
            // Gv tile: positions 16 rt .. 16 rt + 15, state columns 32 m + 16 ct .. + 15
            const int rt = ((wave >> 1) + m) & 3, ct = wave & 1;
            const float *ak = RK + (16 * rt + l16) * LDK + 4 * lq;
            const float *bd = slD + 4 * lq * LSL + 16 * ct + l16;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
            for (int i0 = 0; i0 < DKP; i0 += 16) {
                const float4 a = *reinterpret_cast<const float4 *>(ak + i0);
                acc = mfma16(a.x, bd[(i0 + 0) * LSL], acc);
                acc = mfma16(a.y, bd[(i0 + 1) * LSL], acc);
                acc = mfma16(a.z, bd[(i0 + 2) * LSL], acc);
                acc = mfma16(a.w, bd[(i0 + 3) * LSL], acc);
            }
            gv[m] = acc;
        }

        // ---- intra phase
        __syncthreads();   // slab reads done
        regs_to_lds<CH, DKP, NTW, QPER, LDK>(tid, qbuf, RQ);
        if (tid < CH) {
            bs[tid] = bcur;
            eb[tid] = expf(bcur);
            el[tid] = (tid < rows) ? expf(blh - bcur) : 0.f;
        }
        if (hh + 1 < hpg) {
            load_vy(hh + 1, tid);
            load_slab(hh + 1, 0, tid);
        }
        __syncthreads();

        // state parts of dQ and dK, and their rows' dlog_alpha terms
        if (hasK) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = rbk * 32 + acc_row(r, lane);
                gq[r] *= eb[row];
                gk[r] *= el[row];
                const float sq = sum32(gq[r] * RQ[row * LDK + cbk * 32 + cl]);
                const float sk = sum32(gk[r] * RK[row * LDK + cbk * 32 + cl]);
                if (cl == 0) {
                    redQ[cbk][row] = sq;
                    redK[cbk][row] = sk;
                }
            }
            dQacc += gq;
            dKacc += gk;
        }
#pragma unroll
        for (int m = 0; m < NSL; ++m) {
            const int rt = ((wave >> 1) + m) & 3;
#pragma unroll
            for (int r = 0; r < 4; ++r) gv[m][r] *= el[16 * rt + 4 * lq + r];
        }
        // dY V^T, causal tiles; waves w and w + 3 split dv
        f32x16 aD = zero16();
        if (wave < 6)
            mma_abt<LDV, LDV>(aD, RY + aib * 32 * LDV, RV + ajb * 32 * LDV, ah * (DVP / 2), (ah + 1) * (DVP / 2),
                              lane);
        __syncthreads();   // V reads done
        if (wave >= 3 && wave < 6) {
#pragma unroll
            for (int r = 0; r < 16; ++r) RV[at * 1024 + r * 64 + lane] = aD[r];
        }
        __syncthreads();
        f32x16 pM = zero16();
        if (wave < 3) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = aib * 32 + acc_row(r, lane), j = ajb * 32 + cl;
                const float a = aD[r] + RV[at * 1024 + r * 64 + lane];
                const float D = (j <= i) ? expf(bs[i] - bs[j]) : 0.f;
                const float p = accA[r] * D;
                RP[i * LDP + j] = a * D;   // dP
                Pm[i * LDP + j] = p;       // P
                pM[r] = p * a;             // M
            }
        }
        __syncthreads();

        if (hasK) {
            // dQ += dP K over j <= i
            {
                const float *a = RP + (rbk * 32 + cl) * LDP + 4 * (lane >> 5);
                const float *bk = RK + 4 * (lane >> 5) * LDK + cbk * 32 + cl;
                const int jend = (rbk + 1) * 32;
                for (int j0 = 0; j0 < jend; j0 += 8) {
                    const float4 x = *reinterpret_cast<const float4 *>(a + j0);
                    dQacc = mfma32(x.x, bk[(j0 + 0) * LDK], dQacc);
                    dQacc = mfma32(x.y, bk[(j0 + 1) * LDK], dQacc);
                    dQacc = mfma32(x.z, bk[(j0 + 2) * LDK], dQacc);
                    dQacc = mfma32(x.w, bk[(j0 + 3) * LDK], dQacc);
                }
            }
            // dK += dP^T Q over j >= i
            {
                const float *a = RP + 4 * (lane >> 5) * LDP + rbk * 32 + cl;
                const float *bq = RQ + 4 * (lane >> 5) * LDK + cbk * 32 + cl;
                for (int j0 = rbk * 32; j0 < CH; j0 += 8) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) dKacc = mfma32(a[(j0 + s) * LDP], bq[(j0 + s) * LDK], dKacc);
                }
            }
        }
        // dV = Gv + P^T dY over j >= t, written per 16x16 tile
        float *dvb = dv + (bh * T + c * CH) * dv_;
#pragma unroll
        for (int m = 0; m < NSL; ++m) {
            const int rt = ((wave >> 1) + m) & 3, ct = wave & 1;
            f32x4 acc = gv[m];
            const float *a = Pm + 4 * lq * LDP + 16 * rt + l16;
            const float *by = RY + 4 * lq * LDV + 32 * m + 16 * ct + l16;
            for (int j0 = 16 * rt; j0 < CH; j0 += 16) {
#pragma unroll
                for (int s = 0; s < 4; ++s) acc = mfma16(a[(j0 + s) * LDP], by[(j0 + s) * LDV], acc);
            }
            const int n = 32 * m + 16 * ct + l16;
            if (n < dv_) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * rt + 4 * lq + r;
                    if (t < rows) dvb[(uint32_t)(t * dv_ + n)] = acc[r];
                }
            }
        }
        __syncthreads();   // dP, P, Q and dY reads done

        // M to LDS (its upper-right tile is zero); the next head's V, dY, first slab
        if (wave < 3) {
#pragma unroll
            for (int r = 0; r < 16; ++r) RP[(aib * 32 + acc_row(r, lane)) * LDP + ajb * 32 + cl] = pM[r];
        } else if (wave == 3) {
#pragma unroll
            for (int r = 0; r < 16; ++r) RP[acc_row(r, lane) * LDP + 32 + cl] = 0.f;
        }
        if (hh + 1 < hpg) {
            regs_to_lds<CH, DVP, NTW, TPER, LDV>(tid, vbuf, RV);
            regs_to_lds<CH, DVP, NTW, TPER, LDV>(tid, ybuf, RY);
            fro_next = store_slab(tid);
        }
        __syncthreads();

        // Rectangle sums R_r = sum_{i >= r} sum_{j < r} M_ij: exclusive prefix
        // over j of every row (in place), then a suffix over i.
        for (int i = wave * 8; i < wave * 8 + 8; ++i) {
            float x = RP[i * LDP + lane];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float yv = __shfl_up(x, off);
                if (lane >= off) x += yv;
            }
            // shift, not subtract: the diagonal term must not enter the prefix
            float xe = __shfl_up(x, 1);
            if (lane == 0) xe = 0.f;
            RP[i * LDP + lane] = xe;
        }
        __syncthreads();
        {
            float racc = 0.f;
            for (int i = wave * 8; i < wave * 8 + 8; ++i)
                if (i >= lane) racc += RP[i * LDP + lane];
            redR[wave][lane] = racc;
        }
        fro = sum64(fro);
        if (lane == 0) redB[wave] = fro;
        __syncthreads();

        if (wave == 0) {
            float frob = 0.f, rint = 0.f;
#pragma unroll
            for (int w = 0; w < NTW / 64; ++w) {
                frob += redB[w];
                rint += redR[w][lane];
            }
            float iq = 0.f, ik = 0.f;
#pragma unroll
            for (int cb = 0; cb < NKB; ++cb) {
                iq += redQ[cb][lane];
                ik += redK[cb][lane];
            }
            // inclusive suffix sum of iq, exclusive prefix sum of ik
            float sq = iq, pk = ik;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float a1 = __shfl_down(sq, off);
                const float a2 = __shfl_up(pk, off);
                if (lane + off < 64) sq += a1;
                if (lane >= off) pk += a2;
            }
            float pke = __shfl_up(pk, 1);
            if (lane == 0) pke = 0.f;
            if (lane < rows) dla[bh * T + c * CH + lane] = rint + sq + pke + expf(blh) * frob;
        }
    }

    if (hasK) {
        const int colk = cbk * 32 + cl;
        if (colk < dk_) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = rbk * 32 + acc_row(r, lane);
                if (row < rows) {
                    const int64_t o = (bg * T + c * CH + row) * dk_ + colk;
                    dq[o] = dQacc[r];
                    dk[o] = dKacc[r];
                }
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

// ---------------------------------------------------------------------------
// Kernel timing (optional, process-global).

enum KernelId { KID_CUMSUM = 0, KID_SCAN, KID_OUTPUT, KID_SCAN2, KID_GRADS, KID_COUNT };
static const char *kKernelNames[KID_COUNT] = {"chunk_cumsum", "state_scan", "chunk_output", "state_scan_bidir",
                                              "bwd_grads"};

struct Timing {
    bool on = false;
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

struct TimedLaunch {
    int kid;
    hipStream_t st;
    hipEvent_t a = nullptr, b = nullptr;
    TimedLaunch(int kid_, hipStream_t st_) : kid(kid_), st(st_)
    {
        if (g_timing.on) {
            a = get_event();
            b = get_event();
            if (a && b) hipEventRecord(a, st);
        }
    }
    ~TimedLaunch()
    {
        if (a && b) {
            hipEventRecord(b, st);
            g_timing.pending[kid][0].push_back(a);
            g_timing.pending[kid][1].push_back(b);
        }
    }
};

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

struct Problem {
    ssd_shape s;
    Layout L;
    int DKP, DVP;
    int vecK, vecV;
    float *bcum, *bl, *states, *dstates;
};

static int launch_status()
{
    return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_DEVICE;
}

// Chunk cumsum, then the fused state scan: the forward direction only
// (ndir = 1, fills `states` with S_in) or both directions in one launch
// (ndir = 2, also fills `dstates` with dS_out and writes dh0).
static int run_scan(const Problem &P, int ndir, const float *q, const float *k, const float *v, const float *dy,
                    const float *la, const float *h0, float *dh0, hipStream_t st)
{
    const ssd_shape &s = P.s;
    const int64_t BH = s.B * s.H;
    {
        TimedLaunch tl(KID_CUMSUM, st);
        const int64_t nw = BH * P.L.NC;
        const int64_t grid = (nw + 3) / 4;
        k_chunk_cumsum<<<dim3((unsigned)grid), dim3(NTH), 0, st>>>(la, P.bcum, P.bl, s.T, P.L.NC, P.L.NCp, nw);
    }
    if (launch_status() != SSD_OK) return SSD_ERR_DEVICE;
    {
        TimedLaunch tl(ndir == 1 ? KID_SCAN : KID_SCAN2, st);
        SSD_DISPATCH_DIMS(P.DKP, P.DVP, ({
            constexpr int TJ = VP < 64 ? VP : 64;
            const int64_t per_dir = BH * (KP / TI) * (VP / TJ);
            k_state_scan<KP, VP><<<dim3((unsigned)(ndir * per_dir)), dim3(NTH), 0, st>>>(
                q, k, v, dy, h0, P.bcum, P.bl, P.states, P.dstates, dh0, (int)s.G, (int)s.H, s.T, (int)s.dk,
                (int)s.dv, P.L.NC, P.L.NCp, P.L.Epad, per_dir, P.vecK, P.vecV);
        }));
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
    P->vecK = (shape->dk % 4) == 0;
    P->vecV = (shape->dv % 4) == 0;
    char *w = static_cast<char *>(ws);
    P->bcum = reinterpret_cast<float *>(w + P->L.off[0]);
    P->bl = reinterpret_cast<float *>(w + P->L.off[1]);
    P->states = reinterpret_cast<float *>(w + P->L.off[2]);
    P->dstates = backward ? reinterpret_cast<float *>(w + P->L.off[3]) : nullptr;
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

    rc = run_scan(P, 1, q, k, v, nullptr, log_alpha, h0, nullptr, st);
    if (rc != SSD_OK) return rc;
    {
        TimedLaunch tl(KID_OUTPUT, st);
        SSD_DISPATCH_DIMS(P.DKP, P.DVP,
                          (k_chunk_output<KP, VP><<<dim3((unsigned)(s.B * s.G * P.L.NC)), dim3(NTW), 0, st>>>(
                              q, k, v, P.bcum, P.states, y, (int)s.G, (int)s.H, s.T, (int)s.dk, (int)s.dv, P.L.NC,
                              P.L.Epad, P.vecK, P.vecV)));
    }
    return launch_status();
}

int ssd_bwd(const ssd_shape *shape, const float *q, const float *k, const float *v, const float *log_alpha,
            const float *h0, const float *dy, float *dq, float *dk, float *dv, float *dlog_alpha, float *dh0,
            void *workspace, size_t workspace_bytes, void *stream)
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
        k_zero<<<dim3((unsigned)((n + NTH - 1) / NTH)), dim3(NTH), 0, st>>>(dh0, n);
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

    // S_in (forward) and dS_out (reverse) of every chunk, and dh0.
    rc = run_scan(P, 2, q, k, v, dy, log_alpha, h0, dh0, st);
    if (rc != SSD_OK) return rc;
    {
        TimedLaunch tl(KID_GRADS, st);
        SSD_DISPATCH_DIMS(P.DKP, P.DVP,
                          (k_bwd_grads<KP, VP><<<dim3((unsigned)(s.B * s.G * P.L.NC)), dim3(NTW), 0, st>>>(
                              q, k, v, dy, P.bcum, P.bl, P.states, P.dstates, dq, dk, dv, dlog_alpha, (int)s.G,
                              (int)s.H, s.T, (int)s.dk, (int)s.dv, P.L.NC, P.L.NCp, P.L.Epad, P.vecK, P.vecV)));
    }
    return launch_status();
}

int ssd_kernel_timing_enable(int enable)
{
    g_timing.on = enable != 0;
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
