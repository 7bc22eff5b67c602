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
template <int DP, int LD, bool SCALE>
__device__ __forceinline__ void stage_rows(float *dst, const float *__restrict__ src, int rows, int d,
                                           bool vec, const float *w)
{
    if (vec) {
        constexpr int Q4 = DP / 4;
        for (int idx = threadIdx.x; idx < CH * Q4; idx += NTH) {
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
        for (int idx = threadIdx.x; idx < CH * DP; idx += NTH) {
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
// K3 (MODE 0): X_c = K^T diag(e^{b_L - b}) V  (dk x dv), the chunk's own
//              contribution to the outgoing state.
// B1 (MODE 1): Z_c = Q^T diag(e^{b}) dY      (dk x dv), the chunk's own
//              contribution to the gradient of the incoming state.
// One block per (b,h,chunk); the 32x32 output tiles are spread over the four
// waves; the contraction over the 64 chunk positions reads both operands
// from LDS.
template <int DKP, int DVP, int MODE>
__global__ __launch_bounds__(NTH) void k_chunk_state(const float *__restrict__ Ag, const float *__restrict__ Bg,
                                                     const float *__restrict__ bcum, const float *__restrict__ bl,
                                                     float *__restrict__ states, int G, int H, int64_t T, int dk,
                                                     int dv, int64_t NC, int64_t NCp, int64_t Epad, int vecA,
                                                     int vecB)
{
    constexpr int LDA = DKP, LDB = DVP;
    __shared__ float As[CH * LDA];
    __shared__ float Bs[CH * LDB];
    __shared__ float w[CH];

    const int64_t c = blockIdx.x % NC;
    const int64_t bh = blockIdx.x / NC;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const int g = h / (H / G);
    const int rows = (int)((T - c * CH) < CH ? (T - c * CH) : CH);
    const float *a_src = Ag + ((b * G + g) * T + c * CH) * dk;
    const float *b_src = Bg + (bh * T + c * CH) * dv;

    if (threadIdx.x < CH) {
        const int t = threadIdx.x;
        const float bt = bcum[bh * NC * CH + c * CH + t];
        const float wt = (MODE == 0) ? expf(bl[bh * NCp + c] - bt) : expf(bt);
        w[t] = (t < rows) ? wt : 0.f;
    }
    stage_rows<DKP, LDA, false>(As, a_src, rows, dk, vecA != 0, nullptr);
    __syncthreads();
    stage_rows<DVP, LDB, true>(Bs, b_src, rows, dv, vecB != 0, w);
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cl = lane & 31, kh = lane >> 5;
    constexpr int NIB = DKP / 32, NJB = DVP / 32, NBLK = NIB * NJB, NBW = (NBLK + 3) / 4;
    f32x16 acc[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[j] = zero16();

#pragma unroll 4
    for (int k = 0; k < CH; k += 2) {
        const int kr = k + kh;
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            const int blk = wave + 4 * j;
            if (blk < NBLK) {
                const int ib = blk / NJB, jb = blk % NJB;
                acc[j] = mfma32(As[kr * LDA + ib * 32 + cl], Bs[kr * LDB + jb * 32 + cl], acc[j]);
            }
        }
    }

    float *dst = states + (bh * NC + c) * Epad;
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
        const int blk = wave + 4 * j;
        if (blk < NBLK) {
            const int ib = blk / NJB, jb = blk % NJB;
            const int n = jb * 32 + cl;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = ib * 32 + acc_row(r, lane);
                if (i < dk && n < dv) dst[i * dv + n] = acc[j][r];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// K4 / B2: sequential pass over chunks, in place over the per-chunk slabs.
// Forward (REV = false):  S = h0;  for c = 0..NC-1:  x = slab[c]; slab[c] = S;
//                         S = e^{b_L(c)} S + x.       (slab[c] becomes S_in(c))
// Reverse (REV = true):   S = 0;   for c = NC-1..0:  z = slab[c]; slab[c] = S;
//                         S = e^{b_L(c)} S + z;  fin = S at the end.
//                         (slab[c] becomes dS_out(c), fin = dh0)
// Each thread carries 4 consecutive state elements through every chunk; the
// per-chunk decays are loaded 64 at a time (one per lane) and broadcast with
// readlane.  Loads of 16 chunks are issued before their stores.
template <bool REV>
__global__ __launch_bounds__(NTH) void k_state_pass(float *__restrict__ states, const float *__restrict__ bl,
                                                    const float *__restrict__ init, float *__restrict__ fin,
                                                    int64_t NC, int64_t NCp, int64_t E, int64_t Epad,
                                                    int64_t blocks_per_bh)
{
    constexpr int BATCH = 16;
    const int64_t bh = blockIdx.x / blocks_per_bh;
    const int64_t e0 = ((blockIdx.x - bh * blocks_per_bh) * NTH + threadIdx.x) * 4;
    const bool active = e0 < Epad;
    const int lane = threadIdx.x & 63;
    float *base = states + bh * NC * Epad + e0;

    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    if (!REV && init && active) {
        const float *ip = init + bh * E + e0;
        if (e0 + 0 < E) s0 = ip[0];
        if (e0 + 1 < E) s1 = ip[1];
        if (e0 + 2 < E) s2 = ip[2];
        if (e0 + 3 < E) s3 = ip[3];
    }

    for (int64_t g0 = 0; g0 < NC; g0 += 64) {
        const int cnt = (int)((NC - g0) < 64 ? (NC - g0) : 64);
        float dl = 0.f;
        if (lane < cnt) {
            const int64_t cc = REV ? NC - 1 - (g0 + lane) : g0 + lane;
            dl = expf(bl[bh * NCp + cc]);
        }
        for (int j0 = 0; j0 < cnt; j0 += BATCH) {
            float4 x[BATCH];
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int j = j0 + u;
                if (j < cnt && active) {
                    const int64_t cc = REV ? NC - 1 - (g0 + j) : g0 + j;
                    x[u] = *reinterpret_cast<const float4 *>(base + cc * Epad);
                }
            }
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int j = j0 + u;
                if (j < cnt) {
                    const float d = readlane_f(dl, j);
                    if (active) {
                        const int64_t cc = REV ? NC - 1 - (g0 + j) : g0 + j;
                        *reinterpret_cast<float4 *>(base + cc * Epad) = make_float4(s0, s1, s2, s3);
                        s0 = d * s0 + x[u].x;
                        s1 = d * s1 + x[u].y;
                        s2 = d * s2 + x[u].z;
                        s3 = d * s3 + x[u].w;
                    }
                }
            }
        }
    }
    if (REV && fin && active) {
        float *fp = fin + bh * E + e0;
        if (e0 + 0 < E) fp[0] = s0;
        if (e0 + 1 < E) fp[1] = s1;
        if (e0 + 2 < E) fp[2] = s2;
        if (e0 + 3 < E) fp[3] = s3;
    }
}

// ---------------------------------------------------------------------------
// K2 + K5: output of one chunk for every head of one group.
// One block per (b,g,chunk).  Q K^T (causal 32x32 tiles only) is formed once
// and kept in registers; per head it is masked and decayed into P (LDS),
// then Y = P V + diag(e^b) (Q S_in) with V staged in LDS and S_in read from
// the state slabs.
template <int DKP, int DVP>
__global__ __launch_bounds__(NTH) void k_chunk_output(const float *__restrict__ q, const float *__restrict__ k,
                                                      const float *__restrict__ v, const float *__restrict__ bcum,
                                                      const float *__restrict__ states, float *__restrict__ y,
                                                      int G, int H, int64_t T, int dk, int dv, int64_t NC,
                                                      int64_t Epad, int vecK, int vecV)
{
    constexpr int LDQ = DKP + 1;
    constexpr int LDKV = (DKP > DVP ? DKP : DVP) + 1;
    constexpr int LDP = CH + 1;
    __shared__ float Qs[CH * LDQ];
    __shared__ float KVs[CH * LDKV];
    __shared__ float Ps[CH * LDP];
    __shared__ float bs[CH], eb[CH];

    const int64_t c = blockIdx.x % NC;
    const int64_t bg = blockIdx.x / NC;
    const int g = (int)(bg % G);
    const int64_t b = bg / G;
    const int hpg = H / G;
    const int rows = (int)((T - c * CH) < CH ? (T - c * CH) : CH);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cl = lane & 31, kh = lane >> 5;

    stage_rows<DKP, LDQ, false>(Qs, q + (bg * T + c * CH) * dk, rows, dk, vecK != 0, nullptr);
    stage_rows<DKP, LDKV, false>(KVs, k + (bg * T + c * CH) * dk, rows, dk, vecK != 0, nullptr);
    __syncthreads();

    // Causal tiles of Q K^T: wave 0 -> (0,0), wave 1 -> (1,0), wave 2 -> (1,1).
    const int ib = (wave == 0) ? 0 : 1;
    const int jb = (wave == 2) ? 1 : 0;
    f32x16 accA = zero16();
    if (wave < 3) {
#pragma unroll 8
        for (int kk = 0; kk < DKP; kk += 2)
            accA = mfma32(Qs[(ib * 32 + cl) * LDQ + kk + kh], KVs[(jb * 32 + cl) * LDKV + kk + kh], accA);
    }
    __syncthreads();   // K no longer needed; its LDS holds V from here on

    constexpr int NCB = DVP / 32, NOB = 2 * NCB, NBW = (NOB + 3) / 4;
    for (int hh = 0; hh < hpg; ++hh) {
        const int64_t bh = b * H + (int64_t)g * hpg + hh;
        if (threadIdx.x < CH) {
            const float bt = bcum[bh * NC * CH + c * CH + threadIdx.x];
            bs[threadIdx.x] = bt;
            eb[threadIdx.x] = expf(bt);
        }
        stage_rows<DVP, LDKV, false>(KVs, v + (bh * T + c * CH) * dv, rows, dv, vecV != 0, nullptr);
        __syncthreads();
        if (wave < 3) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = ib * 32 + acc_row(r, lane), j = jb * 32 + cl;
                Ps[i * LDP + j] = (j <= i) ? accA[r] * expf(bs[i] - bs[j]) : 0.f;
            }
        }
        __syncthreads();

        const float *st = states + (bh * NC + c) * Epad;
#pragma unroll
        for (int jw = 0; jw < NBW; ++jw) {
            const int ob = wave + 4 * jw;
            if (ob < NOB) {
                const int rb = ob / NCB, cb = ob % NCB;
                const int n = cb * 32 + cl;
                f32x16 ay = zero16(), ai = zero16();
                const int kend = (rb + 1) * 32;
                for (int kk = 0; kk < kend; kk += 2)
                    ay = mfma32(Ps[(rb * 32 + cl) * LDP + kk + kh], KVs[(kk + kh) * LDKV + n], ay);
#pragma unroll 8
                for (int i = 0; i < DKP; i += 2) {
                    const int ii = i + kh;
                    const float sv = (ii < dk && n < dv) ? st[ii * dv + n] : 0.f;
                    ai = mfma32(Qs[(rb * 32 + cl) * LDQ + ii], sv, ai);
                }
                if (n < dv) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = rb * 32 + acc_row(r, lane);
                        if (row < rows) y[(bh * T + c * CH + row) * dv + n] = ay[r] + eb[row] * ai[r];
                    }
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// B3 + B4: gradients of one chunk for every head of one group.
// One block per (b,g,chunk).  dq and dk are summed over the group's heads in
// registers (ascending head order); dv and dlog_alpha are written per head.
template <int DKP, int DVP>
__global__ __launch_bounds__(NTH) void k_bwd_grads(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ dy, const float *__restrict__ bcum, const float *__restrict__ bl,
    const float *__restrict__ states, const float *__restrict__ dstates, float *__restrict__ dq,
    float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ dla, int G, int H, int64_t T, int dk_,
    int dv_, int64_t NC, int64_t NCp, int64_t Epad, int vecK, int vecV)
{
    constexpr int LDK = DKP + 1;
    constexpr int LDY = DVP + 1;
    constexpr int LDV = (DVP > CH ? DVP : CH) + 1;   // holds V, later P (C x C)
    constexpr int LDP = CH + 1;
    constexpr int NCBK = DKP / 32, NOBK = 2 * NCBK, NBWK = (NOBK + 3) / 4;
    constexpr int NCBV = DVP / 32, NOBV = 2 * NCBV, NBWV = (NOBV + 3) / 4;
    __shared__ float Qs[CH * LDK];
    __shared__ float Ks[CH * LDK];
    __shared__ float dYs[CH * LDY];
    __shared__ float VPs[CH * LDV];
    __shared__ float dPs[CH * LDP];
    __shared__ float bs[CH], eb[CH], el[CH];
    __shared__ float redQ[NCBK][CH], redK[NCBK][CH];
    __shared__ float redB[NTH / 64];
    __shared__ float redR[NTH / 64][CH];

    const int64_t c = blockIdx.x % NC;
    const int64_t bg = blockIdx.x / NC;
    const int g = (int)(bg % G);
    const int64_t b = bg / G;
    const int hpg = H / G;
    const int rows = (int)((T - c * CH) < CH ? (T - c * CH) : CH);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cl = lane & 31, kh = lane >> 5;
    const int64_t E = (int64_t)dk_ * dv_;

    stage_rows<DKP, LDK, false>(Qs, q + (bg * T + c * CH) * dk_, rows, dk_, vecK != 0, nullptr);
    stage_rows<DKP, LDK, false>(Ks, k + (bg * T + c * CH) * dk_, rows, dk_, vecK != 0, nullptr);
    __syncthreads();

    const int ib = (wave == 0) ? 0 : 1;
    const int jb = (wave == 2) ? 1 : 0;
    f32x16 accA = zero16();
    if (wave < 3) {
#pragma unroll 8
        for (int kk = 0; kk < DKP; kk += 2)
            accA = mfma32(Qs[(ib * 32 + cl) * LDK + kk + kh], Ks[(jb * 32 + cl) * LDK + kk + kh], accA);
    }

    f32x16 dQacc[NBWK], dKacc[NBWK];
#pragma unroll
    for (int j = 0; j < NBWK; ++j) {
        dQacc[j] = zero16();
        dKacc[j] = zero16();
    }

    for (int hh = 0; hh < hpg; ++hh) {
        const int64_t bh = b * H + (int64_t)g * hpg + hh;
        const float *Sin = states + (bh * NC + c) * Epad;
        const float *dSo = dstates + (bh * NC + c) * Epad;
        if (threadIdx.x < CH) {
            const int t = threadIdx.x;
            const float bt = bcum[bh * NC * CH + c * CH + t];
            bs[t] = bt;
            eb[t] = expf(bt);
            el[t] = (t < rows) ? expf(bl[bh * NCp + c] - bt) : 0.f;
        }
        stage_rows<DVP, LDV, false>(VPs, v + (bh * T + c * CH) * dv_, rows, dv_, vecV != 0, nullptr);
        stage_rows<DVP, LDY, false>(dYs, dy + (bh * T + c * CH) * dv_, rows, dv_, vecV != 0, nullptr);
        __syncthreads();

        // dP = (dY V^T) o D into LDS; P = (Q K^T) o D and M = P o (dY V^T)
        // kept in registers.
        f32x16 pP = zero16(), pM = zero16();
        if (wave < 3) {
            f32x16 a = zero16();
#pragma unroll 8
            for (int n = 0; n < DVP; n += 2)
                a = mfma32(dYs[(ib * 32 + cl) * LDY + n + kh], VPs[(jb * 32 + cl) * LDV + n + kh], a);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = ib * 32 + acc_row(r, lane), j = jb * 32 + cl;
                const float D = (j <= i) ? expf(bs[i] - bs[j]) : 0.f;
                dPs[i * LDP + j] = a[r] * D;
                pP[r] = accA[r] * D;
                pM[r] = pP[r] * a[r];
            }
        }
        __syncthreads();

        // dQ_h = diag(e^b) dY S_in^T + dP K ; row sums of dQ_h o Q -> redQ.
#pragma unroll
        for (int jw = 0; jw < NBWK; ++jw) {
            const int ob = wave + 4 * jw;
            if (ob < NOBK) {
                const int rb = ob / NCBK, cb = ob % NCBK;
                const int col = cb * 32 + cl;
                f32x16 a = zero16();
#pragma unroll 8
                for (int n = 0; n < DVP; n += 2) {
                    const int nn = n + kh;
                    const float sv = (col < dk_ && nn < dv_) ? Sin[col * dv_ + nn] : 0.f;
                    a = mfma32(dYs[(rb * 32 + cl) * LDY + nn], sv, a);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = rb * 32 + acc_row(r, lane);
                    a[r] *= eb[row];
                    // e^{b_i} q_i . (dY S_in^T)_i, partial over this column block
                    const float s = sum32(a[r] * Qs[row * LDK + col]);
                    if (cl == 0) redQ[cb][row] = s;
                }
                const int kend = (rb + 1) * 32;
                for (int jj = 0; jj < kend; jj += 2)
                    a = mfma32(dPs[(rb * 32 + cl) * LDP + jj + kh], Ks[(jj + kh) * LDK + col], a);
                dQacc[jw] += a;
            }
        }

        // dK_h = diag(e^{bL-b}) V dS_out^T + dP^T Q ; row sums of dK_h o K -> redK.
#pragma unroll
        for (int jw = 0; jw < NBWK; ++jw) {
            const int ob = wave + 4 * jw;
            if (ob < NOBK) {
                const int rb = ob / NCBK, cb = ob % NCBK;
                const int col = cb * 32 + cl;
                f32x16 a = zero16();
#pragma unroll 8
                for (int n = 0; n < DVP; n += 2) {
                    const int nn = n + kh;
                    const float sv = (col < dk_ && nn < dv_) ? dSo[col * dv_ + nn] : 0.f;
                    a = mfma32(VPs[(rb * 32 + cl) * LDV + nn], sv, a);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = rb * 32 + acc_row(r, lane);
                    a[r] *= el[row];
                    // e^{b_L - b_j} k_j . (V dS_out^T)_j, partial over this column block
                    const float s = sum32(a[r] * Ks[row * LDK + col]);
                    if (cl == 0) redK[cb][row] = s;
                }
                for (int jj = rb * 32; jj < CH; jj += 2)
                    a = mfma32(dPs[(jj + kh) * LDP + rb * 32 + cl], Qs[(jj + kh) * LDK + col], a);
                dKacc[jw] += a;
            }
        }
        __syncthreads();   // V and dP are dead; P goes where V was, M where dP was

        if (wave < 3) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = ib * 32 + acc_row(r, lane), j = jb * 32 + cl;
                VPs[i * LDV + j] = pP[r];
                dPs[i * LDP + j] = pM[r];
            }
        } else {
            // upper-right tile of M is zero (j > i)
#pragma unroll
            for (int r = 0; r < 16; ++r) dPs[acc_row(r, lane) * LDP + 32 + cl] = 0.f;
        }
        __syncthreads();

        // dV_h = diag(e^{bL-b}) K dS_out + P^T dY.
#pragma unroll
        for (int jw = 0; jw < NBWV; ++jw) {
            const int ob = wave + 4 * jw;
            if (ob < NOBV) {
                const int rb = ob / NCBV, cb = ob % NCBV;
                const int col = cb * 32 + cl;
                f32x16 a = zero16();
#pragma unroll 8
                for (int i = 0; i < DKP; i += 2) {
                    const int ii = i + kh;
                    const float sv = (ii < dk_ && col < dv_) ? dSo[ii * dv_ + col] : 0.f;
                    a = mfma32(Ks[(rb * 32 + cl) * LDK + ii], sv, a);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) a[r] *= el[rb * 32 + acc_row(r, lane)];
                for (int jj = rb * 32; jj < CH; jj += 2)
                    a = mfma32(VPs[(jj + kh) * LDV + rb * 32 + cl], dYs[(jj + kh) * LDY + col], a);
                if (col < dv_) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = rb * 32 + acc_row(r, lane);
                        if (row < rows) dv[(bh * T + c * CH + row) * dv_ + col] = a[r];
                    }
                }
            }
        }

        // Rectangle sums R_r = sum_{i >= r} sum_{j < r} M_ij: exclusive prefix
        // over j of every row (in place), then a suffix over i per column.
        for (int i = wave * 16; i < wave * 16 + 16; ++i) {
            float x = dPs[i * LDP + lane];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float yv = __shfl_up(x, off);
                if (lane >= off) x += yv;
            }
            // shift, not subtract: the diagonal term must not enter the prefix
            float xe = __shfl_up(x, 1);
            if (lane == 0) xe = 0.f;
            dPs[i * LDP + lane] = xe;
        }
        __syncthreads();
        {
            float racc = 0.f;
            for (int i = wave * 16; i < wave * 16 + 16; ++i)
                if (i >= lane) racc += dPs[i * LDP + lane];
            redR[wave][lane] = racc;
        }

        // <dS_out(c), S_in(c)>_F (dS_out is zero for the last chunk).
        float part = 0.f;
        if (c + 1 < NC) {
            if ((E & 3) == 0) {
                for (int64_t e = (int64_t)threadIdx.x * 4; e < E; e += NTH * 4) {
                    const float4 x = *reinterpret_cast<const float4 *>(dSo + e);
                    const float4 z = *reinterpret_cast<const float4 *>(Sin + e);
                    part += x.x * z.x + x.y * z.y + x.z * z.z + x.w * z.w;
                }
            } else {
                for (int64_t e = threadIdx.x; e < E; e += NTH) part += dSo[e] * Sin[e];
            }
        }
        part = sum64(part);
        if (lane == 0) redB[wave] = part;
        __syncthreads();

        if (wave == 0) {
            const float fro = (redB[0] + redB[1]) + (redB[2] + redB[3]);
            const float ebl = expf(bl[bh * NCp + c]);
            float iq = 0.f, ik = 0.f;
#pragma unroll
            for (int cb = 0; cb < NCBK; ++cb) {
                iq += redQ[cb][lane];
                ik += redK[cb][lane];
            }
            const float rint = (redR[0][lane] + redR[1][lane]) + (redR[2][lane] + redR[3][lane]);
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
            if (lane < rows) dla[bh * T + c * CH + lane] = rint + sq + pke + ebl * fro;
        }
        __syncthreads();
    }

#pragma unroll
    for (int jw = 0; jw < NBWK; ++jw) {
        const int ob = wave + 4 * jw;
        if (ob < NOBK) {
            const int rb = ob / NCBK, cb = ob % NCBK;
            const int col = cb * 32 + cl;
            if (col < dk_) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = rb * 32 + acc_row(r, lane);
                    if (row < rows) {
                        const int64_t o = (bg * T + c * CH + row) * dk_ + col;
                        dq[o] = dQacc[jw][r];
                        dk[o] = dKacc[jw][r];
                    }
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

enum KernelId { KID_CUMSUM = 0, KID_STATE, KID_PASS, KID_OUTPUT, KID_DSTATE, KID_PASS_REV, KID_GRADS, KID_COUNT };
static const char *kKernelNames[KID_COUNT] = {"chunk_cumsum", "chunk_state", "state_pass", "chunk_output",
                                              "chunk_dstate", "state_pass_rev", "bwd_grads"};

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

static int run_prefix(const Problem &P, const float *q, const float *k, const float *v, const float *la,
                      const float *h0, hipStream_t st)
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
        TimedLaunch tl(KID_STATE, st);
        SSD_DISPATCH_DIMS(P.DKP, P.DVP, (k_chunk_state<KP, VP, 0><<<dim3((unsigned)(BH * P.L.NC)), dim3(NTH), 0, st>>>(
                                             k, v, P.bcum, P.bl, P.states, (int)s.G, (int)s.H, s.T, (int)s.dk,
                                             (int)s.dv, P.L.NC, P.L.NCp, P.L.Epad, P.vecK, P.vecV)));
    }
    if (launch_status() != SSD_OK) return SSD_ERR_DEVICE;
    {
        TimedLaunch tl(KID_PASS, st);
        const int64_t bpb = (P.L.Epad / 4 + NTH - 1) / NTH;
        k_state_pass<false><<<dim3((unsigned)(BH * bpb)), dim3(NTH), 0, st>>>(P.states, P.bl, h0, nullptr, P.L.NC,
                                                                             P.L.NCp, P.L.E, P.L.Epad, bpb);
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

    rc = run_prefix(P, q, k, v, log_alpha, h0, st);
    if (rc != SSD_OK) return rc;
    {
        TimedLaunch tl(KID_OUTPUT, st);
        SSD_DISPATCH_DIMS(P.DKP, P.DVP,
                          (k_chunk_output<KP, VP><<<dim3((unsigned)(s.B * s.G * P.L.NC)), dim3(NTH), 0, st>>>(
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

    // Recompute the incoming state of every chunk.
    rc = run_prefix(P, q, k, v, log_alpha, h0, st);
    if (rc != SSD_OK) return rc;
    const int64_t BH = s.B * s.H;
    {
        TimedLaunch tl(KID_DSTATE, st);
        SSD_DISPATCH_DIMS(P.DKP, P.DVP, (k_chunk_state<KP, VP, 1><<<dim3((unsigned)(BH * P.L.NC)), dim3(NTH), 0, st>>>(
                                             q, dy, P.bcum, P.bl, P.dstates, (int)s.G, (int)s.H, s.T, (int)s.dk,
                                             (int)s.dv, P.L.NC, P.L.NCp, P.L.Epad, P.vecK, P.vecV)));
    }
    if (launch_status() != SSD_OK) return SSD_ERR_DEVICE;
    {
        TimedLaunch tl(KID_PASS_REV, st);
        const int64_t bpb = (P.L.Epad / 4 + NTH - 1) / NTH;
        k_state_pass<true><<<dim3((unsigned)(BH * bpb)), dim3(NTH), 0, st>>>(P.dstates, P.bl, nullptr, dh0, P.L.NC,
                                                                            P.L.NCp, P.L.E, P.L.Epad, bpb);
    }
    if (launch_status() != SSD_OK) return SSD_ERR_DEVICE;
    {
        TimedLaunch tl(KID_GRADS, st);
        SSD_DISPATCH_DIMS(P.DKP, P.DVP,
                          (k_bwd_grads<KP, VP><<<dim3((unsigned)(s.B * s.G * P.L.NC)), dim3(NTH), 0, st>>>(
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
