// The selective (Mamba-style) scan for gfx950: forward.
//
// Per batch b, channel d and state n (N <= 16), with h_{-1} = 0:
//     h_t[d,n] = exp(delta_t[d] A[d,n]) h_{t-1}[d,n] + delta_t[d] B_t[n] x_t[d]
//     y_t[d]   = sum_n C_t[n] h_t[d,n] + Dskip[d] x_t[d]
// (the plain reading of the argument set of kernel_mamba_cpu.json, whose
// byte counts fix x, delta [B,L,D], A [D,N], B, C [B,L,N] and Dskip [D]).
//
// The work is elementwise over (b, d) with a linear recurrence over t, and
// bound by the exponentials and the x / delta / y traffic, not by a
// contraction: no MFMA.  One thread owns one (b, d) and all N states in
// registers; the 64 lanes of a wave take 64 consecutive channels, so every
// x, delta and y access of a step is one coalesced 256-byte row segment,
// and B_t, C_t (the same for the whole block) are uniform loads.
//
// B * D threads alone leave most of the chip idle, so the sequence is cut
// into segments that run in parallel (the recurrence is linear):
//   1. k_mamba_scan<false>: each segment from a zero state, keeping its end
//      state and its summed delta (the segment's decay is exp(A sum delta));
//   2. k_mamba_carry: per (b, n, d), in segment order, the state entering
//      each segment, written over the end states;
//   3. k_mamba_scan<true>: each segment again from its entering state,
//      writing y.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

constexpr int MB = 256;                       // threads (channels) per block
constexpr int MNS = MAMBA_MAX_STATE;          // states held per thread
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// FULL: N == MNS, so no state is masked.  The block first stages the B (and
// C) rows of its segment in LDS, so that a step's 16 (32) uniform values are
// broadcast reads, and each thread keeps its x and delta PF steps ahead in
// registers: a step waits on no global load.
template <bool OUT, bool FULL>
__global__ __launch_bounds__(MB) void k_mamba_scan(const float *__restrict__ x, const float *__restrict__ delta,
                                                  const float *__restrict__ A, const float *__restrict__ Bm,
                                                  const float *__restrict__ Cm, const float *__restrict__ Ds,
                                                  float *__restrict__ y, float *__restrict__ hend,
                                                  float *__restrict__ sdl, int64_t L, int64_t D, int N,
                                                  int64_t seg_len, int64_t nseg)
{
    constexpr int PF = 8;
    __shared__ __attribute__((aligned(16))) float BC[OUT ? 2 : 1][kMambaMaxSeg][MNS];
    if constexpr (FULL) N = MNS;
    const int64_t d = (int64_t)blockIdx.x * MB + threadIdx.x;
    const int64_t p = blockIdx.y, b = blockIdx.z;
    const int64_t t0 = p * seg_len, t1 = (t0 + seg_len) < L ? (t0 + seg_len) : L;
    const int nrow = (int)(t1 - t0);
    {
        const float *Bs = Bm + (b * L + t0) * N, *Cs = Cm + (b * L + t0) * N;
        for (int i = threadIdx.x; i < nrow * MNS; i += MB) {
            const int r = i / MNS, n = i % MNS;
            BC[0][r][n] = n < N ? Bs[r * N + n] : 0.f;
            if constexpr (OUT) BC[OUT ? 1 : 0][r][n] = n < N ? Cs[r * N + n] : 0.f;
        }
    }
    __syncthreads();
    if (d >= D) return;   // no barrier below
    float a2[MNS], h[MNS];
#pragma unroll
    for (int n = 0; n < MNS; ++n) {
        a2[n] = n < N ? A[d * N + n] * kLog2e : 0.f;   // exp(delta A) = exp2(delta A log2 e)
        h[n] = 0.f;
    }
    if (OUT && nseg > 1) {
        // the state entering this segment (the carry pass left it here)
#pragma unroll
        for (int n = 0; n < MNS; ++n)
            if (n < N) h[n] = hend[((b * nseg + p) * N + n) * D + d];
    }
    const float dsk = OUT ? Ds[d] : 0.f;
    float sd = 0.f;
    // The segment's rows of x, delta and y as buffer resources: row r of
    // the lane's channel is at the uniform offset r D 4 (an SGPR) plus the
    // lane's d 4, so no step spends vector instructions on addresses.
    // Prefetches past the segment's last row re-read that row (the row index
    // is clamped), and their values are never used.
    const int64_t seg0 = (b * L + t0) * D;
    const rsrc_t xs = make_rsrc(x + seg0, (int64_t)nrow * D * 4), ds = make_rsrc(delta + seg0, (int64_t)nrow * D * 4);
    const rsrc_t ys = make_rsrc(y + seg0, OUT ? (int64_t)nrow * D * 4 : 0);
    const uint32_t lo = (uint32_t)d * 4u;
    const uint32_t rowb = (uint32_t)D * 4u;
    auto ld = [&](rsrc_t r, int row) {
        const int rc = row < nrow ? row : nrow - 1;
        return __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, lo, (int)((uint32_t)rc * rowb), 0));
    };
    float dlb[PF], xvb[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        dlb[i] = ld(ds, i);
        xvb[i] = ld(xs, i);
    }
    for (int r0 = 0; r0 < nrow; r0 += PF) {
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            const int r = r0 + i;
            if (r >= nrow) break;   // uniform
            const float dl = dlb[i], xv = xvb[i];
            dlb[i] = ld(ds, r + PF);   // refill the slot with step r + PF
            xvb[i] = ld(xs, r + PF);
            const float u = dl * xv;
            float bt[MNS], ct[MNS];
#pragma unroll
            for (int m = 0; m < MNS / 4; ++m) {
                const float4 b4 = *reinterpret_cast<const float4 *>(&BC[0][r][4 * m]);
                bt[4 * m] = b4.x;
                bt[4 * m + 1] = b4.y;
                bt[4 * m + 2] = b4.z;
                bt[4 * m + 3] = b4.w;
                if constexpr (OUT) {
                    const float4 c4 = *reinterpret_cast<const float4 *>(&BC[OUT ? 1 : 0][r][4 * m]);
                    ct[4 * m] = c4.x;
                    ct[4 * m + 1] = c4.y;
                    ct[4 * m + 2] = c4.z;
                    ct[4 * m + 3] = c4.w;
                }
            }
            float acc = 0.f;
#pragma unroll
            for (int n = 0; n < MNS; ++n) {
                if (FULL || n < N) {
                    h[n] = exp2_fast(dl * a2[n]) * h[n] + u * bt[n];
                    if (OUT) acc += ct[n] * h[n];
                }
            }
            if (OUT)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(acc + dsk * xv), ys, lo,
                                                      (int)((uint32_t)r * rowb), kStoreNT);
            else
                sd += dl;
        }
    }
    if (!OUT) {
#pragma unroll
        for (int n = 0; n < MNS; ++n)
            if (n < N) hend[((b * nseg + p) * N + n) * D + d] = h[n];
        sdl[(b * nseg + p) * D + d] = sd;
    }
}

// Per (b, n, d): replace each segment's end state by the state entering it,
// S_0 = 0, S_{p+1} = g_p S_p + e_p with g_p = exp(A sum delta over p) and
// e_p the end state.  The chain over p is cut in two levels: a block holds
// 64 channels x CJ groups of gs consecutive segments; each thread composes
// its group's maps (g, e), one thread per channel walks the CJ groups, and
// each thread then walks its group again from the state entering it.  The
// chain depth is 2 gs + CJ instead of nseg.
constexpr int CJ = 16, CD = 64;
__global__ __launch_bounds__(CJ *CD) void k_mamba_carry(const float *__restrict__ A, float *__restrict__ hend,
                                                       const float *__restrict__ sdl, int64_t D, int N, int64_t nseg)
{
    __shared__ float Gm[CJ][CD], Em[CJ][CD], Sin[CJ][CD];
    const int dl = threadIdx.x % CD, j = threadIdx.x / CD;
    const int64_t d = (int64_t)blockIdx.x * CD + dl;
    const int n = blockIdx.y;
    const int64_t b = blockIdx.z;
    const bool live = d < D;
    const int64_t dd = live ? d : 0;   // masked lanes read a valid address and store nothing
    const float a2 = A[dd * N + n] * kLog2e;
    const int64_t gs = (nseg + CJ - 1) / CJ;
    const int64_t p0 = j * gs, p1 = (p0 + gs) < nseg ? (p0 + gs) : nseg;
    float *e = hend + (b * nseg * N + n) * D + dd;   // segment p at e[p N D]
    const float *sg = sdl + b * nseg * D + dd;        // segment p at sg[p D]
    const int64_t es = (int64_t)N * D;
    // compose the maps of segments p0 .. p1 - 1 (all but the last segment carry)
    float G = 1.f, E = 0.f;
    for (int64_t p = p0; p < p1 && p + 1 < nseg; ++p) {
        const float g = exp2_fast(a2 * sg[p * D]);
        G = g * G;
        E = g * E + e[p * es];
    }
    Gm[j][dl] = G;
    Em[j][dl] = E;
    __syncthreads();
    if (j == 0) {
        float S = 0.f;
        for (int q = 0; q < CJ; ++q) {
            Sin[q][dl] = S;
            S = Gm[q][dl] * S + Em[q][dl];
        }
    }
    __syncthreads();
    float S = Sin[j][dl];
    for (int64_t p = p0; p < p1; ++p) {
        const float end = e[p * es], s = sg[p * D];
        if (live) e[p * es] = S;
        if (p + 1 < nseg) S = exp2_fast(a2 * s) * S + end;
    }
}

}  // namespace ssd

using namespace ssd;

extern "C" int mamba_fwd(const mamba_shape *shape, const float *x, const float *delta, const float *A,
                         const float *Bm, const float *Cm, const float *Ds, float *y, void *workspace,
                         size_t workspace_bytes, void *stream)
{
    const int rc = mamba_check_shape(shape);
    if (rc != SSD_OK) return rc;
    const mamba_shape &s = *shape;
    if (s.B == 0 || s.L == 0) return SSD_OK;   // y has no elements
    if (!x || !delta || !A || !Bm || !Cm || !Ds || !y) return SSD_ERR_NULL;
    const void *ptrs[] = {x, delta, A, Bm, Cm, Ds, y};
    for (const void *q : ptrs)
        if ((reinterpret_cast<uintptr_t>(q) & 3u) != 0) return SSD_ERR_ALIGN;
    const MambaPlan P = mamba_plan(shape, device_cus());
    if (workspace_bytes < P.total) return SSD_ERR_WORKSPACE;
    float *hend = nullptr, *sdl = nullptr;
    if (P.total > 0) {
        if (!workspace) return SSD_ERR_NULL;
        if (!aligned16(workspace)) return SSD_ERR_ALIGN;
        hend = reinterpret_cast<float *>(static_cast<char *>(workspace) + P.hend);
        sdl = reinterpret_cast<float *>(static_cast<char *>(workspace) + P.sdl);
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int N = (int)s.N;
    const unsigned nb = (unsigned)((s.D + MB - 1) / MB);
    const dim3 grid(nb, (unsigned)P.nseg, (unsigned)s.B);
    auto pass = [&](auto out_c) {
        constexpr bool OUT = decltype(out_c)::value;
        if (N == MNS)
            launch(nullptr, -1, k_mamba_scan<OUT, true>, grid, dim3(MB), st, x, delta, A, Bm, Cm, Ds, y, hend, sdl,
                   s.L, s.D, N, P.seg_len, P.nseg);
        else
            launch(nullptr, -1, k_mamba_scan<OUT, false>, grid, dim3(MB), st, x, delta, A, Bm, Cm, Ds, y, hend, sdl,
                   s.L, s.D, N, P.seg_len, P.nseg);
    };
    if (P.nseg > 1) {
        pass(BoolC<false>{});
        if (launch_status() != SSD_OK) return SSD_ERR_DEVICE;
        launch(nullptr, -1, k_mamba_carry, dim3((unsigned)((s.D + CD - 1) / CD), (unsigned)N, (unsigned)s.B),
               dim3(CJ * CD), st, A, hend, (const float *)sdl, s.D, N, P.nseg);
        if (launch_status() != SSD_OK) return SSD_ERR_DEVICE;
    }
    pass(BoolC<true>{});
    return launch_status();
}
