// The selective (Mamba-style) scan for gfx950: forward and backward.
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
// and B_t, C_t (the same for the whole block) are broadcast reads from LDS.
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

// FULL: N == MNS, a constant in the index arithmetic.  The block first
// stages the B (and C) rows of its segment in LDS, so that a step's 16 (32)
// uniform values are broadcast reads, and each thread keeps its x and delta
// PF steps ahead in registers: a step waits on no global load.
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
    // One step on the values of step r (the caller refills their slot).
    auto step = [&](float dl, float xv, int r) {
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
            // states past N have a zero exponent, zero B and C rows and a zero
            // start: they stay 0 and add nothing, so no state is branched on
            float acc = 0.f;
#pragma unroll
            for (int n = 0; n < MNS; ++n) {
                h[n] = exp2_fast(dl * a2[n]) * h[n] + u * bt[n];
                if (OUT) acc += ct[n] * h[n];
            }
            if (OUT)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(acc + dsk * xv), ys, lo,
                                                      (int)((uint32_t)r * rowb), kStoreNT);
            else
                sd += dl;
    };
    // Whole groups of PF steps: each slot is used, then refilled with the
    // step PF later, after a scheduling barrier, so that the new value takes
    // the old one's register and a step waits only on loads issued PF steps
    // earlier.  (An exit inside the group, or a refill issued while the old
    // value is still live, turns the slots into register copies that wait on
    // the loads just issued.)
    int r0 = 0;
    for (; r0 + PF <= nrow; r0 += PF) {
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            step(dlb[i], xvb[i], r0 + i);
            __builtin_amdgcn_sched_barrier(0);
            dlb[i] = ld(ds, r0 + i + PF);
            xvb[i] = ld(xs, r0 + i + PF);
        }
    }
    // the last nrow - r0 < PF steps, already loaded
#pragma unroll
    for (int i = 0; i < PF - 1; ++i)
        if (r0 + i < nrow) step(dlb[i], xvb[i], r0 + i);
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
struct CarryLds {
    float G[CJ][CD], E[CJ][CD], S[CJ][CD];
};
__device__ __forceinline__ void carry_body(const float *__restrict__ A, float *__restrict__ hend,
                                           const float *__restrict__ sdl, int64_t D, int N, int64_t nseg, int n,
                                           int64_t b, CarryLds &sh)
{
    auto &Gm = sh.G, &Em = sh.E, &Sin = sh.S;
    const int dl = threadIdx.x % CD, j = threadIdx.x / CD;
    const int64_t d = (int64_t)blockIdx.x * CD + dl;
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

__global__ __launch_bounds__(CJ *CD) void k_mamba_carry(const float *__restrict__ A, float *__restrict__ hend,
                                                       const float *__restrict__ sdl, int64_t D, int N, int64_t nseg)
{
    __shared__ CarryLds sh;
    carry_body(A, hend, sdl, D, N, nseg, blockIdx.y, blockIdx.z, sh);
}


// ---- backward
//
// With G_t[d,n] = dL/dh_t (L = sum dy . y), a_t = exp(delta_t A):
//     G_t        = C_t[n] dy_t[d] + a_{t+1} G_{t+1}
//     dx_t[d]    = Dskip[d] dy_t[d] + delta_t[d] sum_n G_t B_t[n]
//     ddelta_t[d]= sum_n G_t (A[d,n] a_t h_{t-1} + B_t[n] x_t[d])
//     dA[d,n]    = sum_{b,t} G_t delta_t[d] a_t h_{t-1}
//     dB_t[n]    = sum_d G_t delta_t[d] x_t[d]       dC_t[n] = sum_d dy_t[d] h_t[d,n]
//     dDskip[d]  = sum_{b,t} dy_t[d] x_t[d]
// The sequence is cut into segments of kMambaBwdSeg steps:
//   1. k_mamba_seg_ends: per segment, the forward from a zero state (its end
//      state and summed delta) and the adjoint from zero at its end (the
//      adjoint at its first step); one thread per (b, d) as in the forward;
//   2. k_mamba_carries, one launch: the forward's carry (the state entering
//      every segment from the left) and the reverse one (the adjoint entering
//      it from the right, a_{t1} G_{t1});
//   3. k_mamba_bwd_seg: per segment, h over its steps again (kept in
//      registers), then the steps in reverse with the true adjoint: dx and
//      ddelta (sums over n in the lane and over the channel's 8 lanes), dB
//      and dC (sums over the block's channels: channel pairs by DPP, then an
//      LDS transpose; the block walks all channel chunks of its segment), dA
//      and dDskip per segment;
//   4. k_mamba_wsum: dA and dDskip summed over batch and segments, and the
//      dB / dC partials of blocks that split the channels, in fixed order.
// Threads of pass 3 own two states of one (b, d): eight consecutive lanes
// hold one channel's 16 states.  The chunk's x, delta and dy (and the
// segment's B and C rows) are staged in LDS with coalesced loads, and each
// row of lanes reads its channel's value there as a broadcast.

namespace {
constexpr int NS = MAMBA_MAX_STATE;   // states per channel
constexpr int SB = kMambaBwdSeg;      // steps per backward segment
constexpr int LPC = 8;                // lanes per channel in pass 3, two states each
constexpr int BD = kMambaBwdChans;    // channels per block in pass 3
constexpr int BT = BD * LPC;          // threads per block (512)
constexpr int WIN = 8;                // steps per dB / dC transpose window
constexpr int XP = SB + 4;            // pitch of a channel's staged steps (16-byte rows)
constexpr int kQuadXor1 = 0xB1;       // DPP quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // DPP quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // DPP: lane i of each 8-lane half row reads lane 7 - i
static_assert(SB % 4 == 0 && (SB * BD) % BT == 0 && 2 * LPC == NS, "tile shapes");
}  // namespace

// 1. per (b, segment, d), in one walk from the segment's last step back:
// its end state from a zero start, h_end = sum_t W_t delta_t x_t B_t with
// W_t = a_{t+1} ... a_{end} (the product of the decays after t), its summed
// delta, and the adjoint at its first step from zero past its end,
// G_t = C_t dy_t + a_{t+1} G_{t+1}.  Both take the same decay a_{t+1} at
// step t, so one exponential serves them.  Steps past the sequence's end read
// as delta = x = dy = 0 (and B = C = 0 in LDS): a decay of 1 and no input,
// which leaves both sums unchanged, so the walk does not branch on them.
template <bool FULL>
__global__ __launch_bounds__(MB) void k_mamba_seg_ends(const float *__restrict__ x, const float *__restrict__ delta,
                                                      const float *__restrict__ A, const float *__restrict__ Bm,
                                                      const float *__restrict__ Cm, const float *__restrict__ dy,
                                                      float *__restrict__ hend, float *__restrict__ sdl,
                                                      float *__restrict__ gl, int64_t L, int64_t D, int N,
                                                      int64_t nseg)
{
    __shared__ __attribute__((aligned(16))) float BC[2][SB][MNS];
    if constexpr (FULL) N = MNS;
    const int64_t d = (int64_t)blockIdx.x * MB + threadIdx.x, p = blockIdx.y, b = blockIdx.z;
    const int64_t t0 = p * SB, t1 = (t0 + SB) < L ? (t0 + SB) : L;
    const int nrow = (int)(t1 - t0);
    for (int i = threadIdx.x; i < SB * MNS; i += MB) {
        const int r = i / MNS, n = i % MNS;
        const bool in = r < nrow && n < N;
        BC[0][r][n] = in ? Bm[(b * L + t0 + r) * N + n] : 0.f;
        BC[1][r][n] = in ? Cm[(b * L + t0 + r) * N + n] : 0.f;
    }
    __syncthreads();
    if (d >= D) return;   // no barrier below
    const int64_t seg0 = (b * L + t0) * D;
    const int64_t segb = (int64_t)nrow * D * 4;   // bytes of the segment's rows
    const rsrc_t rx = make_rsrc(x + seg0, segb), rdl = make_rsrc(delta + seg0, segb);
    const rsrc_t rdy = make_rsrc(dy + seg0, segb);
    const uint32_t lo = (uint32_t)d * 4u, rowb = (uint32_t)D * 4u;
    // The row offset goes in the lane offset, which the buffer range check
    // covers: rows past the segment (the resource's end) read 0.  Loaded
    // last step first, the order the walk uses them.
    auto ld = [&](rsrc_t r_, int r) {
        return __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_, lo + (uint32_t)r * rowb, 0, 0));
    };
    float dl[SB], xv[SB], dv[SB];
#pragma unroll
    for (int r = SB - 1; r >= 0; --r) {
        dl[r] = ld(rdl, r);
        xv[r] = ld(rx, r);
        dv[r] = ld(rdy, r);
    }
    float a2[MNS], W[MNS], he[MNS], G[MNS];
#pragma unroll
    for (int n = 0; n < MNS; ++n) {
        a2[n] = n < N ? A[d * N + n] * kLog2e : 0.f;
        W[n] = 1.f;
        he[n] = 0.f;
        G[n] = 0.f;
    }
    float sd = 0.f;
#pragma unroll
    for (int r = SB - 1; r >= 0; --r) {
        const float u = dl[r] * xv[r];
        sd += dl[r];
#pragma unroll
        for (int n = 0; n < MNS; ++n) {
            if (FULL || n < N) {
                const float a = r + 1 < SB ? exp2_fast(dl[r + 1] * a2[n]) : 1.f;   // a_{r+1}
                W[n] *= a;
                he[n] += W[n] * (u * BC[0][r][n]);
                G[n] = BC[1][r][n] * dv[r] + a * G[n];
            }
        }
        __builtin_amdgcn_sched_barrier(0);   // one step at a time: bounds the LDS reads in flight
    }
    const int64_t o = (b * nseg + p) * N * D + d;   // state n at o + n D
#pragma unroll
    for (int n = 0; n < MNS; ++n) {
        if (n < N) {
            hend[o + n * D] = he[n];
            gl[o + n * D] = G[n];
        }
    }
    sdl[(b * nseg + p) * D + d] = sd;
}

// 2. per (b, n, d): the adjoint entering each segment from the right.  With
// Gf_p the adjoint at segment p's first step and gl_p its part from inside
// the segment, Gf_p = F_p Gf_{p+1} + gl_p, F_p = exp(A (sum delta over p -
// delta_{t0(p)} + delta_{t0(p+1)})), walked from the last segment back; gl_p
// is replaced by exp(A delta_{t0(p+1)}) Gf_{p+1} (0 for the last segment).
// Two levels as in k_mamba_carry: CJ groups of gs segments per channel.
__device__ __forceinline__ void rcarry_body(const float *__restrict__ delta, const float *__restrict__ A,
                                            const float *__restrict__ sdl, float *__restrict__ gl, int64_t L,
                                            int64_t D, int N, int64_t nseg, int n, int64_t b, CarryLds &sh)
{
    auto &Fm = sh.G, &Em = sh.E, &Gs = sh.S;
    const int dl = threadIdx.x % CD, j = threadIdx.x / CD;
    const int64_t d = (int64_t)blockIdx.x * CD + dl;
    const bool live = d < D;
    const int64_t dd = live ? d : 0;   // masked lanes read a valid address and store nothing
    const float a2 = A[dd * N + n] * kLog2e;
    const int64_t gs = (nseg + CJ - 1) / CJ;
    const int64_t p0 = j * gs, p1 = (p0 + gs) < nseg ? (p0 + gs) : nseg;
    float *g = gl + (b * nseg * N + n) * D + dd;   // segment q at g[q N D]
    const float *sg = sdl + b * nseg * D + dd;      // segment q at sg[q D]
    const float *fd = delta + b * L * D + dd;       // step t at fd[t D]
    const int64_t es = (int64_t)N * D, fs = (int64_t)SB * D;
    auto Fof = [&](int64_t q) {   // F_q, 0 for the last segment
        return q + 1 < nseg ? exp2_fast(a2 * (sg[q * D] - fd[q * fs] + fd[(q + 1) * fs])) : 0.f;
    };
    float F = 1.f, E = 0.f;   // the group's map, composed from its last segment back
    for (int64_t q = p1 - 1; q >= p0; --q) {
        const float f = Fof(q);
        E = f * E + g[q * es];
        F = f * F;
    }
    Fm[j][dl] = F;
    Em[j][dl] = E;
    __syncthreads();
    if (j == 0) {
        float Gv = 0.f;   // nothing follows the last group
        for (int q = CJ - 1; q >= 0; --q) {
            Gs[q][dl] = Gv;   // the adjoint at the first segment after group q
            Gv = Fm[q][dl] * Gv + Em[q][dl];
        }
    }
    __syncthreads();
    float Gn = Gs[j][dl];   // Gf_{p1}
    for (int64_t q = p1 - 1; q >= p0; --q) {
        const float glq = g[q * es];
        const float hat = q + 1 < nseg ? exp2_fast(a2 * fd[(q + 1) * fs]) * Gn : 0.f;
        if (live) g[q * es] = hat;
        Gn = Fof(q) * Gn + glq;   // Gf_q
    }
}

// Both carries in one launch (they are independent; one launch instead of
// two matters at short sequences).  Grid y: states 0 .. N-1 run the forward
// carry, N .. 2N-1 the reverse one.
__global__ __launch_bounds__(CJ *CD) void k_mamba_carries(const float *__restrict__ delta,
                                                         const float *__restrict__ A, float *__restrict__ hend,
                                                         const float *__restrict__ sdl, float *__restrict__ gl,
                                                         int64_t L, int64_t D, int N, int64_t nseg)
{
    __shared__ CarryLds sh;
    const int y = blockIdx.y;   // uniform
    if (y < N) carry_body(A, hend, sdl, D, N, nseg, y, blockIdx.z, sh);
    else rcarry_body(delta, A, sdl, gl, L, D, N, nseg, y - N, blockIdx.z, sh);
}

// 3. per (b, segment): gradients of the segment's steps.  Block = BD channels x
// LPC lanes; lane j of a channel's eight holds states 2j and 2j + 1.  The
// block walks the channel chunks blockIdx.x, + gridDim.x, ... and adds up dB,
// dC over all of them in LDS.  dBC: the segment's dB / dC rows (nsplit == 1)
// or this split's partial rows [nsplit][B][L][2][N].  hin and ghat are the
// entering states and right adjoints, [B][nseg][N][D].  At most 128 VGPRs
// (4 waves per SIMD), so that two blocks (67 KiB of LDS each) share a CU.
template <bool WY>   // also y, from the recomputed states (mamba_fwd_bwd)
__global__ __launch_bounds__(BT) __attribute__((amdgpu_waves_per_eu(4))) void k_mamba_bwd_seg(
    const float *__restrict__ x, const float *__restrict__ delta, const float *__restrict__ A,
    const float *__restrict__ Bm, const float *__restrict__ Cm, const float *__restrict__ Ds,
    const float *__restrict__ dy, const float *__restrict__ hin, const float *__restrict__ ghat,
    float *__restrict__ y, float *__restrict__ dx, float *__restrict__ ddelta, float *__restrict__ dB,
    float *__restrict__ dC,
    float *__restrict__ dBCp, float *__restrict__ dApart, float *__restrict__ dDpart, int64_t L, int64_t D, int N,
    int64_t nseg, int nsplit)
{
    __shared__ __attribute__((aligned(16))) float Tw[WIN][2][BD / 2][NS];   // one window of channel-pair dB / dC terms
    __shared__ float acc[SB][2][NS];                                    // the segment's dB / dC so far
    __shared__ __attribute__((aligned(16))) float BCs[2][SB][NS];       // the segment's B, C rows
    __shared__ __attribute__((aligned(16))) float Xs[3][BD][XP];        // the chunk's x, delta, dy by channel
    const int tid = threadIdx.x, dl = tid / LPC, j = tid % LPC, n0 = 2 * j;
    const int64_t p = blockIdx.y, b = blockIdx.z;
    const int64_t t0 = p * SB, t1 = (t0 + SB) < L ? (t0 + SB) : L;
    const int nrow = (int)(t1 - t0);
    for (int i = tid; i < SB * 2 * NS; i += BT) (&acc[0][0][0])[i] = 0.f;
    for (int i = tid; i < 2 * SB * NS; i += BT) {
        const int w = i / (SB * NS), r = (i / NS) % SB, m = i % NS;
        (&BCs[0][0][0])[i] = r < nrow && m < N ? (w ? Cm : Bm)[(b * L + t0 + r) * N + m] : 0.f;
    }
    // Staging: element e = tid + k BT of a chunk's tile is step e / BD,
    // channel e % BD (a wave loads one 256-byte row); steps past the
    // sequence and channels past D are staged as 0.
    constexpr int KS = SB * BD / BT;
    const int64_t nchunk = (D + BD - 1) / BD;
    const int64_t row0 = (b * L + t0) * D;
    float stg[3][KS];
    auto fetch = [&](int64_t c) {
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            const int e = tid + k * BT, r = e / BD;
            const int64_t ch = c * BD + e % BD;
            const bool in = r < nrow && ch < D;
            const int64_t gi = row0 + (int64_t)r * D + (in ? ch : 0);
            stg[0][k] = in ? x[gi] : 0.f;
            stg[1][k] = in ? delta[gi] : 0.f;
            stg[2][k] = in ? dy[gi] : 0.f;
        }
    };
    auto put = [&]() {
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            const int e = tid + k * BT, r = e / BD, q = e % BD;
            Xs[0][q][r] = stg[0][k];
            Xs[1][q][r] = stg[1][k];
            Xs[2][q][r] = stg[2][k];
        }
    };
    fetch(blockIdx.x);
    put();
    __syncthreads();
    for (int64_t c = blockIdx.x; c < nchunk; c += nsplit) {
        const bool more = c + nsplit < nchunk;   // uniform
        const int64_t d = c * BD + dl;
        const bool dlive = d < D, live0 = dlive && n0 < N, live1 = dlive && n0 + 1 < N;
        const int64_t dd = dlive ? d : D - 1;
        const float Av0 = live0 ? A[dd * N + n0] : 0.f, Av1 = live1 ? A[dd * N + n0 + 1] : 0.f;
        const float a20 = Av0 * kLog2e, a21 = Av1 * kLog2e;
        const float dsk = Ds[dd];
        // the first segment starts from zero, and nothing enters the last from
        // the right (with one segment neither carry pass runs)
        const int64_t so = ((b * nseg + p) * N + n0) * D + dd;   // state n0; n0 + 1 at so + D
        const float S0 = live0 && p > 0 ? hin[so] : 0.f, S1 = live1 && p > 0 ? hin[so + D] : 0.f;
        const float Gh0 = live0 && p + 1 < nseg ? ghat[so] : 0.f, Gh1 = live1 && p + 1 < nseg ? ghat[so + D] : 0.f;
        const float *xr = Xs[0][dl], *dr = Xs[1][dl], *yr = Xs[2][dl];
        // dx / ddelta: lane 0 of a live channel stores at its lane offset plus
        // the row's; other lanes store at kOOB, and rows past the segment land
        // past the resource's end: the range check drops both.
        const int64_t segb = (int64_t)nrow * D * 4;   // bytes of the segment's rows
        const rsrc_t rdx = make_rsrc(dx + row0, segb), rdd = make_rsrc(ddelta + row0, segb);
        const rsrc_t ry = make_rsrc(WY ? y + row0 : dx + row0, WY ? segb : 0);
        const uint32_t lxs = j == 0 && dlive ? (uint32_t)d * 4u : kOOB, stx = (uint32_t)D * 4u;
        // h over the segment (the decays are formed again in the reverse
        // walk: keeping them too would not fit the registers).  Steps past
        // the sequence are staged as zeros, which leaves h, the adjoint
        // sums and the dB / dC terms unchanged: neither walk branches on
        // them, only the dx / ddelta stores are masked.
        float hs0[SB], hs1[SB];
        {
            float h0 = S0, h1 = S1;
#pragma unroll
            for (int r = 0; r < SB; ++r) {
                const float dlt = dr[r], u = dlt * xr[r];
                const float2 bt = *reinterpret_cast<const float2 *>(&BCs[0][r][n0]);
                h0 = exp2_fast(dlt * a20) * h0 + u * bt.x;
                h1 = exp2_fast(dlt * a21) * h1 + u * bt.y;
                hs0[r] = h0;
                hs1[r] = h1;
                if (r % 4 == 3) __builtin_amdgcn_sched_barrier(0);   // bound the LDS reads in flight
            }
        }
        // (a barrier: the tile is read again below, not kept in registers)
        __syncthreads();
        // The walk starts from the right adjoint with decay 1: padded steps
        // (delta = dy = 0) pass it down unchanged to the last real step.
        float G0 = Gh0, G1 = Gh1, an0 = 1.f, an1 = 1.f, dA0 = 0.f, dA1 = 0.f, dD = 0.f;
#pragma unroll
        for (int r = SB - 1; r >= 0; --r) {
            const float dlt = dr[r], xt = xr[r], dyt = yr[r];
            const float2 bt = *reinterpret_cast<const float2 *>(&BCs[0][r][n0]);
            const float2 ct = *reinterpret_cast<const float2 *>(&BCs[1][r][n0]);
            G0 = ct.x * dyt + an0 * G0;
            G1 = ct.y * dyt + an1 * G1;
            const float a0 = exp2_fast(dlt * a20), a1 = exp2_fast(dlt * a21);
            an0 = a0;
            an1 = a1;
            const float ah0 = a0 * (r > 0 ? hs0[r - 1] : S0), ah1 = a1 * (r > 0 ? hs1[r - 1] : S1);
            float sx = G0 * bt.x + G1 * bt.y;
            float q = G0 * (Av0 * ah0) + G1 * (Av1 * ah1);
            dA0 += G0 * dlt * ah0;
            dA1 += G1 * dlt * ah1;
            dD += dyt * xt;
            // (the empty asm keeps the sums step by step: left alone, the
            // compiler sinks them past the walk and holds every step's terms)
            asm volatile("" : "+v"(dA0), "+v"(dA1), "+v"(dD));
            // sums over the channel's eight lanes
            sx = dpp_add<kQuadXor1>(sx);
            sx = dpp_add<kQuadXor2>(sx);
            sx = dpp_add<kRowHalfMirror>(sx);
            q = dpp_add<kQuadXor1>(q);
            q = dpp_add<kQuadXor2>(q);
            q = dpp_add<kRowHalfMirror>(q);
            const uint32_t o = lxs + (uint32_t)r * stx;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(dsk * dyt + dlt * sx), rdx, o, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(q + xt * sx), rdd, o, 0, 0);
            if constexpr (WY) {   // y_t = sum_n C_t h_t + Dskip x_t: the lane's two states, then its 8 lanes
                float yv = ct.x * hs0[r] + ct.y * hs1[r];
                yv = dpp_add<kQuadXor1>(yv);
                yv = dpp_add<kQuadXor2>(yv);
                yv = dpp_add<kRowHalfMirror>(yv);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(yv + dsk * xt), ry, o, 0, 0);
            }
            // dB / dC terms, summed first over the two channels of a 16-lane
            // row (lanes 8 apart hold the same states): the even channel's
            // lanes write the pair's sums, so a window holds twice the steps
            const float u = dlt * xt;
            float tb0 = G0 * u, tb1 = G1 * u, tc0 = dyt * hs0[r], tc1 = dyt * hs1[r];
            tb0 = dpp_add<kRowRor + 8>(tb0);
            tb1 = dpp_add<kRowRor + 8>(tb1);
            tc0 = dpp_add<kRowRor + 8>(tc0);
            tc1 = dpp_add<kRowRor + 8>(tc1);
            if ((dl & 1) == 0) {
                *reinterpret_cast<float2 *>(&Tw[r % WIN][0][dl / 2][n0]) = make_float2(tb0, tb1);
                *reinterpret_cast<float2 *>(&Tw[r % WIN][1][dl / 2][n0]) = make_float2(tc0, tc1);
            }
            if (r % 2 == 0) __builtin_amdgcn_sched_barrier(0);
            if (r % WIN == 0) {
                // the window's steps r .. r + WIN - 1: sum each (step, which, n)
                // over the block's BD / 2 channel pairs, two threads per
                // column, each over half of them
                static_assert(BT == 2 * WIN * 2 * NS, "two threads per column");
                __syncthreads();
                const int col = tid / 2, part = tid % 2;   // WIN x 2 x NS columns
                const int w = col / (2 * NS), which = (col / NS) % 2, cn = col % NS;
                float s = 0.f;
#pragma unroll
                for (int k = 0; k < BD / 4; ++k) s += Tw[w][which][part * (BD / 4) + k][cn];
                s = dpp_add<kQuadXor1>(s);   // lanes 2c and 2c + 1 hold one column's halves
                if (part == 0 && r + w < nrow) acc[r + w][which][cn] += s;
                __syncthreads();
            }
            // The next chunk's tile is loaded halfway through the walk, when
            // the later steps' states no longer hold registers; it lands while
            // the rest of the walk computes (with no next chunk, this one's
            // tile is loaded again and not used).
            if (r == SB / 2) fetch(more ? c + nsplit : c);
        }
        const int64_t ao = ((b * nseg + p) * D + d) * N + n0;
        if (live0) dApart[ao] = dA0;
        if (live1) dApart[ao + 1] = dA1;
        if (j == 0 && dlive) dDpart[(b * nseg + p) * D + d] = dD;
        if (more) {   // every read of this chunk's tile is behind the last window's barrier
            put();
            __syncthreads();
        }
    }
    __syncthreads();
    for (int i = tid; i < nrow * 2 * NS; i += BT) {
        const int r = i / (2 * NS), which = (i / NS) % 2, m = i % NS;
        if (m >= N) continue;
        const float v = acc[r][which][m];
        const int64_t row = b * L + t0 + r;
        if (nsplit == 1) (which ? dC : dB)[row * N + m] = v;
        else dBCp[((blockIdx.x * (int64_t)gridDim.z * L + row) * 2 + which) * N + m] = v;
    }
}

// 4. fixed-order sums.  Element i of [dA (D N) | dDskip (D) | dB, dC rows
// (B L 2 N, only with nsplit > 1)] is the sum of Q partials M apart (Q = B
// nseg for dA and dDskip, nsplit for dB / dC).  A block takes WE elements x
// WQ slices; slice s adds partials s, s + WQ, ... in four chains, and the
// first slice adds the WQ slice sums in order: the order depends on the
// shape only.
constexpr int WE = 64, WQ = 16;
__global__ __launch_bounds__(WE *WQ) void k_mamba_wsum(const float *__restrict__ dApart,
                                                      const float *__restrict__ dDpart,
                                                      const float *__restrict__ dBCp, float *__restrict__ dA,
                                                      float *__restrict__ dD, float *__restrict__ dB,
                                                      float *__restrict__ dC, int64_t B, int64_t L, int64_t D,
                                                      int N, int64_t nseg, int nsplit)
{
    __shared__ float part[WQ][WE];
    const int e = threadIdx.x % WE, s = threadIdx.x / WE;
    const int64_t i = (int64_t)blockIdx.x * WE + e;
    const int64_t nA = D * N, nD = D, nBC = nsplit > 1 ? B * L * 2 * N : 0;
    const float *src = dApart;
    int64_t Q = 0, M = 1, k = 0;
    if (i < nA) {
        Q = B * nseg, M = nA, k = i;
    } else if (i < nA + nD) {
        src = dDpart, Q = B * nseg, M = nD, k = i - nA;
    } else if (i < nA + nD + nBC) {
        src = dBCp, Q = nsplit, M = nBC, k = i - nA - nD;
    }
    float c0 = 0.f, c1 = 0.f, c2 = 0.f, c3 = 0.f;
    int64_t q = s;
    for (; q + 3 * WQ < Q; q += 4 * WQ) {
        c0 += src[q * M + k];
        c1 += src[(q + WQ) * M + k];
        c2 += src[(q + 2 * WQ) * M + k];
        c3 += src[(q + 3 * WQ) * M + k];
    }
    for (; q < Q; q += WQ) c0 += src[q * M + k];
    part[s][e] = (c0 + c1) + (c2 + c3);
    __syncthreads();
    if (s != 0) return;
    float t = 0.f;
#pragma unroll
    for (int u = 0; u < WQ; ++u) t += part[u][e];
    if (i < nA) {
        dA[i] = t;
    } else if (i < nA + nD) {
        dD[i - nA] = t;
    } else if (i < nA + nD + nBC) {
        const int64_t row = k / (2 * N), which = (k / N) % 2, m = k % N;
        (which ? dC : dB)[row * N + m] = t;
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

// The backward; with with_y (mamba_fwd_bwd) also the forward's output, from
// the states the gradient kernel recomputes.
static int mamba_bwd_impl(const mamba_shape *shape, const float *x, const float *delta, const float *A,
                          const float *Bm, const float *Cm, const float *Ds, const float *dy, float *y, float *dx,
                          float *ddelta, float *dA, float *dB, float *dC, float *dD, void *workspace,
                          size_t workspace_bytes, void *stream, bool with_y)
{
    int rc = mamba_check_shape(shape);
    if (rc != SSD_OK) return rc;
    const mamba_shape &s = *shape;
    if (s.L > 65535 * kMambaBwdSeg) return SSD_ERR_UNSUPPORTED;
    if (!dA || !dD) return SSD_ERR_NULL;   // dA, dDskip have elements even when B or L is 0
    const MambaBwdPlan P = mamba_bwd_plan(shape, device_cus());
    const bool work = s.B > 0 && s.L > 0;
    if (work && (!x || !delta || !A || !Bm || !Cm || !Ds || !dy || !dx || !ddelta || !dB || !dC))
        return SSD_ERR_NULL;
    if (work && with_y && !y) return SSD_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(y) & 3u) != 0) return SSD_ERR_ALIGN;
    const void *ptrs[] = {x, delta, A, Bm, Cm, Ds, dy, dx, ddelta, dA, dB, dC, dD};
    for (const void *q : ptrs)
        if ((reinterpret_cast<uintptr_t>(q) & 3u) != 0) return SSD_ERR_ALIGN;
    if (workspace_bytes < P.total) return SSD_ERR_WORKSPACE;
    if (P.total > 0) {
        if (!workspace) return SSD_ERR_NULL;
        if (!aligned16(workspace)) return SSD_ERR_ALIGN;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *w = static_cast<char *>(workspace);
    float *hend = reinterpret_cast<float *>(w + P.hend), *sdl = reinterpret_cast<float *>(w + P.sdl);
    float *gl = reinterpret_cast<float *>(w + P.gl), *dAp = reinterpret_cast<float *>(w + P.dApart);
    float *dDp = reinterpret_cast<float *>(w + P.dDpart), *dBCp = reinterpret_cast<float *>(w + P.dBC);
    const int N = (int)s.N;
    const int64_t nseg = P.nseg;
    if (work) {
        // 1. every segment from zero, both ways
        const dim3 g1((unsigned)((s.D + MB - 1) / MB), (unsigned)nseg, (unsigned)s.B);
        if (N == MNS)
            launch(nullptr, -1, k_mamba_seg_ends<true>, g1, dim3(MB), st, x, delta, A, Bm, Cm, dy, hend, sdl, gl, s.L,
                   s.D, N, nseg);
        else
            launch(nullptr, -1, k_mamba_seg_ends<false>, g1, dim3(MB), st, x, delta, A, Bm, Cm, dy, hend, sdl, gl,
                   s.L, s.D, N, nseg);
        if (launch_status() != SSD_OK) return SSD_ERR_DEVICE;
        // 2. the state entering every segment, and the adjoint entering it from the right
        if (nseg > 1) {
            const dim3 g2((unsigned)((s.D + CD - 1) / CD), (unsigned)(2 * N), (unsigned)s.B);
            launch(nullptr, -1, k_mamba_carries, g2, dim3(CJ * CD), st, delta, A, hend, (const float *)sdl, gl, s.L,
                   s.D, N, nseg);
            if (launch_status() != SSD_OK) return SSD_ERR_DEVICE;
        }
        // 3. the gradients of every segment (and with y, the forward's output
        // from the states recomputed on the way)
        const dim3 g3((unsigned)P.nsplit, (unsigned)nseg, (unsigned)s.B);
        if (with_y)
            launch(nullptr, -1, k_mamba_bwd_seg<true>, g3, dim3(BT), st, x, delta, A, Bm, Cm, Ds, dy,
                   (const float *)hend, (const float *)gl, y, dx, ddelta, dB, dC, dBCp, dAp, dDp, s.L, s.D, N, nseg,
                   P.nsplit);
        else
            launch(nullptr, -1, k_mamba_bwd_seg<false>, g3, dim3(BT), st, x, delta, A, Bm, Cm, Ds, dy,
                   (const float *)hend, (const float *)gl, y, dx, ddelta, dB, dC, dBCp, dAp, dDp, s.L, s.D, N, nseg,
                   P.nsplit);
        if (launch_status() != SSD_OK) return SSD_ERR_DEVICE;
    }
    // 4. fixed-order sums (dA, dDskip are zero when B or L is 0)
    const int64_t tot = s.D * s.N + s.D + (P.nsplit > 1 ? s.B * s.L * 2 * s.N : 0);
    launch(nullptr, -1, k_mamba_wsum, dim3((unsigned)((tot + WE - 1) / WE)), dim3(WE * WQ), st, (const float *)dAp,
           (const float *)dDp, (const float *)dBCp, dA, dD, dB, dC, s.B, s.L, s.D, N, work ? nseg : 0, P.nsplit);
    return launch_status();
}

extern "C" int mamba_bwd(const mamba_shape *shape, const float *x, const float *delta, const float *A,
                         const float *Bm, const float *Cm, const float *Ds, const float *dy, float *dx,
                         float *ddelta, float *dA, float *dB, float *dC, float *dD, void *workspace,
                         size_t workspace_bytes, void *stream)
{
    return mamba_bwd_impl(shape, x, delta, A, Bm, Cm, Ds, dy, nullptr, dx, ddelta, dA, dB, dC, dD, workspace,
                          workspace_bytes, stream, false);
}

extern "C" int mamba_fwd_bwd(const mamba_shape *shape, const float *x, const float *delta, const float *A,
                             const float *Bm, const float *Cm, const float *Ds, const float *dy, float *y,
                             float *dx, float *ddelta, float *dA, float *dB, float *dC, float *dD,
                             void *workspace, size_t workspace_bytes, void *stream)
{
    return mamba_bwd_impl(shape, x, delta, A, Bm, Cm, Ds, dy, y, dx, ddelta, dA, dB, dC, dD, workspace,
                          workspace_bytes, stream, true);
}
