// The per-chunk cumulative log-decay (K1) and the fused chunk-state and
// state-pass scan (K3 + K4, and the reverse pass of the backward) for gfx950.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

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
// K1: per-chunk cumulative log-decay, turned into what the scan's loader
// waves apply.  One wave per (b, h, chunk), lane t at position 64 c + t
// (positions past T read log_alpha = 0, so they repeat the last b):
//   wts[bh][c][t]      = e^{b_L - b_t}   (forward: weight of k_t in X_c)
//   wts[bh][c][64 + t] = e^{b_t}         (reverse: weight of dy_t in Z_c)
//   cdec[bh][c]        = e^{b_L}         (decay of the state over the chunk)
// b comes from chunk_cumsum, as in every other kernel, so all of them see
// the same b bitwise.
constexpr int NTP = 256;
__global__ __launch_bounds__(NTP) void k_chunk_decay(const float *__restrict__ la, float *__restrict__ wts,
                                                     float *__restrict__ cdec, int64_t T, int64_t NC, int64_t nwaves)
{
    const int64_t wv = (int64_t)blockIdx.x * (NTP / 64) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (wv >= nwaves) return;   // whole waves only
    const int64_t bh = wv / NC, c = wv - bh * NC;
    const int64_t rows = (T - c * CH) < CH ? (T - c * CH) : CH;
    const float x = gload1(make_rsrc(la + bh * T + c * CH, rows * 4), (uint32_t)lane * 4u);
    const float b = chunk_cumsum(x);
    const float bL = readlane_f(b, 63);
    float *w = wts + wv * (2 * CH);
    w[lane] = __expf(bL - b);
    w[CH + lane] = __expf(b);
    if (lane == 0) cdec[wv] = expf(bL);
}

constexpr int TI = 32;
constexpr int NTS = 512;        // 4 compute + 4 loader waves

template <int DKP, int DVP, bool VEC, int TJ, int CPS, bool EXD>
__global__ __launch_bounds__(NTS) void k_state_scan(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ dy, const float *__restrict__ h0, const float *__restrict__ wts,
    const float *__restrict__ cdec, float *__restrict__ states, float *__restrict__ dstates, float *__restrict__ dh0,
    float *__restrict__ ends, int G, int H, int64_t T, int dk, int dv, int64_t NC, int64_t Epad, int64_t per_dir,
    int dir0, int nseg, int64_t seg_len, int spar)
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
    // segment p of the chunk sequence (in scan order), then (b h, tile)
    const int64_t per_seg = per_dir / nseg, BHn = per_seg / NTILE;
    const int64_t p = rem / per_seg;
    const int64_t rem2 = rem - p * per_seg;
    const int64_t bh = rem2 / NTILE;
    const int tile = (int)(rem2 - bh * NTILE);
    const int64_t n0 = p * seg_len;                                     // first chunk of the segment
    const int64_t nch = (NC - n0) < seg_len ? (NC - n0) : seg_len;      // its chunks
    const int i0 = (tile / NTJ) * TI, j0 = (tile % NTJ) * TJ;
    const int h = (int)(bh % H);
    const int64_t b = bh / H;
    const int g = h / (H / G);
    const int64_t E = (int64_t)dk * dv;
    const int64_t NSC = (nch + CPS - 1) / CPS;       // steps holding real chunks
    const int64_t NS = (NSC + PD - 1) / PD * PD;      // steps, rounded up
    const int wave = threadIdx.x >> 6;

    if (wave >= 4) {
        // ---------------- loader waves
        const int lt = threadIdx.x - 256;
        const float *Asrc = (dir == 0 ? k : q) + (b * G + g) * T * dk;   // row 0, column 0
        const float *Bsrc = (dir == 0 ? v : dy) + bh * T * dv;
        const float *wb = wts + bh * NC * (2 * CH) + (dir == 0 ? 0 : CH);   // this direction's weights
        const rsrc_t dr = make_rsrc(cdec + bh * NC, NC * 4);
        const int lima = dk - i0, limb = dv - j0;
        struct Stage {
            float4 a[APER], b[BPER];
            float w[APER], dec;   // decay weights of the A rows, e^{b_L} of the chunk
            bool live;
        };
        Stage stg[PD][CPS];
        // operands of chunk n of the scan order; chunks past the end load zeros
        auto prefetch = [&](Stage &S, int64_t n) {
            const bool live = n < nch;
            const int64_t c = live ? (dir == 0 ? n0 + n : NC - 1 - (n0 + n)) : 0;
            const int rows = (int)((T - c * CH) < CH ? (T - c * CH) : CH);
            const rsrc_t ab = make_rsrc(Asrc + c * CH * dk, live ? (int64_t)rows * dk * 4 : 0);
            const rsrc_t bb = make_rsrc(Bsrc + c * CH * dv, live ? (int64_t)rows * dv * 4 : 0);
            const rsrc_t wr = make_rsrc(wb + c * (2 * CH), live ? CH * 4 : 0);
#pragma unroll
            for (int u = 0; u < APER; ++u) {
                const int r = f4_row<TI / 4, NLT>(lt, u), c4 = f4_col<TI / 4>(lt);
                const bool ok = A4 % NLT == 0 || r < CH;
                S.a[u] = load4(ab, (uint32_t)(r * dk + i0), c4, lima, ok, VEC);
                S.w[u] = gload1(wr, ok ? (uint32_t)r * 4u : kOOB);
            }
#pragma unroll
            for (int u = 0; u < BPER; ++u) {
                const int r = f4_row<TJ / 4, NLT>(lt, u), c4 = f4_col<TJ / 4>(lt);
                S.b[u] = load4(bb, (uint32_t)(r * dv + j0), c4, limb, B4 % NLT == 0 || r < CH, VEC);
            }
            // a vector load: a scalar one would be waited for right here
            S.dec = gload1(dr, live ? (uint32_t)c * 4u : kOOB);
            S.live = live;
        };
        // stage S into LDS half `buf`, slot cc; the rows of the A tile (TI
        // wide, the narrower one) are scaled by the decay weights
        auto stage = [&](const Stage &S, int buf, int cc) {
#pragma unroll
            for (int u = 0; u < APER; ++u) {
                const int r = f4_row<TI / 4, NLT>(lt, u), c4 = f4_col<TI / 4>(lt);
                if (A4 % NLT == 0 || r < CH) {
                    const float w = S.w[u];
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
            // chunks past the end leave the state as it is
            if (lt == 0) decs[buf][cc] = S.live ? S.dec : 1.f;
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
        // the forward pass starts at h0, the reverse at 0, later segments at 0
        const rsrc_t hr = make_rsrc(h0 + bh * E, (dir == 0 && p == 0) ? E * 4 : 0);
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
        // The chunks' decays are read before their operands: LDS reads
        // return in order, and the state is scaled by the decay before the
        // first MFMA, so a decay read last would hold that MFMA until every
        // operand read of the chunk had returned.
        float dec[CPS];
#pragma unroll
        for (int cc = 0; cc < CPS; ++cc) dec[cc] = decs[buf][cc];
        __builtin_amdgcn_sched_barrier(0);
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
            const float decay = dec[cc];
            // slab[c] = S (state entering the chunk in this direction); no-op chunks store nothing
            const int64_t n = s * CPS + cc;
            // spar 1 (2): the forward direction stores the states of even (odd) chunks only
            const bool live = n < nch && (spar == 0 || dir != 0 || (int)((n0 + n) & 1) == spar - 1);
            const rsrc_t dst =
                make_rsrc(slab + (live ? (dir == 0 ? n0 + n : NC - 1 - (n0 + n)) : 0) * Epad, live ? E * 4 : 0);
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
    if (nseg > 1) {
        // the state leaving the segment, for the fix-up pass (ends[dl][p][bh])
        const rsrc_t er = make_rsrc(ends + ((dl * nseg + p) * BHn + bh) * Epad, E * 4);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
#pragma unroll
            for (int r = 0; r < 4; ++r) gstore1(er, soff(u, r), acc[u][r]);
        }
    } else if (dir == 1) {
        const rsrc_t hr = make_rsrc(dh0 + bh * E, E * 4);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
#pragma unroll
            for (int r = 0; r < 4; ++r) gstore1(hr, soff(u, r), acc[u][r]);
        }
    }
}

// Fix-up of a segmented scan, in two passes.  Segment p of the chunk
// sequence (scan order) was scanned from a zero state, the first from the
// true initial state, and ends[dl][p][bh] holds the state leaving it.  With
// S_p the true state entering segment p, A_p the decay over segment p and
// D(n) the decay from the segment's start to chunk n,
//     S_1 = ends[0],  S_{p+1} = ends[p] + A_p S_p,   state(n) = local state(n) + D(n) S_p.
// Pass 1, per (direction, b h) and block of state elements: first D and A
// (the products of the chunk decays within each segment), one wave per
// segment taking 64 chunks at a time with an inclusive product scan across
// the lanes (the DPP steps of scan64 with products, and 1 where a step has
// no source lane) shifted by one lane; the first block of the (direction,
// b h) writes D to segd for pass 2.  Then one thread per state element walks
// the segments in order and overwrites ends[p] with S_{p+1}, so that
// ends[p - 1] holds the state entering segment p; for the reverse direction
// it also writes dh0, the state leaving the last segment.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_mul(float x)
{
    return x * __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(x), CTRL, ROWS, 0xf, false));
}
constexpr int NTF = 256;
__global__ __launch_bounds__(NTF) void k_seg_carry(float *__restrict__ ends, float *__restrict__ segd,
                                                   const float *__restrict__ cdec, float *__restrict__ dh0,
                                                   int64_t BH, int64_t NC, int64_t E, int64_t Epad, int nseg,
                                                   int64_t seg_len, int dir0)
{
    __shared__ float Ap[kMaxSegs];
    const int64_t dlbh = blockIdx.y, bh = dlbh % BH;
    const int dl = (int)(dlbh / BH), dir = dir0 + dl;
    const float *dc = cdec + bh * NC;
    auto chunk = [&](int64_t n) { return dir == 0 ? n : NC - 1 - n; };
    {
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        float *sd = segd + dlbh * NC;
        for (int p = wave; p < nseg; p += NTF / 64) {
            const int64_t n0 = p * seg_len, n1 = (n0 + seg_len) < NC ? (n0 + seg_len) : NC;
            float carry = 1.f;
            for (int64_t base = n0; base < n1; base += 64) {
                const int64_t n = base + lane;
                float x = n < n1 ? dc[chunk(n)] : 1.f;
                x = dpp_mul<kRowShr + 1>(x);
                x = dpp_mul<kRowShr + 2>(x);
                x = dpp_mul<kRowShr + 4>(x);
                x = dpp_mul<kRowShr + 8>(x);
                x = dpp_mul<kRowBcast15, 0xa>(x);
                x = dpp_mul<kRowBcast31, 0xc>(x);   // lane l: product over lanes 0..l
                const float ex = __int_as_float(
                    __builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(x), kWaveShr1, 0xf, 0xf, false));
                if (blockIdx.x == 0 && n < n1) sd[n] = carry * ex;
                carry *= readlane_f(x, 63);
            }
            if (lane == 0) Ap[p] = carry;
        }
    }
    __syncthreads();
    const int64_t e = (int64_t)blockIdx.x * NTF + threadIdx.x;
    if (e >= E) return;
    float *en = ends + ((int64_t)dl * nseg * BH + bh) * Epad + e;   // en[p BH Epad]: segment p
    float S = en[0];   // S_1
    for (int p = 1; p < nseg - 1; ++p) {
        S = en[(int64_t)p * BH * Epad] + Ap[p] * S;
        en[(int64_t)p * BH * Epad] = S;   // S_{p+1}
    }
    if (dir == 1) dh0[bh * E + e] = en[(int64_t)(nseg - 1) * BH * Epad] + Ap[nseg - 1] * S;
}

// Pass 2: one thread per 4 consecutive state elements of each chunk of
// segments p >= 1 adds D(n) S_p.  blockIdx.x = (n - seg_len) neb + element
// block (neb blocks of 4 NTF elements per state), blockIdx.y: direction and
// b h.
__global__ __launch_bounds__(NTF) void k_seg_apply(float *__restrict__ states, float *__restrict__ dstates,
                                                   const float *__restrict__ ends, const float *__restrict__ segd,
                                                   int64_t BH, int64_t NC, int E, int64_t Epad, int nseg,
                                                   int64_t seg_len, int dir0, int neb, bool vec, int spar)
{
    const int64_t xb = blockIdx.x / (unsigned)neb;
    const int e4 = (int)((blockIdx.x - xb * neb) * NTF + threadIdx.x) * 4;
    const int64_t n = seg_len + xb;
    const int64_t dlbh = blockIdx.y, bh = dlbh % BH;
    const int dl = (int)(dlbh / BH), dir = dir0 + dl;
    if (spar && dir == 0 && (int)(n & 1) != spar - 1) return;   // a chunk whose state is not stored
    const int64_t p = n / seg_len;
    const float d = segd[dlbh * NC + n];
    const rsrc_t cr = make_rsrc(ends + (((int64_t)dl * nseg + p - 1) * BH + bh) * Epad, (int64_t)E * 4);
    const float4 c = load4(cr, 0, e4, E, true, vec);
    float *slab = (dir == 0 ? states : dstates) + (bh * NC + (dir == 0 ? n : NC - 1 - n)) * Epad;
    const rsrc_t sr = make_rsrc(slab, (int64_t)E * 4);
    const float4 x = load4(sr, 0, e4, E, true, vec);
    const float o[4] = {x.x + d * c.x, x.y + d * c.y, x.z + d * c.z, x.w + d * c.w};
    if (vec) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, make_float4(o[0], o[1], o[2], o[3])), sr,
                                               e4 < E ? (uint32_t)e4 * 4u : kOOB, 0, 0);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) gstore1(sr, e4 + i < E ? (uint32_t)(e4 + i) * 4u : kOOB, o[i]);
    }
}

// The fused state scan over the directions in `dirs` (see ssd_launch.h).
int run_scan(const Problem &P, int dirs, bool prep, StoreSet store, const float *q, const float *k, const float *v,
             const float *dy, const float *la, const float *h0, float *dh0, hipStream_t st)
{
    const ssd_shape &s = P.s;
    const int64_t BH = s.B * s.H;
    if (prep) {
        const int64_t nw = BH * P.L.NC;
        launch(P.timer, KID_AUX, k_chunk_decay, dim3((unsigned)((nw + 3) / 4)), dim3(NTP), st, la, P.wts, P.cdec,
               s.T, P.L.NC, nw);
        if (launch_status() != SSD_OK) return SSD_ERR_DEVICE;
    }
    // Two chunks per step when there is at most one block per CU (the paired
    // tiles fill most of a CU's LDS); otherwise one.  State tiles are 32 x 64
    // (32 x dv for dv < 64): wider tiles re-read fewer operand tiles but
    // halve the number of independent sequential chains per CU, which
    // measured slower.  Small grids take narrow tiles and segments (ScanPlan).
    const int ndir = dirs == 3 ? 2 : 1, dir0 = dirs == 2 ? 1 : 0;
    const int64_t tiles_k = BH * (P.DKP / TI);
    const ScanPlan plan = scan_plan(&s, ndir, P.cus);
    const int spar = (int)store;
    const bool narrow = plan.narrow;
    const bool pair = plan.blocks <= P.cus;
    const int kid = dirs == 1 ? KID_SCAN : dirs == 2 ? KID_SCANR : KID_SCAN2;
    auto run = [&](auto tj_c) {
        SSD_DISPATCH(P, ({
            constexpr int TJ = decltype(tj_c)::value ? 32 : (VP < 64 ? VP : 64);
            const int64_t per_dir = tiles_k * (VP / TJ) * plan.nseg;
            const dim3 grid((unsigned)(ndir * per_dir)), blk(NTS);
            if (pair)
                launch(P.timer, kid, k_state_scan<KP, VP, VE, TJ, 2, EXD>, grid, blk, st, q, k, v, dy, h0, P.wts, P.cdec,
                       P.states, P.dstates, dh0, P.ends, (int)s.G, (int)s.H, s.T, (int)s.dk, (int)s.dv, P.L.NC,
                       P.L.Epad, per_dir, dir0, plan.nseg, plan.seg_len, spar);
            else
                launch(P.timer, kid, k_state_scan<KP, VP, VE, TJ, 1, EXD>, grid, blk, st, q, k, v, dy, h0, P.wts, P.cdec,
                       P.states, P.dstates, dh0, P.ends, (int)s.G, (int)s.H, s.T, (int)s.dk, (int)s.dv, P.L.NC,
                       P.L.Epad, per_dir, dir0, plan.nseg, plan.seg_len, spar);
        }));
    };
    if (narrow) run(BoolC<true>{});
    else run(BoolC<false>{});
    if (plan.nseg > 1) {
        // ndir * BH is small here: a segmented plan fills at most the CUs
        if (launch_status() != SSD_OK) return SSD_ERR_DEVICE;
        const int64_t E = s.dk * s.dv;
        launch(P.timer, KID_AUX, k_seg_carry, dim3((unsigned)((E + NTF - 1) / NTF), (unsigned)(ndir * BH)), dim3(NTF),
               st, P.ends, P.segd, (const float *)P.cdec, dh0, BH, P.L.NC, E, P.L.Epad, plan.nseg,
               plan.seg_len, dir0);
        if (launch_status() != SSD_OK) return SSD_ERR_DEVICE;
        const int64_t nfix = P.L.NC - plan.seg_len;   // chunks of segments 1 ..
        const int neb = (int)((E + 4 * NTF - 1) / (4 * NTF));
        launch(P.timer, KID_AUX, k_seg_apply, dim3((unsigned)(nfix * neb), (unsigned)(ndir * BH)), dim3(NTF), st,
               P.states, P.dstates, (const float *)P.ends, (const float *)P.segd, BH, P.L.NC, (int)E, P.L.Epad,
               plan.nseg, plan.seg_len, dir0, neb, E % 4 == 0, spar);
    }
    return launch_status();
}

}  // namespace ssd
