// The gradient kernel (B3 + B4) for gfx950: per (b, g, chunk), the five
// gradient terms of every head of the group and dlog_alpha, with the
// per-chunk cumulative log-decay (K1) formed in-block; and the fixed-order
// sum of split partial dq, dk.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

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
    const float *__restrict__ dy, const float *__restrict__ la,
    const float *__restrict__ states, const float *__restrict__ dstates, float *__restrict__ dq,
    float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ dla, int G, int H, int64_t T, int dk_,
    int dv_, int64_t NC, int64_t Epad, int hpb, int64_t pstride, int64_t nunits)
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

    // Unit ((b G + g) nsplit + split) NC + c takes heads [split hpb, split hpb + hpg)
    // of group g at chunk c.  The block walks units blockIdx.x, + gridDim.x, ...
    // and loads the next unit's first-head operands during its last head.
    const int hpg_all = H / G, nsplit = (hpg_all + hpb - 1) / hpb;
    struct Unit {
        int64_t c, bg, bh0;
        int hpg, rows, split;
        bool live;
    };
    auto unit_of = [&](int64_t u) {
        Unit U;
        U.live = u < nunits;
        if (!U.live) u = 0;
        U.c = u % NC;
        const int64_t bgs = u / NC;
        U.split = (int)(bgs % nsplit);
        U.bg = bgs / nsplit;
        const int g = (int)(U.bg % G);
        const int64_t b = U.bg / G;
        U.hpg = U.live ? min(hpb, hpg_all - U.split * hpb) : 0;   // heads of the unit
        U.bh0 = b * H + (int64_t)g * hpg_all + (int64_t)U.split * hpb;
        U.rows = (int)((T - U.c * CH) < CH ? (T - U.c * CH) : CH);
        return U;
    };
    // the current unit (set at the top of each unit)
    int64_t c = 0, bg = 0, bh0 = 0;
    int hpg = 0, rows = 0;
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
    float lapre = 0.f;   // log_alpha of position tid % 64 of the next head
    float blpre = 0.f;   // its chunk total b_L, once staged

    auto load_a1 = [&](const Unit &Ux, int hh, int tid, int m) {   // float4 m of the wave's A rows of head hh
        const bool live = hh < Ux.hpg;
        const int64_t bh = Ux.bh0 + (live ? hh : 0);
        const float *src = (grp ? v : dy) + (bh * T + Ux.c * CH) * dv_;
        const rsrc_t r = make_rsrc(src, live ? (int64_t)Ux.rows * dv_ * 4 : 0);
        const int lane = tid & 63, cl = lane & 31, kh = lane >> 5;
        ar[m] = load4(r, (uint32_t)((32 * rt + cl) * dv_), 8 * m + 4 * kh, dv_, true, VEC);
    };
    // float4 u of one slab of S_in and of dS_out
    auto load_slab1 = [&](Slab &p, const Unit &Ux, int hh, int ks, int tid, int u) {
        const bool live = hh < Ux.hpg;
        const int64_t off = ((Ux.bh0 + (live ? hh : 0)) * NC + Ux.c) * Epad;
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
    auto spread_ld = [&](const Unit &Ux, int hh, int tid, int s) {
        if (s < SPER) load_slab1(p0, Ux, hh, 0, tid, s);
        else if (NKS > 1 && s < 2 * SPER) load_slab1(pn, Ux, hh, 1, tid, s - SPER);
    };
    auto load_slab = [&](Slab &p, const Unit &Ux, int hh, int ks, int tid) {
#pragma unroll
        for (int u = 0; u < SPER; ++u) load_slab1(p, Ux, hh, ks, tid, u);
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
    auto load_b = [&](const Unit &Ux, int hh, int tid) {
        const bool live = hh < Ux.hpg;
        const int64_t bh = Ux.bh0 + (live ? hh : 0);
        lapre = gload1(make_rsrc(la + bh * T + Ux.c * CH, live ? (int64_t)Ux.rows * 4 : 0),
                       (uint32_t)(tid & 63) * 4u);
    };
    // every wave scans the head's log_alpha (so each holds b_L), wave 0 stages b
    auto stage_b = [&](int tid) {
        const float b = chunk_cumsum(lapre);
        blpre = readlane_f(b, 63);
        if (tid < CH) {
            bs[tid] = b;
            eb[tid] = expf(b);
            el[tid] = (tid < rows) ? expf(blpre - b) : 0.f;
        }
    };

    // The first unit's first-head operands.
    Unit U = unit_of(blockIdx.x);
    {
        const int tid = threadIdx.x;
#pragma unroll
        for (int m = 0; m < NA; ++m) load_a1(U, 0, tid, m);
        load_slab(p0, U, 0, 0, tid);
        if (NKS > 1) load_slab(pn, U, 0, 1, tid);
        load_b(U, 0, tid);
    }
    for (int64_t ui = blockIdx.x; ui < nunits; ui += gridDim.x) {
    const Unit Un = unit_of(ui + gridDim.x);
    c = U.c;
    bg = U.bg;
    bh0 = U.bh0;
    hpg = U.hpg;
    rows = U.rows;
    // ---- unit set-up: Q, K in LDS; Q K^T; the first head's operands staged.
    float fro_next;
    {
        const int tid = threadIdx.x, lane = tid & 63, cl = lane & 31, kh = lane >> 5;
        {
            float4 qb[QPER], kb[QPER];
            const int64_t tb = (int64_t)rows * dk_ * 4;
            tile_to_regs<CH, DKP, NTB, QPER>(tid, qb, make_rsrc(q + (bg * T + c * CH) * dk_, tb), dk_, VEC);
            tile_to_regs<CH, DKP, NTB, QPER>(tid, kb, make_rsrc(k + (bg * T + c * CH) * dk_, tb), dk_, VEC);
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
        // the last head loads the next unit's first head, and stages nothing
        const bool lasth = hh == hpg - 1;
        const Unit &Ux = lasth ? Un : U;
        const int hx = lasth ? 0 : hh + 1;
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
                        if (ks + 2 < NKS) load_slab1(pn, U, hh, ks + 2, tid, m >> 1);
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
                    for (int l = 0; l < LPG; ++l) load_a1(Ux, hx, tid, (m - m0) * LPG + l);
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
        load_b(Ux, hx, tid);
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
                            spread_ld(Ux, hx, tid, f);
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
                        spread_ld(Ux, hx, tid, f - 16 * RT);
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
        if (!lasth) {
            fro_next = store_slab(p0, 0, tid);
            if (NKS > 1) fro_next += store_slab(pn, 1, tid);
            stage_b(tid);
            block_sync();
        }
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
        // dq and dk: the split's partial sums over its heads (pstride = 0 without a split)
        float *dqu = dq + U.split * pstride, *dku = dk + U.split * pstride;
        const rsrc_t rq = make_rsrc(dqu + (bg * T + c * CH) * dk_, tb), rk = make_rsrc(dku + (bg * T + c * CH) * dk_, tb);
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
    U = Un;
    }   // units
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
int run_grads(const Problem &P, const float *q, const float *k, const float *v, const float *dy, const float *la,
              float *dq, float *dk, float *dv, float *dla, hipStream_t st)
{
    const ssd_shape &s = P.s;
    // With a head split the gradient kernel writes each split's dq and dk
    // partial sums to the workspace, and k_sum_splits adds them up.
    const int hs = P.L.hsplit;
    const int64_t nqk = s.B * s.G * s.T * s.dk;
    float *pq = hs > 1 ? P.parts : dq, *pk = hs > 1 ? P.parts + hs * P.L.nqk_pad : dk;
    const int64_t pstride = hs > 1 ? P.L.nqk_pad : 0;
    // one block per CU at most (a block fills most of a CU's LDS); each block
    // walks its units, loading the next unit's first head during its last
    const int64_t nunits = s.B * s.G * hs * P.L.NC;
    const int64_t grid = nunits < P.cus ? nunits : P.cus;
    SSD_DISPATCH(P, launch(P.timer, KID_GRADS, k_bwd_grads<KP, VP, VE, EXD>, dim3((unsigned)grid), dim3(NTB), st, q,
                           k, v, dy, la, P.states, P.dstates, pq, pk, dv, dla, (int)s.G, (int)s.H, s.T, (int)s.dk,
                           (int)s.dv, P.L.NC, P.L.Epad, P.L.hpb, pstride, nunits));
    if (hs > 1) {
        if (launch_status() != SSD_OK) return SSD_ERR_DEVICE;
        const int64_t nb = (nqk + NTH - 1) / NTH;
        const dim3 grid((unsigned)(nb < 4096 ? nb : 4096));
        launch(P.timer, KID_AUX, k_sum_splits, grid, dim3(NTH), st, dq, (const float *)pq, hs, pstride, nqk);
        launch(P.timer, KID_AUX, k_sum_splits, grid, dim3(NTH), st, dk, (const float *)pk, hs, pstride, nqk);
    }
    return launch_status();
}

}  // namespace ssd
