// The output kernel (K2 + K5) for gfx950: the intra-chunk decay-masked
// Q K^T V product and the inter-chunk term diag(e^b) Q S_in, with the
// per-chunk cumulative log-decay (K1) formed in-block.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

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
                                                      const float *__restrict__ v, const float *__restrict__ la,
                                                      const float *__restrict__ states, float *__restrict__ y,
                                                      int G, int H, int64_t T, int dk, int dv, int64_t NC,
                                                      int64_t Epad, int hpb, int64_t nunits)
{
    using Cfg = OutCfg<DKP, DVP>;
    if constexpr (EXD) {   // dk == DKP, dv == DVP: index arithmetic on constants
        dk = DKP;
        dv = DVP;
        Epad = (int64_t)DKP * DVP;
    }
    constexpr int NCT = Cfg::NCT, HPS = Cfg::HPS, LS = Cfg::LS, LDK = Cfg::LDK;
    constexpr int SPH = Cfg::SPH, VPH = Cfg::VPH, NL = Cfg::NL, NQ = Cfg::NQ, NQQ = Cfg::NQQ;
    constexpr int QPER = Cfg::QPER;
    // S_in tiles; Q, K and then the K Q^T partial sums at set-up
    __shared__ __attribute__((aligned(16))) float SX[Cfg::SXN];
    __shared__ __attribute__((aligned(16))) float VS[Cfg::VN];
    __shared__ __attribute__((aligned(16))) float bs[HPS * CH];
    __shared__ __attribute__((aligned(16))) float eb[HPS * CH];
    __shared__ __attribute__((aligned(16))) float PS[Cfg::PN];   // [head][tile rt + jt][r][lane]

    // Unit ((b G + g) nsplit + split) NC + c takes heads [split hpb, split hpb + hpg)
    // of group g at chunk c.  The block walks units blockIdx.x, + gridDim.x, ...
    const int hpg_all = H / G, nsplit = (hpg_all + hpb - 1) / hpb;
    struct Unit {
        int64_t c, bg, bh0;
        int hpg, rows;
        bool live;
    };
    auto unit_of = [&](int64_t u) {
        Unit U;
        U.live = u < nunits;
        if (!U.live) u = 0;
        U.c = u % NC;
        const int64_t bgs = u / NC;
        const int split = (int)(bgs % nsplit);
        U.bg = bgs / nsplit;
        const int g = (int)(U.bg % G);
        const int64_t b = U.bg / G;
        U.hpg = U.live ? min(hpb, hpg_all - split * hpb) : 0;   // heads of the unit
        U.bh0 = b * H + (int64_t)g * hpg_all + (int64_t)split * hpb;
        U.rows = (int)((T - U.c * CH) < CH ? (T - U.c * CH) : CH);
        return U;
    };
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int rt = wave >> 2, slot = wave & 3;
    const int hs = slot / NCT, ct = slot % NCT;
    const int64_t E = (int64_t)dk * dv;

    // A step's S_in and V tiles and log_alpha values, in registers, loaded
    // one step ahead (the first step of the next unit during the last step
    // of this one).  Heads past the group's last, and units past the last,
    // load zeros, so no load is conditional and the compiler's count of loads
    // in flight stays exact.  issue() issues load u of the NL loads of head
    // step `step` of unit U.
    float4 sbuf[HPS][SPH], vbuf[HPS][VPH];
    float lapre = 0.f;   // log_alpha of position tid % 64 of head `wave` of the step
    auto issue = [&](const Unit &U, int step, int tid, int u) {
        if (u < NL - 1) {
            const bool isv = u >= HPS * SPH;
            const int uu = isv ? u - HPS * SPH : u;
            const int h2 = isv ? uu / VPH : uu / SPH, e = isv ? uu % VPH : uu % SPH;
            const int hh = step * HPS + h2;
            const bool live = hh < U.hpg;
            const int64_t bh = U.bh0 + (live ? hh : 0);
            // float4 tid + e NTW of the tile: row tid / (DVP/4) + e NTW / (DVP/4)
            const int r = (int)((unsigned)tid / (DVP / 4)) + e * (NTW / (DVP / 4));
            const int c4 = (int)((unsigned)tid % (DVP / 4)) * 4;
            if (!isv) {
                const rsrc_t sr = make_rsrc(states + (bh * NC + U.c) * Epad, live ? E * 4 : 0);
                sbuf[h2][e] = load4(sr, (uint32_t)(r * dv), c4, dv, (DKP * DVP / 4) % NTW == 0 || r < DKP, VEC);
            } else {
                const rsrc_t vr = make_rsrc(v + (bh * T + U.c * CH) * dv, live ? (int64_t)U.rows * dv * 4 : 0);
                vbuf[h2][e] = load4(vr, (uint32_t)(r * dv), c4, dv, true, VEC);
            }
        } else {
            // wave w < HPS loads head w's 64 log_alpha values
            const int hh = step * HPS + (wave < HPS ? wave : 0);
            const bool live = hh < U.hpg && wave < HPS;
            lapre = gload1(make_rsrc(la + (U.bh0 + (live ? hh : 0)) * T + U.c * CH, live ? (int64_t)U.rows * 4 : 0),
                           (uint32_t)(tid & 63) * 4u);
        }
    };
    // Q and K tiles of a unit in registers (float4 j of 2 QPER: Q, then K)
    float4 qkb[2][QPER];
    auto issue_qk = [&](const Unit &U, int tid, int j) {
        const int which = j / QPER, e = j % QPER;
        const rsrc_t r = make_rsrc((which ? k : q) + (U.bg * T + U.c * CH) * dk, U.live ? (int64_t)U.rows * dk * 4 : 0);
        constexpr int Q4 = DKP / 4;
        const int row = f4_row<Q4, NTW>(tid, e), c4 = f4_col<Q4>(tid);
        qkb[which][e] = load4(r, (uint32_t)(row * dk), c4, dk, (CH * Q4) % NTW == 0 || row < CH, VEC);
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
            const float b = chunk_cumsum(lapre);
            bs[wave * CH + (tid & 63)] = b;
            eb[wave * CH + (tid & 63)] = expf(b);
        }
    };

    // The first unit's Q, K and first-step tiles.
    Unit U = unit_of(blockIdx.x);
    {
        const int tid = threadIdx.x;
#pragma unroll
        for (int j = 0; j < 2 * QPER; ++j) issue_qk(U, tid, j);
#pragma unroll
        for (int u = 0; u < NL; ++u) issue(U, 0, tid, u);
    }
    for (int64_t ui = blockIdx.x; ui < nunits; ui += gridDim.x) {
        const Unit Un = unit_of(ui + gridDim.x);
        const int64_t c = U.c, bh0 = U.bh0;
        const int hpg = U.hpg, rows = U.rows;

        // ---- unit set-up: Q rows in registers, K Q^T, the first step staged.
        float4 qa[NQ];   // Q[32 rt + i][8m + 4kh .. 8m + 4kh + 3] in lane (kh, i)
        f32x16 kqt[2];   // (K Q^T)[32 jt + row(r)][32 rt + i], jt <= rt
        {
            const int tid = threadIdx.x, lane = tid & 63, cl = lane & 31, kh = lane >> 5;
            regs_to_lds<CH, DKP, NTW, QPER, LDK>(tid, qkb[0], SX);
            regs_to_lds<CH, DKP, NTW, QPER, LDK>(tid, qkb[1], SX + CH * LDK);
            block_sync();
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
                            const float4 x = *reinterpret_cast<const float4 *>(
                                SX + ((((rt + jt) * 4 + qq) * 4 + a) * 64 + lane) * 4);
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
        // A step is instantiated per row block, so that with rt a constant the
        // causal tests of P fold (the tile below the diagonal needs none) and
        // the P V loop has no branch, and for the last step of the unit, which
        // loads the next unit's first step and (once the Q rows in registers
        // are dead) its Q and K tiles, and stages nothing.
        auto one_step = [&](auto rt_c, auto last_c, int st) {
            constexpr int rt = decltype(rt_c)::value ? 1 : 0;
            constexpr bool last = decltype(last_c)::value;
            {
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
                const Unit &Ul = last ? Un : U;
                const int sl = last ? 0 : st + 1;

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
                        for (int u = m * NL / NQ; u < (m + 1) * NL / NQ; ++u) issue(Ul, sl, tid, u);
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
                            for (int r = 0; r < 16; ++r) {
                                // the next unit's Q and K, one load per two MFMAs of the first tile
                                if constexpr (last) {
                                    if (jt == 0 && r % 2 == 0 && r / 2 < 2 * QPER) issue_qk(Un, tid, r / 2);
                                }
                                acc = mfma32(p[r], bv[r], acc);
                            }
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
                block_sync();   // S_in, V and decay reads done before the next writes
                if constexpr (!last) {
                    stage(tid);
                    block_sync();
                }
            }
        };
        auto steps = [&](auto rt_c) {
            for (int st = 0; st < nstep - 1; ++st) one_step(rt_c, BoolC<false>{}, st);
            one_step(rt_c, BoolC<true>{}, nstep - 1);
        };
        if (rt) steps(BoolC<true>{});
        else steps(BoolC<false>{});
        U = Un;
    }
}
int run_output(const Problem &P, const float *q, const float *k, const float *v, const float *la, float *y,
               hipStream_t st)
{
    if (P.pair) return run_pair_output(P, q, k, v, la, y, st);
    const ssd_shape &s = P.s;
    // one block per CU at most (a block fills most of a CU's LDS); each block
    // walks its units and prefetches the next unit's tiles during the last
    // step of the current one
    const int64_t nunits = s.B * s.G * P.L.hsplit * P.L.NC;
    const int64_t grid = nunits < P.cus ? nunits : P.cus;
    SSD_DISPATCH(P, launch(P.timer, KID_OUTPUT, k_chunk_output<KP, VP, VE, EXD>, dim3((unsigned)grid), dim3(NTW), st,
                           q, k, v, la, P.states, y, (int)s.G, (int)s.H, s.T, (int)s.dk, (int)s.dv, P.L.NC, P.L.Epad,
                           P.L.hpb, nunits));
    return launch_status();
}

}  // namespace ssd
