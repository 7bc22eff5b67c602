// The output kernel (K2 + K5) on chunk pairs for gfx950: the state scan
// stores S_in of even chunks only, and the odd chunk of each pair takes its
// inter-chunk term from the even chunk's state.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

// ---------------------------------------------------------------------------
// Output of the chunk pair (2m, 2m + 1), 128 positions, for every head of
// one group.  With b the within-chunk cumulative log-decay of each chunk,
// b_L its value at the even chunk's last position and S = S_in(2m):
//
//   even rows i:  y_i = e^{b_i} q_i S + sum_{j <= i, same chunk} (q_i . k_j) e^{b_i - b_j} v_j
//   odd rows i:   y_i = e^{b_L + b_i} q_i S
//                     + sum_{j in the even chunk} (q_i . k_j) e^{b_i + (b_L - b_j)} v_j
//                     + sum_{j <= i, same chunk} (q_i . k_j) e^{b_i - b_j} v_j
//
// since S_in(2m + 1) = e^{b_L} S + sum_j e^{b_L - b_j} k_j v_j^T.  The pair
// is one chunk of 128 positions for the intra term; the decay exponents are
// formed from the chunk-local b (every difference b_i - b_j, and every
// cross exponent b_i + (b_L - b_j), is a sum of non-positive terms of the
// size of the decay itself, not a difference of two large cumulative sums).
//
// Eight waves.  Wave w owns the 32 rows rb(w) of the pair (rb = 0, 0, 1, 1,
// 3, 3, 2, 2, so that the two waves of each SIMD have 80 + 128 or 96 + 112
// MFMAs per step) and, per step, the 32 output columns cb = w % 2 of a
// 64-column half of dv; a head takes dv / 64 steps.  On
// v_mfma_f32_32x32x2f32:
//   * Q[rb] (32 x dk), the A operand of Q S, stays in registers for the unit;
//   * K Q^T is formed once per unit (the 10 causal 32 x 32 tiles (kb, rb),
//     kb <= rb) and kept in LDS in the accumulator layout, which is the
//     A-operand layout of P: register r of lane (kh, i) holds key
//     32 kb + 8 (r / 4) + 4 kh + r % 4 of query row 32 rb + i.  Per head
//     the waves form P = (K Q^T)^T o D into LDS in the same layout, five
//     register groups each;
//   * a step's S half (dk x 64) and V half (128 x 64) are staged in LDS,
//     row stride 72 (rows 4 apart, which the two lane halves read, fall in
//     different banks).
// The next step's tiles are loaded into registers during the Q S MFMAs; in
// the last step of a unit, the next unit's first step, and its Q and K
// tiles during the P V MFMAs (the Q rows in registers are dead by then).
constexpr int NTW2 = 512;
constexpr int PR = 2 * CH;   // positions per unit

template <int DKP, int DVP>
struct PairCfg {
    static_assert(DVP == 64 || DVP == 128, "64 or 128 columns of dv");
    static constexpr int NSH = DVP / 64;                          // steps per head
    static constexpr int LS = 64 + 8;                             // S half and V half row stride
    static constexpr int LDK = DKP + 4;                           // Q and K row stride (set-up)
    static constexpr int SN = DKP * LS;                           // S half
    static constexpr int VN = PR * LS;                            // V half
    static constexpr int XN = (SN + VN) > PR * LDK ? (SN + VN) : PR * LDK;
    static constexpr int SPH = DKP * 64 / 4 / NTW2;               // float4 / thread, S half
    static constexpr int VPH = PR * 64 / 4 / NTW2;                // float4 / thread, V half
    static constexpr int NL = SPH + VPH + 1;                      // loads / thread / step
    static constexpr int NQ = DKP / 8;                            // float4 of a Q row per lane
    static constexpr int QPER = PR * DKP / 4 / NTW2;              // float4 / thread, one 128 x dk tile
    static_assert(SPH >= 1 && QPER >= 1, "tile sizes");
};

// Tile (kb, rb), kb <= rb, of the 10 causal 32 x 32 tiles of the pair.
__device__ __forceinline__ int pair_tile(int kb, int rb) { return rb * (rb + 1) / 2 + kb; }

template <int DKP, int DVP, bool VEC, bool EXD>
__global__ __launch_bounds__(NTW2) void k_pair_output(const float *__restrict__ q, const float *__restrict__ k,
                                                      const float *__restrict__ v, const float *__restrict__ la,
                                                      const float *__restrict__ states, float *__restrict__ y,
                                                      int G, int H, int64_t T, int dk, int dv, int64_t NC,
                                                      int64_t Epad, int hpb, int64_t nunits)
{
    using Cfg = PairCfg<DKP, DVP>;
    if constexpr (EXD) {
        dk = DKP;
        dv = DVP;
        Epad = (int64_t)DKP * DVP;
    }
    constexpr int NSH = Cfg::NSH, LS = Cfg::LS, LDK = Cfg::LDK, SPH = Cfg::SPH, VPH = Cfg::VPH, NL = Cfg::NL;
    constexpr int NQ = Cfg::NQ, QPER = Cfg::QPER;
    __shared__ __attribute__((aligned(16))) float KQ[10 * 1024];   // K Q^T, [tile][r][lane]
    __shared__ __attribute__((aligned(16))) float PS[10 * 1024];   // P of the head; set-up: split partial sums
    __shared__ __attribute__((aligned(16))) float XS[Cfg::XN];     // S half + V half; set-up: Q, then K
    __shared__ __attribute__((aligned(16))) float bs[PR];          // chunk-local b of each position
    __shared__ __attribute__((aligned(16))) float eb[PR];          // e^{b_i} (even), e^{b_L + b_i} (odd)
    __shared__ __attribute__((aligned(16))) float wx[CH];          // b_L - b_j of the even chunk
    float *const SS = XS, *const VV = XS + Cfg::SN;

    const int NP = (int)((NC + 1) / 2);
    const int hpg_all = H / G, nsplit = (hpg_all + hpb - 1) / hpb;
    struct Unit {
        int64_t m, bg, bh0;
        int hpg, rows;
        bool live;
    };
    // unit ((b G + g) nsplit + split) NP + m: heads [split hpb, ...) of group g at pair m
    auto unit_of = [&](int64_t u) {
        Unit U;
        U.live = u < nunits;
        if (!U.live) u = 0;
        U.m = u % NP;
        const int64_t bgs = u / NP;
        const int split = (int)(bgs % nsplit);
        U.bg = bgs / nsplit;
        const int g = (int)(U.bg % G);
        const int64_t b = U.bg / G;
        U.hpg = U.live ? min(hpb, hpg_all - split * hpb) : 0;
        U.bh0 = b * H + (int64_t)g * hpg_all + (int64_t)split * hpb;
        U.rows = (int)((T - U.m * PR) < PR ? (T - U.m * PR) : PR);
        return U;
    };
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    // rows of wave w: 0, 0, 1, 1, 3, 3, 2, 2
    const int rbw = (wave >> 1) == 0 ? 0 : (wave >> 1) == 1 ? 1 : (wave >> 1) == 2 ? 3 : 2;
    const int cb = wave & 1;
    const int64_t E = (int64_t)dk * dv;

    // Step loads: S half and V half of head step `step`, and for the first
    // step of a head (waves 0 and 1) the log_alpha of both chunks.
    float4 sbuf[SPH], vbuf[VPH];
    float la0 = 0.f, la1 = 0.f;
    auto issue = [&](const Unit &U, int step, int tid, int u) {
        const int hh = step / NSH, half = step % NSH;
        const bool live = hh < U.hpg;
        const int64_t bh = U.bh0 + (live ? hh : 0);
        if (u < SPH + VPH) {
            const bool isv = u >= SPH;
            const int e = isv ? u - SPH : u;
            const int r = f4_row<16, NTW2>(tid, e), c4 = f4_col<16>(tid);
            if (!isv) {
                const rsrc_t sr = make_rsrc(states + (bh * NC + 2 * U.m) * Epad, live ? E * 4 : 0);
                sbuf[e] = load4(sr, (uint32_t)(r * dv + 64 * half), c4, dv - 64 * half, true, VEC);
            } else {
                const rsrc_t vr = make_rsrc(v + (bh * T + U.m * PR) * dv, live ? (int64_t)U.rows * dv * 4 : 0);
                vbuf[e] = load4(vr, (uint32_t)(r * dv + 64 * half), c4, dv - 64 * half, true, VEC);
            }
        } else {
            // waves 0 and 1 load the 128 log_alpha values of the head's first step
            const bool first = half == 0 && wave < 2;
            const rsrc_t lr = make_rsrc(la + (U.bh0 + (live ? hh : 0)) * T + U.m * PR,
                                        (live && first) ? (int64_t)U.rows * 4 : 0);
            la0 = gload1(lr, (uint32_t)(tid & 63) * 4u);
            la1 = gload1(lr, (uint32_t)(64 + (tid & 63)) * 4u);
        }
    };
    float4 qkb[2][QPER];
    auto issue_qk = [&](const Unit &U, int tid, int j) {
        const int which = j / QPER, e = j % QPER;
        const rsrc_t r = make_rsrc((which ? k : q) + (U.bg * T + U.m * PR) * dk, U.live ? (int64_t)U.rows * dk * 4 : 0);
        constexpr int Q4 = DKP / 4;
        const int row = f4_row<Q4, NTW2>(tid, e), c4 = f4_col<Q4>(tid);
        qkb[which][e] = load4(r, (uint32_t)(row * dk), c4, dk, true, VEC);
    };
    // stage the step's tiles; for a head's first step also b, e^b, b_L - b
    auto stage = [&](int tid, bool first) {
#pragma unroll
        for (int u = 0; u < SPH; ++u) {
            const int r = f4_row<16, NTW2>(tid, u), c4 = f4_col<16>(tid);
            *reinterpret_cast<float4 *>(SS + r * LS + c4) = sbuf[u];
        }
#pragma unroll
        for (int u = 0; u < VPH; ++u) {
            const int r = f4_row<16, NTW2>(tid, u), c4 = f4_col<16>(tid);
            *reinterpret_cast<float4 *>(VV + r * LS + c4) = vbuf[u];
        }
        if (first && wave < 2) {
            const int l = tid & 63;
            const float b0 = chunk_cumsum(la0);
            const float bL = readlane_f(b0, 63);
            if (wave == 0) {
                bs[l] = b0;
                eb[l] = expf(b0);
                wx[l] = bL - b0;
            } else {
                const float b1 = chunk_cumsum(la1);
                bs[CH + l] = b1;
                eb[CH + l] = expf(bL + b1);
            }
        }
    };

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
        const int64_t m = U.m, bh0 = U.bh0;
        const int hpg = U.hpg, rows = U.rows;

        // ---- unit set-up: Q rows in registers, K Q^T into LDS, first step staged
        float4 qa[NQ];   // Q[32 rb + i][8m + 4kh .. 8m + 4kh + 3] in lane (kh, i)
        {
            const int tid = threadIdx.x, lane = tid & 63, cl = lane & 31, kh = lane >> 5;
            regs_to_lds<PR, DKP, NTW2, QPER, LDK>(tid, qkb[0], XS);
            block_sync();
#pragma unroll
            for (int mm = 0; mm < NQ; ++mm)
                qa[mm] = *reinterpret_cast<const float4 *>(XS + (32 * rbw + cl) * LDK + 8 * mm + 4 * kh);
            block_sync();   // Q read before K overwrites it
            regs_to_lds<PR, DKP, NTW2, QPER, LDK>(tid, qkb[1], XS);
            block_sync();
            // K Q^T tiles (kb, rb) of this wave over dk range [m0, m1) (float4 steps):
            // waves 0/1: (0,0) halves; 2: (0,1); 3: (1,1); 4: (0,3), (1,3); 5: (2,3), (3,3);
            // 6: (0,2) and half 0 of (2,2); 7: (1,2) and half 1 of (2,2).
            auto ktile = [&](f32x16 &acc, int kb, auto m0_c, auto m1_c) {
                constexpr int m0 = decltype(m0_c)::value, m1 = decltype(m1_c)::value;
                const float *ka = XS + (32 * kb + cl) * LDK + 4 * kh;
                float4 xb[2];
                xb[m0 & 1] = *reinterpret_cast<const float4 *>(ka + 8 * m0);
#pragma unroll
                for (int mm = m0; mm < m1; ++mm) {
                    {
                        if (mm + 1 < m1) xb[(mm + 1) & 1] = *reinterpret_cast<const float4 *>(ka + 8 * (mm + 1));
                        const float4 x = xb[mm & 1], yq = qa[mm];
                        acc = mfma32(x.x, yq.x, acc);
                        acc = mfma32(x.y, yq.y, acc);
                        acc = mfma32(x.z, yq.z, acc);
                        acc = mfma32(x.w, yq.w, acc);
                    }
                }
            };
            auto put = [&](float *dst, const f32x16 &acc) {
#pragma unroll
                for (int r = 0; r < 16; ++r) dst[r * 64 + lane] = acc[r];
            };
            f32x16 a0 = zero16(), a1 = zero16();
            if (wave == 0) {
                ktile(a0, 0, IntC<0>{}, IntC<NQ / 2>{});
                put(PS + 0 * 1024, a0);
            } else if (wave == 1) {
                ktile(a0, 0, IntC<NQ / 2>{}, IntC<NQ>{});
                put(PS + 1 * 1024, a0);
            } else if (wave == 2) {
                ktile(a0, 0, IntC<0>{}, IntC<NQ>{});
                put(KQ + pair_tile(0, 1) * 1024, a0);
            } else if (wave == 3) {
                ktile(a0, 1, IntC<0>{}, IntC<NQ>{});
                put(KQ + pair_tile(1, 1) * 1024, a0);
            } else if (wave == 4) {
                ktile(a0, 0, IntC<0>{}, IntC<NQ>{});
                ktile(a1, 1, IntC<0>{}, IntC<NQ>{});
                put(KQ + pair_tile(0, 3) * 1024, a0);
                put(KQ + pair_tile(1, 3) * 1024, a1);
            } else if (wave == 5) {
                ktile(a0, 2, IntC<0>{}, IntC<NQ>{});
                ktile(a1, 3, IntC<0>{}, IntC<NQ>{});
                put(KQ + pair_tile(2, 3) * 1024, a0);
                put(KQ + pair_tile(3, 3) * 1024, a1);
            } else if (wave == 6) {
                ktile(a0, 0, IntC<0>{}, IntC<NQ>{});
                ktile(a1, 2, IntC<0>{}, IntC<NQ / 2>{});
                put(KQ + pair_tile(0, 2) * 1024, a0);
                put(PS + 2 * 1024, a1);
            } else {
                ktile(a0, 1, IntC<0>{}, IntC<NQ>{});
                ktile(a1, 2, IntC<NQ / 2>{}, IntC<NQ>{});
                put(KQ + pair_tile(1, 2) * 1024, a0);
                put(PS + 3 * 1024, a1);
            }
            block_sync();   // K read, tiles and partial sums written
            {
                // the two split tiles: (0,0) = parts 0 + 1, (2,2) = parts 2 + 3
                const int half = tid >> 8, e4 = (tid & 255) * 4;
                const float4 x = *reinterpret_cast<const float4 *>(PS + (2 * half) * 1024 + e4);
                const float4 z = *reinterpret_cast<const float4 *>(PS + (2 * half + 1) * 1024 + e4);
                *reinterpret_cast<float4 *>(KQ + (half ? pair_tile(2, 2) : pair_tile(0, 0)) * 1024 + e4) =
                    make_float4(x.x + z.x, x.y + z.y, x.z + z.z, x.w + z.w);
            }
            stage(tid, true);
            block_sync();
        }

        const int nstep = hpg * NSH;
        // One step: P for a head's first step, then Q S, then P V.  The last
        // step of the unit loads the next unit's first step and its Q and K.
        auto one_step = [&](auto last_c, int st) {
            constexpr bool last = decltype(last_c)::value;
            int tid = threadIdx.x;
            asm volatile("" : "+v"(tid));
            const int lane = tid & 63, cl = lane & 31, kh = lane >> 5;
            const int hh = st / NSH, half = st % NSH;
            const bool live = hh < hpg;
            const int64_t bh = bh0 + (live ? hh : 0);
            const Unit &Ul = last ? Un : U;
            const int sl = last ? 0 : st + 1;

            if (half == 0) {
                // P = (K Q^T)^T o D: register groups 5 w .. 5 w + 4 of the 40
                // (tile t = group / 4, group a = group % 4 of its 16 registers)
#pragma unroll
                for (int gi = 0; gi < 5; ++gi) {
                    const int gidx = 5 * wave + gi, t = gidx >> 2, a = gidx & 3;
                    // tile t = (kb, rb): rb = the largest with rb (rb + 1) / 2 <= t
                    const int rbt = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
                    const int kbt = t - rbt * (rbt + 1) / 2;
                    const int i = 32 * rbt + cl;
                    const float bi = bs[i];
                    const bool cross = rbt >= 2 && kbt < 2;
                    const float4 bj4 = *reinterpret_cast<const float4 *>((cross ? wx : bs) + 32 * kbt + 8 * a + 4 * kh);
                    const float bjs[4] = {bj4.x, bj4.y, bj4.z, bj4.w};
                    const bool diag = kbt == rbt;
                    const int lim = cl - 4 * kh;   // diagonal tile: key j <= row i is 8a + e <= lim
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * a + e;
                        const float kq = KQ[t * 1024 + r * 64 + lane];
                        const float x = cross ? bi + bjs[e] : bi - bjs[e];
                        const bool ok = !diag || 8 * a + e <= lim;
                        PS[t * 1024 + r * 64 + lane] = kq * __expf(ok ? x : -INFINITY);
                    }
                }
            }

            // Q S over dk; MFMA group mm issues the next step's loads [mm NL / NQ, (mm + 1) NL / NQ)
            f32x16 acc = zero16();
            {
                const float *sb = SS + 4 * kh * LS + 32 * cb + cl;
                float bq[2][4];
#pragma unroll
                for (int s = 0; s < 4; ++s) bq[0][s] = sb[s * LS];
#pragma unroll
                for (int mm = 0; mm < NQ; ++mm) {
                    if (mm + 1 < NQ) {
#pragma unroll
                        for (int s = 0; s < 4; ++s) bq[(mm + 1) & 1][s] = sb[(8 * (mm + 1) + s) * LS];
                    }
#pragma unroll
                    for (int u = mm * NL / NQ; u < (mm + 1) * NL / NQ; ++u) issue(Ul, sl, tid, u);
                    acc = mfma32(qa[mm].x, bq[mm & 1][0], acc);
                    acc = mfma32(qa[mm].y, bq[mm & 1][1], acc);
                    acc = mfma32(qa[mm].z, bq[mm & 1][2], acc);
                    acc = mfma32(qa[mm].w, bq[mm & 1][3], acc);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            block_sync();   // P of the head formed
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const float4 e = *reinterpret_cast<const float4 *>(eb + 32 * rbw + 8 * a + 4 * kh);
                acc[4 * a] *= e.x;
                acc[4 * a + 1] *= e.y;
                acc[4 * a + 2] *= e.z;
                acc[4 * a + 3] *= e.w;
            }
            // P V over the keys of tiles kb <= rb
            {
                const float *vb = VV + 4 * kh * LS + 32 * cb + cl;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    if (kb <= rbw) {
                        const float *pr = PS + pair_tile(kb, rbw) * 1024 + lane;
                        float bv[16], p[16];
#pragma unroll
                        for (int a = 0; a < 4; ++a) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                bv[4 * a + e] = vb[(32 * kb + 8 * a + e) * LS];
                                p[4 * a + e] = pr[(4 * a + e) * 64];
                            }
                        }
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            // the next unit's Q and K, one load per MFMA of the first tile
                            if constexpr (last) {
                                if (kb == 0 && r < 2 * QPER) issue_qk(Un, tid, r);
                            }
                            acc = mfma32(p[r], bv[r], acc);
                        }
                    }
                }
            }
            {
                const rsrc_t yb = make_rsrc(y + (bh * T + m * PR) * dv, live ? (int64_t)rows * dv * 4 : 0);
                const int n = 64 * half + 32 * cb + cl;
                const uint32_t base = n < dv ? (uint32_t)((32 * rbw + 4 * kh) * dv + n) * 4u : kOOB;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    gstore1_nt(yb, base + (uint32_t)(8 * (r / 4) + r % 4) * (uint32_t)(dv * 4), acc[r]);
            }
            block_sync();   // S half, V half, P and decays read before the next writes
            if constexpr (!last) {
                stage(tid, (st + 1) % NSH == 0);
                block_sync();
            }
        };
        for (int st = 0; st < nstep - 1; ++st) one_step(BoolC<false>{}, st);
        one_step(BoolC<true>{}, nstep - 1);
        U = Un;
    }
}

int run_pair_output(const Problem &P, const float *q, const float *k, const float *v, const float *la, float *y,
                    hipStream_t st)
{
    const ssd_shape &s = P.s;
    const int64_t NP = (P.L.NC + 1) / 2;
    int hsplit = 1, hpb = 1;
    head_split(&s, NP, P.cus, &hsplit, &hpb);
    const int64_t nunits = s.B * s.G * hsplit * NP;
    const int64_t grid = nunits < P.cus ? nunits : P.cus;
    auto go = [&](auto vp_c) {
        constexpr int VP = decltype(vp_c)::value ? 128 : 64;
        auto body = [&](auto kp_c, auto ve_c, auto ex_c) {
            constexpr int KP = decltype(kp_c)::value;
            constexpr bool VE = decltype(ve_c)::value, EXD = decltype(ex_c)::value;
            launch(P.timer, KID_OUTPUT, k_pair_output<KP, VP, VE, EXD>, dim3((unsigned)grid), dim3(NTW2), st, q, k, v,
                   la, P.states, y, (int)s.G, (int)s.H, s.T, (int)s.dk, (int)s.dv, P.L.NC, P.L.Epad, hpb, nunits);
        };
        auto modes = [&](auto kp_c) {
            if (P.exact) body(kp_c, BoolC<true>{}, BoolC<true>{});
            else if (P.vec) body(kp_c, BoolC<true>{}, BoolC<false>{});
            else body(kp_c, BoolC<false>{}, BoolC<false>{});
        };
        if (P.DKP == 32) modes(IntC<32>{});
        else if (P.DKP == 64) modes(IntC<64>{});
        else modes(IntC<128>{});
    };
    if (P.DVP == 128) go(BoolC<true>{});
    else go(BoolC<false>{});
    return launch_status();
}

}  // namespace ssd
