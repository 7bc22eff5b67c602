/*
 * ssd_oracle.c -- fp64 CPU oracle for the scalar-decay SSD scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU product path
 * never calls it, links it or falls back to it, and it shares no code,
 * header or constant with the GPU path.
 *
 * What is computed (plain definition, no chunking).  For every batch b and
 * head h, with g = h / (H/G) the group whose q and k the head reads:
 *
 *     S_{-1} = h0[b,h]                                   (dk x dv)
 *     S_t    = exp(la[b,h,t]) * S_{t-1} + k[b,g,t] v[b,h,t]^T
 *     y[b,h,t] = S_t^T q[b,g,t]                           (dv)
 *
 * The benchmark pages (kernel_ssd_cpu.json / kernel_ssd_gpu.json) fix the
 * tensor set and layouts through their byte counts: in every "chunked" fwd
 * record xla_arg_mb equals q[B,G,T,dk] + k[B,G,T,dk] + v[B,H,T,dv] +
 * log_alpha[B,H,T] + h0[B,H,dk,dv] in float32 and xla_out_mb equals
 * y[B,H,T,dv] alone (no final state).  The pages' "scan" implementation is
 * the per-step form of the recurrence above; the pages print no formula, so
 * the recurrence is the standard definition of this scan.  The fwd_bwd
 * records list exactly five gradients (rel_err_grads keys q, k, v,
 * log_alpha, h0).  The loss is read as L = sum_t dy_t . y_t for a given
 * upstream gradient dy.
 *
 * Backward (reverse-mode adjoint of the recurrence, derived by hand):
 *
 *     Gbar_t  = q_t dy_t^T + exp(la_{t+1}) Gbar_{t+1},   Gbar_{T-1} = q dy^T
 *     dq_t^h  = S_t dy_t         dk_t^h = Gbar_t v_t      dv_t = Gbar_t^T k_t
 *     dla_t   = exp(la_t) <Gbar_t, S_{t-1}>_F             dh0 = exp(la_0) Gbar_0
 *     dq[b,g,t] = sum over the heads h of g (ascending h) of dq_t^h, same for dk.
 *
 * All arithmetic is IEEE double, inputs are given as doubles (callers
 * promote float32 inputs exactly).  The only liberty taken with the plain
 * definition is memory: the backward keeps S_t every 64 steps and
 * recomputes the states in between with the same operations in the same
 * order, so the recomputed values are bitwise those of the forward sweep.
 * Work is split over (b, h) pairs with OpenMP; each pair's arithmetic is
 * sequential, so the result does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_CKPT 64

static int check_shape(int64_t B, int64_t G, int64_t H, int64_t T, int64_t dk, int64_t dv)
{
    if (B < 0 || G < 1 || H < 1 || T < 0 || dk < 1 || dv < 1) return 1;
    if (H % G != 0) return 1;
    return 0;
}

int ssd_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One recurrence step: S <- a*S + k v^T. */
static void step_state(double *S, double a, const double *kt, const double *vt, int64_t dk, int64_t dv)
{
    for (int64_t i = 0; i < dk; ++i) {
        double *row = S + i * dv;
        const double ki = kt[i];
        for (int64_t j = 0; j < dv; ++j) row[j] = a * row[j] + ki * vt[j];
    }
}

/*
 * Forward.  y: [B,H,T,dv].  If states_in is not NULL it receives, for every
 * c in [0, ceil(T/chunk)), the state entering step c*chunk, i.e.
 * S_{c*chunk-1} (S_{-1} = h0): layout [B,H,NC,dk,dv].  Returns 0 on success.
 */
int ssd_oracle_fwd(int64_t B, int64_t G, int64_t H, int64_t T, int64_t dk, int64_t dv,
                   const double *q, const double *k, const double *v,
                   const double *la, const double *h0, double *y,
                   double *states_in, int64_t chunk)
{
    if (check_shape(B, G, H, T, dk, dv)) return 1;
    if (states_in && chunk < 1) return 1;
    const int64_t hpg = H / G;
    const int64_t NC = states_in ? (T + chunk - 1) / chunk : 0;
    int err = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const int64_t b = bh / H, h = bh % H, g = h / hpg;
        double *S = (double *)malloc(sizeof(double) * dk * dv);
        if (!S) {
#pragma omp atomic write
            err = 2;
            continue;
        }
        memcpy(S, h0 + bh * dk * dv, sizeof(double) * dk * dv);
        for (int64_t t = 0; t < T; ++t) {
            if (states_in && t % chunk == 0)
                memcpy(states_in + (bh * NC + t / chunk) * dk * dv, S, sizeof(double) * dk * dv);
            const double a = exp(la[bh * T + t]);
            const double *kt = k + ((b * G + g) * T + t) * dk;
            const double *qt = q + ((b * G + g) * T + t) * dk;
            const double *vt = v + (bh * T + t) * dv;
            step_state(S, a, kt, vt, dk, dv);
            double *yt = y + (bh * T + t) * dv;
            for (int64_t j = 0; j < dv; ++j) yt[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i) {
                const double qi = qt[i];
                const double *row = S + i * dv;
                for (int64_t j = 0; j < dv; ++j) yt[j] += row[j] * qi;
            }
        }
        free(S);
    }
    return err;
}

/*
 * Backward for the loss L = sum_{b,h,t} dy[b,h,t] . y[b,h,t].
 * Outputs: dq, dk [B,G,T,dk]; dv [B,H,T,dv]; dla [B,H,T]; dh0 [B,H,dk,dv].
 * Returns 0 on success.
 */
int ssd_oracle_bwd(int64_t B, int64_t G, int64_t H, int64_t T, int64_t dk, int64_t dv,
                   const double *q, const double *k, const double *v,
                   const double *la, const double *h0, const double *dy,
                   double *dq, double *dkk, double *dvv, double *dla, double *dh0)
{
    if (check_shape(B, G, H, T, dk, dv)) return 1;
    const int64_t hpg = H / G;
    const int64_t nseg = (T + ORACLE_CKPT - 1) / ORACLE_CKPT;
    /* per-head dq and dk before the group sum */
    double *dqh = (double *)calloc((size_t)(B * H * T * dk) + 1, sizeof(double));
    double *dkh = (double *)calloc((size_t)(B * H * T * dk) + 1, sizeof(double));
    if (!dqh || !dkh) {
        free(dqh);
        free(dkh);
        return 2;
    }
    int err = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const int64_t b = bh / H, h = bh % H, g = h / hpg;
        const int64_t E = dk * dv;
        double *S = (double *)malloc(sizeof(double) * E);
        double *Gb = (double *)malloc(sizeof(double) * E);
        double *ckpt = (double *)malloc(sizeof(double) * E * (nseg + 1));
        double *seg = (double *)malloc(sizeof(double) * E * ORACLE_CKPT);
        if (!S || !Gb || !ckpt || !seg) {
#pragma omp atomic write
            err = 2;
            free(S);
            free(Gb);
            free(ckpt);
            free(seg);
            continue;
        }
        const double *qb = q + (b * G + g) * T * dk;
        const double *kb = k + (b * G + g) * T * dk;
        const double *vb = v + bh * T * dv;
        const double *lab = la + bh * T;
        const double *dyb = dy + bh * T * dv;

        /* Forward sweep: checkpoints and dq^h_t = S_t dy_t. */
        memcpy(S, h0 + bh * E, sizeof(double) * E);
        for (int64_t t = 0; t < T; ++t) {
            if (t % ORACLE_CKPT == 0) memcpy(ckpt + (t / ORACLE_CKPT) * E, S, sizeof(double) * E);
            step_state(S, exp(lab[t]), kb + t * dk, vb + t * dv, dk, dv);
            double *o = dqh + (bh * T + t) * dk;
            const double *dyt = dyb + t * dv;
            for (int64_t i = 0; i < dk; ++i) {
                double acc = 0.0;
                const double *row = S + i * dv;
                for (int64_t j = 0; j < dv; ++j) acc += row[j] * dyt[j];
                o[i] = acc;
            }
        }

        /* Reverse sweep, one checkpoint segment at a time. */
        for (int64_t i = 0; i < E; ++i) Gb[i] = 0.0;
        for (int64_t s = nseg - 1; s >= 0; --s) {
            const int64_t t0 = s * ORACLE_CKPT;
            const int64_t t1 = (t0 + ORACLE_CKPT < T) ? t0 + ORACLE_CKPT : T;
            /* recompute S_t for t in [t0, t1) from the checkpoint */
            memcpy(S, ckpt + s * E, sizeof(double) * E);
            for (int64_t t = t0; t < t1; ++t) {
                step_state(S, exp(lab[t]), kb + t * dk, vb + t * dv, dk, dv);
                memcpy(seg + (t - t0) * E, S, sizeof(double) * E);
            }
            for (int64_t t = t1 - 1; t >= t0; --t) {
                const double anext = (t + 1 < T) ? exp(lab[t + 1]) : 0.0;
                const double *qt = qb + t * dk;
                const double *kt = kb + t * dk;
                const double *vt = vb + t * dv;
                const double *dyt = dyb + t * dv;
                for (int64_t i = 0; i < dk; ++i) {
                    double *row = Gb + i * dv;
                    const double qi = qt[i];
                    for (int64_t j = 0; j < dv; ++j) row[j] = qi * dyt[j] + anext * row[j];
                }
                /* dk^h_t = Gbar_t v_t */
                double *dko = dkh + (bh * T + t) * dk;
                for (int64_t i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    const double *row = Gb + i * dv;
                    for (int64_t j = 0; j < dv; ++j) acc += row[j] * vt[j];
                    dko[i] = acc;
                }
                /* dv_t = Gbar_t^T k_t */
                double *dvo = dvv + (bh * T + t) * dv;
                for (int64_t j = 0; j < dv; ++j) dvo[j] = 0.0;
                for (int64_t i = 0; i < dk; ++i) {
                    const double ki = kt[i];
                    const double *row = Gb + i * dv;
                    for (int64_t j = 0; j < dv; ++j) dvo[j] += row[j] * ki;
                }
                /* dla_t = exp(la_t) <Gbar_t, S_{t-1}> */
                const double *Sprev = (t == t0) ? ckpt + s * E : seg + (t - 1 - t0) * E;
                double acc = 0.0;
                for (int64_t e = 0; e < E; ++e) acc += Gb[e] * Sprev[e];
                dla[bh * T + t] = exp(lab[t]) * acc;
            }
        }
        /* dh0 = exp(la_0) Gbar_0 ; with T == 0 the gradient of h0 is zero */
        const double a0 = (T > 0) ? exp(lab[0]) : 0.0;
        for (int64_t e = 0; e < E; ++e) dh0[bh * E + e] = a0 * Gb[e];
        free(S);
        free(Gb);
        free(ckpt);
        free(seg);
    }

    if (!err) {
        /* group sums over the heads of each group, in ascending head order */
#pragma omp parallel for schedule(static)
        for (int64_t bg = 0; bg < B * G; ++bg) {
            const int64_t b = bg / G, g = bg % G;
            for (int64_t x = 0; x < T * dk; ++x) {
                double sq = 0.0, sk = 0.0;
                for (int64_t hh = 0; hh < hpg; ++hh) {
                    const int64_t bh = b * H + g * hpg + hh;
                    sq += dqh[bh * T * dk + x];
                    sk += dkh[bh * T * dk + x];
                }
                dq[bg * T * dk + x] = sq;
                dkk[bg * T * dk + x] = sk;
            }
        }
    }
    free(dqh);
    free(dkh);
    return err;
}
