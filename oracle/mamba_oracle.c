/*
 * mamba_oracle.c -- fp64 CPU oracle for the selective (Mamba-style) scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite and the benchmark's
 * CPU-baseline leg may load this library.  The GPU product path never calls
 * it, links it or falls back to it, and it shares no code, header or
 * constant with the GPU path.
 *
 * What is computed (plain definition, step by step).  For every batch b,
 * channel d < D and state n < N, with h_{-1} = 0:
 *
 *     a_t[d,n] = exp(delta[b,t,d] * A[d,n])
 *     h_t[d,n] = a_t[d,n] * h_{t-1}[d,n] + delta[b,t,d] * B[b,t,n] * x[b,t,d]
 *     y[b,t,d] = sum_n C[b,t,n] * h_t[d,n] + Dskip[d] * x[b,t,d]
 *
 * The benchmark page kernel_mamba_cpu.json fixes the tensor set through its
 * byte counts: at batch 4, seq 512, dim 256, state 16 every fwd record has
 * xla_arg_mb 4.27, which is x[B,L,D] + delta[B,L,D] + A[D,N] + B[B,L,N] +
 * C[B,L,N] + Dskip[D] in float32 (4.2666 MiB), and xla_out_mb 2.0, which is
 * y[B,L,D]; its fwd_bwd records output 4.27 MiB, the six input gradients.
 * The page prints no formula; the recurrence above is the plain reading of
 * that argument set (the selective scan with per-channel diagonal state, the
 * input weighted by delta * B, no softplus of delta and no gating).  The loss
 * is L = sum dy . y for a given upstream dy.
 *
 * Backward (reverse-mode adjoint of the recurrence, derived by hand), with
 * G_t[d,n] = dL/dh_t:
 *
 *     G_t      = C_t[n] dy_t[d] + a_{t+1} G_{t+1},            G_{L-1} = C dy
 *     dx_t[d]  = Dskip[d] dy_t[d] + sum_n G_t delta_t[d] B_t[n]
 *     ddelta_t[d] = sum_n G_t (A[d,n] a_t h_{t-1} + B_t[n] x_t[d])
 *     dA[d,n]  = sum_{b,t} G_t delta_t[d] a_t h_{t-1}
 *     dB_t[n]  = sum_d G_t delta_t[d] x_t[d]
 *     dC_t[n]  = sum_d dy_t[d] h_t[d,n]
 *     dDskip[d] = sum_{b,t} dy_t[d] x_t[d]
 *
 * All arithmetic is IEEE double; inputs are given as doubles (callers
 * promote float32 inputs exactly).  The backward stores every h_t of one
 * (b, d) (L x N doubles) and walks it in reverse.  The forward splits its
 * (b, d) pairs over OpenMP threads, each pair's arithmetic sequential; the
 * backward runs on one thread, with the sums over b (dA, dDskip) and over d
 * (dB, dC) taken in ascending b and d.  Results do not depend on the thread
 * count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static int check_shape(int64_t B, int64_t L, int64_t D, int64_t N)
{
    return (B < 0 || L < 0 || D < 1 || N < 1) ? 1 : 0;
}

/* y[B,L,D] */
int mamba_oracle_fwd(int64_t B, int64_t L, int64_t D, int64_t N, const double *x, const double *delta,
                     const double *A, const double *Bm, const double *Cm, const double *Ds, double *y)
{
    if (check_shape(B, L, D, N)) return 1;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : fail)
    for (int64_t bd = 0; bd < B * D; ++bd) {
        const int64_t b = bd / D, d = bd % D;
        double *h = (double *)calloc((size_t)N, sizeof(double));
        if (!h) {
            fail |= 1;
            continue;
        }
        for (int64_t t = 0; t < L; ++t) {
            const int64_t i = (b * L + t) * D + d;
            const double dl = delta[i], xv = x[i];
            const double *Bt = Bm + (b * L + t) * N, *Ct = Cm + (b * L + t) * N;
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                const double a = exp(dl * A[d * N + n]);
                h[n] = a * h[n] + dl * Bt[n] * xv;
                acc += Ct[n] * h[n];
            }
            y[i] = acc + Ds[d] * xv;
        }
        free(h);
    }
    return fail;
}

/* Gradients of L = sum dy * y: dx, ddelta [B,L,D]; dA [D,N]; dB, dC [B,L,N];
 * dD [D].  Every output is overwritten. */
int mamba_oracle_bwd(int64_t B, int64_t L, int64_t D, int64_t N, const double *x, const double *delta,
                     const double *A, const double *Bm, const double *Cm, const double *Ds, const double *dy,
                     double *dx, double *ddelta, double *dA, double *dB, double *dC, double *dD)
{
    if (check_shape(B, L, D, N)) return 1;
    memset(dA, 0, sizeof(double) * (size_t)(D * N));
    memset(dD, 0, sizeof(double) * (size_t)D);
    memset(dB, 0, sizeof(double) * (size_t)(B * L * N));
    memset(dC, 0, sizeof(double) * (size_t)(B * L * N));
    if (B == 0 || L == 0) return 0;
    double *hs = (double *)malloc(sizeof(double) * (size_t)(L * N));   // h_t of one (b, d)
    double *G = (double *)malloc(sizeof(double) * (size_t)N);
    if (!hs || !G) {
        free(hs);
        free(G);
        return 1;
    }
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t d = 0; d < D; ++d) {
            // forward sweep, keeping every state
            for (int64_t t = 0; t < L; ++t) {
                const int64_t i = (b * L + t) * D + d;
                const double dl = delta[i], xv = x[i];
                const double *Bt = Bm + (b * L + t) * N;
                for (int64_t n = 0; n < N; ++n) {
                    const double prev = t > 0 ? hs[(t - 1) * N + n] : 0.0;
                    hs[t * N + n] = exp(dl * A[d * N + n]) * prev + dl * Bt[n] * xv;
                }
            }
            // reverse sweep
            for (int64_t n = 0; n < N; ++n) G[n] = 0.0;
            for (int64_t t = L - 1; t >= 0; --t) {
                const int64_t i = (b * L + t) * D + d;
                const double dl = delta[i], xv = x[i], g = dy[i];
                const double *Bt = Bm + (b * L + t) * N, *Ct = Cm + (b * L + t) * N;
                double sx = 0.0, sdl = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    // G_t = C_t dy_t + a_{t+1} G_{t+1}
                    const double anext =
                        t + 1 < L ? exp(delta[(b * L + t + 1) * D + d] * A[d * N + n]) : 0.0;
                    G[n] = Ct[n] * g + anext * G[n];
                    const double a = exp(dl * A[d * N + n]);
                    const double prev = t > 0 ? hs[(t - 1) * N + n] : 0.0;
                    sx += G[n] * dl * Bt[n];
                    sdl += G[n] * (A[d * N + n] * a * prev + Bt[n] * xv);
                    dA[d * N + n] += G[n] * dl * a * prev;
                    dB[(b * L + t) * N + n] += G[n] * dl * xv;
                    dC[(b * L + t) * N + n] += g * hs[t * N + n];
                }
                dx[i] = Ds[d] * g + sx;
                ddelta[i] = sdl;
                dD[d] += g * xv;
            }
        }
    }
    free(hs);
    free(G);
    return 0;
}

int mamba_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
