/*
 * ssd_oracle.c -- fp64 CPU oracle for the Mamba-2 SSD forward and the
 * single-token state update.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header or constant with the HIP
 * library: it includes only the C standard library.
 *
 * What it computes is the plain serial recurrence of the selective state
 * space model with a scalar decay per head (the "mamba" discretisation of
 * the lrnnx `selective_scan_ref` sequential loop, and the single-token
 * branch of fla `Mamba2.torch_forward` applied token after token):
 *
 *   for each batch b and head h, with group g = h / (nheads / ngroups) and
 *   a state S (headdim x dstate) that starts at initial_state[b,h] (or 0):
 *     for t = 0 .. seqlen-1:
 *       alpha   = exp(dt[b,t,h] * A[h])
 *       S[p,n]  = alpha * S[p,n] + dt[b,t,h] * x[b,t,h,p] * B[b,t,g,n]
 *       y[b,t,h,p] = sum_n S[p,n] * C[b,t,g,n] + D[h] * x[b,t,h,p]
 *     final_state[b,h] = S
 *
 * The output uses the state after the token's own update, as the decode
 * branch of the fla layer does.  All arithmetic is IEEE double.  Slices
 * (b,h) are independent, so they are spread over OpenMP threads; inside a
 * slice the order of operations is the textbook one above.
 *
 * Layouts (all dense, row-major, double):
 *   x [batch][seqlen][nheads][headdim]     dt [batch][seqlen][nheads]
 *   A [nheads]   D [nheads] (NULL = 0)     B, C [batch][seqlen][ngroups][dstate]
 *   init, final [batch][nheads][headdim][dstate] (init NULL = zeros,
 *   final NULL = not written)               y [batch][seqlen][nheads][headdim]
 *
 * Returns 0 on success, -1 on a shape that the recurrence does not define
 * (non-positive sizes, nheads not a multiple of ngroups), -2 on allocation
 * failure.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int ssd_oracle_forward(int batch, int seqlen, int nheads, int headdim,
                       int dstate, int ngroups,
                       const double *x, const double *dt, const double *A,
                       const double *B, const double *C, const double *D,
                       const double *init, double *y, double *final_state,
                       int nthreads)
{
    if (batch <= 0 || seqlen <= 0 || nheads <= 0 || headdim <= 0 ||
        dstate <= 0 || ngroups <= 0 || nheads % ngroups != 0)
        return -1;
    const int heads_per_group = nheads / ngroups;
    const long nslices = (long)batch * nheads;
    int failed = 0;

#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
    for (long slice = 0; slice < nslices; ++slice) {
        const int b = (int)(slice / nheads);
        const int h = (int)(slice % nheads);
        const int g = h / heads_per_group;
        double *S = (double *)malloc(sizeof(double) * (size_t)headdim * dstate);
        if (!S) {
            failed |= 1;
            continue;
        }
        const size_t state_off = ((size_t)b * nheads + h) * headdim * dstate;
        if (init)
            memcpy(S, init + state_off, sizeof(double) * (size_t)headdim * dstate);
        else
            memset(S, 0, sizeof(double) * (size_t)headdim * dstate);
        const double Dh = D ? D[h] : 0.0;

        for (int t = 0; t < seqlen; ++t) {
            const size_t tok = (size_t)b * seqlen + t;
            const double dth = dt[tok * nheads + h];
            const double alpha = exp(dth * A[h]);
            const double *xt = x + (tok * nheads + h) * headdim;
            const double *Bt = B + (tok * ngroups + g) * dstate;
            const double *Ct = C + (tok * ngroups + g) * dstate;
            double *yt = y + (tok * nheads + h) * headdim;
            for (int p = 0; p < headdim; ++p) {
                double *Sp = S + (size_t)p * dstate;
                const double u = dth * xt[p];
                double acc = 0.0;
                for (int n = 0; n < dstate; ++n) {
                    Sp[n] = alpha * Sp[n] + u * Bt[n];
                    acc += Sp[n] * Ct[n];
                }
                yt[p] = acc + Dh * xt[p];
            }
        }
        if (final_state)
            memcpy(final_state + state_off, S, sizeof(double) * (size_t)headdim * dstate);
        free(S);
    }
    return failed ? -2 : 0;
}

/* Number of threads OpenMP would use for the loop above (1 without OpenMP). */
int ssd_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
