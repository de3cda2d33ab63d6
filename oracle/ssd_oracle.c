/*
 * ssd_oracle.c -- fp64 CPU oracle for the Mamba-2 SSD forward, the
 * single-token state update, and the gradients of the forward.
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

/*
 * ssd_oracle_backward -- gradients of the recurrence above, by reverse-mode
 * differentiation of its loop, in fp64.
 *
 * Given dy = dLoss/dy [batch][seqlen][nheads][headdim] and dfinal =
 * dLoss/dfinal_state [batch][nheads][headdim][dstate] (NULL = 0), it
 * returns the gradients of the same loss with respect to every input:
 *   dx [b][L][H][P], ddt [b][L][H], dA [H], dB, dC [b][L][G][N],
 *   dD [H] (NULL = not written), dinit [b][H][P][N] (NULL = not written).
 *
 * With lambda the gradient with respect to the state S_t, the loop is run
 * backwards token by token (per batch b and head h, group g):
 *   lambda = dfinal[b,h] (or 0)
 *   for t = seqlen-1 .. 0:
 *     lambda[p,n] += dy_t[p] * C_t[n]                  (y_t = S_t C_t + D x_t)
 *     dC_t[n]     += sum_p dy_t[p] * S_t[p,n]
 *     dD          += sum_p dy_t[p] * x_t[p]
 *     dx_t[p]      = D dy_t[p] + dt_t * sum_n lambda[p,n] B_t[n]
 *     dB_t[n]     += dt_t * sum_p lambda[p,n] x_t[p]
 *     e            = sum_{p,n} lambda[p,n] * alpha_t * S_{t-1}[p,n]   (dLoss/d(dt_t A))
 *     ddt_t        = sum_{p,n} lambda[p,n] x_t[p] B_t[n] + A e
 *     dA          += dt_t * e
 *     lambda       = alpha_t * lambda                  (the gradient w.r.t. S_{t-1})
 *   dinit[b,h] = lambda
 * dB and dC sum over the heads of a group.  The states S_t are recomputed:
 * the forward loop keeps S at every 64th token, and each 64-token segment
 * is replayed from its checkpoint before it is walked backwards.
 *
 * Returns 0, -1 on a bad shape, -2 on allocation failure.
 */
int ssd_oracle_backward(int batch, int seqlen, int nheads, int headdim,
                        int dstate, int ngroups,
                        const double *x, const double *dt, const double *A,
                        const double *B, const double *C, const double *D,
                        const double *init, const double *dy, const double *dfinal,
                        double *dx, double *ddt, double *dA, double *dB, double *dC,
                        double *dD, double *dinit, int nthreads)
{
    if (batch <= 0 || seqlen <= 0 || nheads <= 0 || headdim <= 0 ||
        dstate <= 0 || ngroups <= 0 || nheads % ngroups != 0)
        return -1;
    enum { K = 64 };
    const int hpg = nheads / ngroups;
    const long nslices = (long)batch * nheads;
    const size_t PN = (size_t)headdim * dstate;
    const size_t bc_elems = (size_t)batch * seqlen * ngroups * dstate;
    const int nseg = (seqlen + K - 1) / K;
    int failed = 0;

    memset(dB, 0, sizeof(double) * bc_elems);
    memset(dC, 0, sizeof(double) * bc_elems);
    memset(dA, 0, sizeof(double) * nheads);
    if (dD)
        memset(dD, 0, sizeof(double) * nheads);

#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel reduction(| : failed)
#endif
    {
        /* per-thread partial sums of the group and head reductions */
        double *pB = (double *)calloc(bc_elems, sizeof(double));
        double *pC = (double *)calloc(bc_elems, sizeof(double));
        double *pA = (double *)calloc((size_t)nheads, sizeof(double));
        double *pD = (double *)calloc((size_t)nheads, sizeof(double));
        double *ck = (double *)malloc(sizeof(double) * PN * (size_t)(nseg + 1));
        double *seg = (double *)malloc(sizeof(double) * PN * (K + 1));
        double *lam = (double *)malloc(sizeof(double) * PN);
        /* (every thread takes part in the loop, with or without its buffers) */
        const int ok = pB && pC && pA && pD && ck && seg && lam;
        if (!ok)
            failed |= 1;
        {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (long slice = 0; slice < nslices; ++slice) {
                if (!ok)
                    continue;
                const int b = (int)(slice / nheads);
                const int h = (int)(slice % nheads);
                const int g = h / hpg;
                const size_t soff = ((size_t)b * nheads + h) * PN;
                const double Ah = A[h], Dh = D ? D[h] : 0.0;
                /* forward: the state before each 64-token segment */
                double *S = ck;
                if (init)
                    memcpy(S, init + soff, sizeof(double) * PN);
                else
                    memset(S, 0, sizeof(double) * PN);
                for (int sg = 0; sg < nseg; ++sg) {
                    double *Sn = ck + PN * (size_t)(sg + 1);
                    memcpy(Sn, ck + PN * (size_t)sg, sizeof(double) * PN);
                    const int t1 = (sg + 1) * K < seqlen ? (sg + 1) * K : seqlen;
                    for (int t = sg * K; t < t1; ++t) {
                        const size_t tok = (size_t)b * seqlen + t;
                        const double dth = dt[tok * nheads + h];
                        const double alpha = exp(dth * Ah);
                        const double *xt = x + (tok * nheads + h) * headdim;
                        const double *Bt = B + (tok * ngroups + g) * dstate;
                        for (int p = 0; p < headdim; ++p)
                            for (int n = 0; n < dstate; ++n)
                                Sn[(size_t)p * dstate + n] = alpha * Sn[(size_t)p * dstate + n] +
                                                            dth * xt[p] * Bt[n];
                    }
                }
                /* backward, segment by segment from the end */
                if (dfinal)
                    memcpy(lam, dfinal + soff, sizeof(double) * PN);
                else
                    memset(lam, 0, sizeof(double) * PN);
                for (int sg = nseg - 1; sg >= 0; --sg) {
                    const int t0 = sg * K;
                    const int t1 = (sg + 1) * K < seqlen ? (sg + 1) * K : seqlen;
                    /* seg[i] = the state after token t0 + i - 1 (seg[0]: before t0) */
                    memcpy(seg, ck + PN * (size_t)sg, sizeof(double) * PN);
                    for (int t = t0; t < t1; ++t) {
                        const size_t tok = (size_t)b * seqlen + t;
                        const double dth = dt[tok * nheads + h];
                        const double alpha = exp(dth * Ah);
                        const double *xt = x + (tok * nheads + h) * headdim;
                        const double *Bt = B + (tok * ngroups + g) * dstate;
                        const double *Sp = seg + PN * (size_t)(t - t0);
                        double *Sq = seg + PN * (size_t)(t - t0 + 1);
                        for (int p = 0; p < headdim; ++p)
                            for (int n = 0; n < dstate; ++n)
                                Sq[(size_t)p * dstate + n] = alpha * Sp[(size_t)p * dstate + n] +
                                                            dth * xt[p] * Bt[n];
                    }
                    for (int t = t1 - 1; t >= t0; --t) {
                        const size_t tok = (size_t)b * seqlen + t;
                        const double dth = dt[tok * nheads + h];
                        const double alpha = exp(dth * Ah);
                        const double *xt = x + (tok * nheads + h) * headdim;
                        const double *Bt = B + (tok * ngroups + g) * dstate;
                        const double *Ct = C + (tok * ngroups + g) * dstate;
                        const double *dyt = dy + (tok * nheads + h) * headdim;
                        const double *St = seg + PN * (size_t)(t - t0 + 1);   /* S_t */
                        const double *Sm = seg + PN * (size_t)(t - t0);       /* S_{t-1} */
                        double *dBt = pB + (tok * ngroups + g) * dstate;
                        double *dCt = pC + (tok * ngroups + g) * dstate;
                        double *dxt = dx + (tok * nheads + h) * headdim;
                        double dxd = 0.0, e = 0.0, dd = 0.0;
                        for (int p = 0; p < headdim; ++p) {
                            double *lp = lam + (size_t)p * dstate;
                            const double *sp = St + (size_t)p * dstate;
                            const double *mp = Sm + (size_t)p * dstate;
                            double lb = 0.0;
                            for (int n = 0; n < dstate; ++n) {
                                lp[n] += dyt[p] * Ct[n];
                                dCt[n] += dyt[p] * sp[n];
                                lb += lp[n] * Bt[n];
                                dBt[n] += dth * lp[n] * xt[p];
                                e += lp[n] * alpha * mp[n];
                            }
                            dxt[p] = Dh * dyt[p] + dth * lb;
                            dxd += xt[p] * lb;
                            dd += dyt[p] * xt[p];
                        }
                        ddt[tok * nheads + h] = dxd + Ah * e;
                        pA[h] += dth * e;
                        pD[h] += dd;
                        for (size_t i = 0; i < PN; ++i)
                            lam[i] *= alpha;
                    }
                }
                if (dinit)
                    memcpy(dinit + soff, lam, sizeof(double) * PN);
            }
#ifdef _OPENMP
#pragma omp critical
#endif
            if (ok) {
                for (size_t i = 0; i < bc_elems; ++i) {
                    dB[i] += pB[i];
                    dC[i] += pC[i];
                }
                for (int h = 0; h < nheads; ++h) {
                    dA[h] += pA[h];
                    if (dD)
                        dD[h] += pD[h];
                }
            }
        }
        free(pB);
        free(pC);
        free(pA);
        free(pD);
        free(ck);
        free(seg);
        free(lam);
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
