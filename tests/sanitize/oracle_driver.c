/*
 * Drives the C oracle (oracle/ssd_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built by tests/test_sanitizers.py): every
 * optional pointer NULL and set, length 1, ragged shapes, grouped B and C,
 * the shapes it must refuse.  Test infrastructure only.  Each result is
 * also checked against a second evaluation of the recurrence written here
 * token by token for one slice, so a run that is memory-clean but wrong
 * fails too.  Prints "ok" and exits 0 on success.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int ssd_oracle_forward(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups,
                       const double *x, const double *dt, const double *A, const double *B,
                       const double *C, const double *D, const double *init, double *y,
                       double *final_state, int nthreads);

static double urand(unsigned *s) {
    *s = *s * 1664525u + 1013904223u;
    return (double)(*s >> 8) / (double)(1u << 24) - 0.5;
}

static double *fill(size_t n, unsigned *s) {
    double *p = (double *)malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = urand(s);
    return p;
}

/* y of slice (b, h) at token t, column p, by the recurrence, for checking */
static double slice_y(int b, int h, int t, int p, int L, int H, int P, int N, int G,
                      const double *x, const double *dt, const double *A, const double *B,
                      const double *C, const double *D, const double *init) {
    const int g = h / (H / G);
    double *S = (double *)calloc((size_t)N, sizeof(double));
    if (init)
        for (int n = 0; n < N; ++n) S[n] = init[(((size_t)b * H + h) * P + p) * N + n];
    double y = 0.0;
    for (int s = 0; s <= t; ++s) {
        const size_t tok = (size_t)b * L + s;
        const double d = dt[tok * H + h];
        const double a = exp(d * A[h]);
        const double xv = x[(tok * H + h) * P + p];
        y = 0.0;
        for (int n = 0; n < N; ++n) {
            S[n] = a * S[n] + d * xv * B[(tok * G + g) * N + n];
            y += S[n] * C[(tok * G + g) * N + n];
        }
        if (D) y += D[h] * xv;
    }
    free(S);
    return y;
}

static int run(int b, int L, int H, int P, int N, int G, int use_d, int use_init, int use_fin,
               unsigned seed) {
    unsigned s = seed;
    double *x = fill((size_t)b * L * H * P, &s);
    double *dt = fill((size_t)b * L * H, &s);
    for (size_t i = 0; i < (size_t)b * L * H; ++i) dt[i] = fabs(dt[i]) * 0.2;
    double *A = fill((size_t)H, &s);
    for (int i = 0; i < H; ++i) A[i] = -fabs(A[i]) * 4.0 - 0.1;
    double *B = fill((size_t)b * L * G * N, &s);
    double *C = fill((size_t)b * L * G * N, &s);
    double *D = use_d ? fill((size_t)H, &s) : NULL;
    double *init = use_init ? fill((size_t)b * H * P * N, &s) : NULL;
    double *y = (double *)malloc(sizeof(double) * (size_t)b * L * H * P);
    double *fin = use_fin ? (double *)malloc(sizeof(double) * (size_t)b * H * P * N) : NULL;
    int rc = ssd_oracle_forward(b, L, H, P, N, G, x, dt, A, B, C, D, init, y, fin, 0);
    int bad = rc != 0;
    if (!bad) {
        /* the last token of the last slice and a middle token of the first */
        const int cases[2][4] = {{b - 1, H - 1, L - 1, P - 1}, {0, 0, L / 2, 0}};
        for (int k = 0; k < 2; ++k) {
            const int cb = cases[k][0], ch = cases[k][1], ct = cases[k][2], cp = cases[k][3];
            const double want = slice_y(cb, ch, ct, cp, L, H, P, N, G, x, dt, A, B, C, D, init);
            const double got = y[(((size_t)cb * L + ct) * H + ch) * P + cp];
            if (fabs(got - want) > 1e-12 * (1.0 + fabs(want))) bad = 1;
        }
    }
    free(x); free(dt); free(A); free(B); free(C); free(D); free(init); free(y); free(fin);
    if (bad) fprintf(stderr, "case b%d L%d H%d P%d N%d G%d failed (rc %d)\n", b, L, H, P, N, G, rc);
    return bad;
}

int main(void) {
    int bad = 0;
    bad |= run(1, 1, 1, 1, 1, 1, 0, 0, 0, 1);
    bad |= run(2, 37, 4, 8, 5, 2, 1, 1, 1, 2);
    bad |= run(3, 17, 6, 3, 7, 3, 1, 0, 1, 3);
    bad |= run(1, 64, 2, 16, 16, 1, 0, 1, 0, 4);
    bad |= run(2, 5, 8, 4, 2, 8, 1, 1, 1, 5);
    /* shapes the recurrence does not define */
    double v = 0.0;
    if (ssd_oracle_forward(0, 4, 2, 2, 2, 1, &v, &v, &v, &v, &v, NULL, NULL, &v, NULL, 0) != -1) bad = 1;
    if (ssd_oracle_forward(1, 4, 3, 2, 2, 2, &v, &v, &v, &v, &v, NULL, NULL, &v, NULL, 0) != -1) bad = 1;
    if (ssd_oracle_forward(1, -1, 2, 2, 2, 1, &v, &v, &v, &v, &v, NULL, NULL, &v, NULL, 0) != -1) bad = 1;
    if (!bad) printf("ok\n");
    return bad;
}
