/* Drives every route of the oracle (oracle/gdr_oracle.c) on small ragged inputs, with all
 * intermediate exports, under AddressSanitizer and UndefinedBehaviorSanitizer: built and run
 * on the host by tests/test_sanitizers.py.  Exit status 0 and "oracle sanitize ok" mean no
 * sanitizer report and that the chunked and tree routes agree with the sequential one. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_gdr_sequential(int64_t B, int64_t T, int64_t HK, int64_t HV, int64_t dk, int64_t dv,
                          const double* q, const double* k, const double* v, const double* g,
                          const double* beta, const double* h0, double* o, double* ht, int nthreads);
int oracle_gdr_chunked(int64_t B, int64_t T, int64_t HK, int64_t HV, int64_t dk, int64_t dv,
                       int64_t C, const double* q, const double* k, const double* v,
                       const double* g, const double* beta, const double* h0, double* o,
                       double* ht, double* A_out, double* P_out, double* W_out,
                       double* Ubar_out, double* U_out, double* gam_out, int nthreads);
int oracle_gdr_tree(int64_t B, int64_t T, int64_t HK, int64_t HV, int64_t dk, int64_t dv,
                    const double* q, const double* k, const double* v, const double* g,
                    const double* beta, const double* h0, const int32_t* parent, double* o,
                    int nthreads);

static uint64_t rng_state = 88172645463325252ull;
static double urand(void) { /* xorshift64, uniform in [-1, 1) */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (double)(rng_state >> 11) / 4503599627370496.0 - 1.0;
}
static double* fill(size_t n, double scale, double shift) {
    double* p = (double*)malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = shift + scale * urand();
    return p;
}

int main(void) {
    const int64_t B = 2, T = 37, HK = 2, HV = 4, dk = 8, dv = 6, C = 16;
    const int64_t NC = (T + C - 1) / C;
    const size_t nq = B * T * HK * dk, nv = B * T * HV * dv, ng = B * T * HV * dk, nb = B * T * HV;
    const size_t ns = B * HV * dk * dv;
    double *q = fill(nq, 0.3, 0), *k = fill(nq, 0.3, 0), *v = fill(nv, 1, 0), *g = fill(ng, 0.2, -0.3);
    double *beta = fill(nb, 0.4, 0.5), *h0 = fill(ns, 0.3, 0);
    double *o1 = calloc(nv, sizeof(double)), *o2 = calloc(nv, sizeof(double)), *o3 = calloc(nv, sizeof(double));
    double *h1 = calloc(ns, sizeof(double)), *h2 = calloc(ns, sizeof(double));
    const size_t nmid = B * HV * NC * C;
    double *A = calloc(nmid * C, sizeof(double)), *P = calloc(nmid * C, sizeof(double));
    double *W = calloc(nmid * dk, sizeof(double)), *Ub = calloc(nmid * dv, sizeof(double));
    double *U = calloc(nmid * dv, sizeof(double)), *gam = calloc(nmid * dk, sizeof(double));
    int32_t* parent = malloc(B * T * sizeof(int32_t));
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < T; ++t) parent[b * T + t] = (int32_t)(t - 1); /* a chain */
    int rc = 0;
    rc |= oracle_gdr_sequential(B, T, HK, HV, dk, dv, q, k, v, g, beta, h0, o1, h1, 2);
    rc |= oracle_gdr_chunked(B, T, HK, HV, dk, dv, C, q, k, v, g, beta, h0, o2, h2, A, P, W, Ub, U, gam, 2);
    rc |= oracle_gdr_tree(B, T, HK, HV, dk, dv, q, k, v, g, beta, h0, parent, o3, 2);
    /* invalid dims are refused, not read */
    rc |= oracle_gdr_sequential(B, T, 3, HV, dk, dv, q, k, v, g, beta, h0, o1, h1, 1) == 0;
    double e = 0;
    for (size_t i = 0; i < nv; ++i) e = fmax(e, fmax(fabs(o1[i] - o2[i]), fabs(o1[i] - o3[i])));
    for (size_t i = 0; i < ns; ++i) e = fmax(e, fabs(h1[i] - h2[i]));
    free(q); free(k); free(v); free(g); free(beta); free(h0); free(o1); free(o2); free(o3);
    free(h1); free(h2); free(A); free(P); free(W); free(Ub); free(U); free(gam); free(parent);
    if (rc || !(e < 1e-10)) {
        fprintf(stderr, "oracle routes disagree or failed: rc=%d err=%g\n", rc, e);
        return 1;
    }
    printf("oracle sanitize ok\n");
    return 0;
}
