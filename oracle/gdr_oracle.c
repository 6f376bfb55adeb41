/*
 * TEST INFRASTRUCTURE ONLY -- fp64 CPU oracle for the channelwise gated delta rule.
 *
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark may load
 * this library.  The GPU product path never links, calls or includes anything here,
 * and nothing here is shared with it.
 *
 * What it computes (per batch b and value head h, key head kh = h / (HV/HK)):
 *   state S[dk][dv] (fp64), initialised from h0 or zero; for every token t
 *     1. decay      S[i][:] *= exp(g[t][i])                  (per key channel i)
 *     2. predict    pred[j]  = sum_i k[t][i] * S[i][j]        (from the decayed state)
 *     3. update     S[i][j] += k[t][i] * beta[t] * (v[t][j] - pred[j])
 *     4. output     o[t][j]  = sum_i q[t][i] * S[i][j]        (from the updated state)
 *   and ht = S after the last token.
 * The order decay -> predict -> update -> output is the one described in the first
 * commit summary of ExecuTorch PR #21021 ("Reorder channelwise gated delta rule chunked
 * hot loops for autovectorization"): the prediction is taken with the decay folded in,
 * then decay and the rank-one update are applied and the output is accumulated from the
 * new state.  Inner loops run with unit stride over the value dimension (third commit
 * summary of the same page).
 *
 * oracle_gdr_chunked() is a second, independent route to the same numbers: the
 * chunkwise WY/UT form named in the second commit summary of that page (per-channel
 * log-decay prefixes, beta-folded strictly-lower gram, triangular solve, WY pseudo-keys
 * and pseudo-values, causal query/key terms, inter-chunk state carry, ragged final chunk
 * handled as a shorter chunk).  The solve is exact forward substitution in fp64, the
 * choice defended in the review thread of uzu PR #576 ("Support TreeUpdateSolve kernel").
 * It optionally exports its per-chunk intermediates for kernel unit tests.
 *
 * Layouts (row-major, all fp64 here):
 *   q, k  [B][T][HK][dk]      v, o  [B][T][HV][dv]
 *   g     [B][T][HV][dk]      beta  [B][T][HV]
 *   h0,ht [B][HV][dk][dv]     (h0 may be NULL = zero state; ht may be NULL)
 * oracle_gdr_tree() runs the same token step over a tree of T nodes per batch element (the
 * speculative token tree that the tree-verify solve of uzu PR #576 serves): node t
 * continues from the state its parent node reached, parent[b][t] in [-1, t) with -1
 * meaning the initial state, and its output is taken from its own updated state.  A chain
 * (parent t-1) is exactly the sequential recurrence.
 *
 * Return value: 0 on success, -1 on invalid sizes, -2 on allocation failure, -3 on a
 * parent index outside [-1, t).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int dims_ok(int64_t B, int64_t T, int64_t HK, int64_t HV, int64_t dk, int64_t dv) {
    return B >= 1 && T >= 1 && HK >= 1 && HV >= 1 && dk >= 1 && dv >= 1 && (HV % HK) == 0;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------------------ */
/* Sequential token recurrence.                                                          */
/* ------------------------------------------------------------------------------------ */
int oracle_gdr_sequential(int64_t B, int64_t T, int64_t HK, int64_t HV, int64_t dk, int64_t dv,
                          const double* q, const double* k, const double* v, const double* g,
                          const double* beta, const double* h0, double* o, double* ht,
                          int nthreads) {
    if (!dims_ok(B, T, HK, HV, dk, dv)) return -1;
    set_threads(nthreads);
    const int64_t G = HV / HK;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < B * HV; ++bh) {
        const int64_t b = bh / HV, h = bh % HV, kh = h / G;
        double* S = (double*)malloc(sizeof(double) * (size_t)(dk * dv + 2 * dv));
        if (!S) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        double* pred = S + dk * dv;
        double* d = pred + dv;
        if (h0)
            memcpy(S, h0 + bh * dk * dv, sizeof(double) * (size_t)(dk * dv));
        else
            memset(S, 0, sizeof(double) * (size_t)(dk * dv));
        for (int64_t t = 0; t < T; ++t) {
            const double* kt = k + ((b * T + t) * HK + kh) * dk;
            const double* qt = q + ((b * T + t) * HK + kh) * dk;
            const double* vt = v + ((b * T + t) * HV + h) * dv;
            const double* gt = g + ((b * T + t) * HV + h) * dk;
            const double bt = beta[(b * T + t) * HV + h];
            double* ot = o + ((b * T + t) * HV + h) * dv;
            /* 1. decay */
            for (int64_t i = 0; i < dk; ++i) {
                const double e = exp(gt[i]);
                double* Si = S + i * dv;
                for (int64_t j = 0; j < dv; ++j) Si[j] *= e;
            }
            /* 2. predict */
            for (int64_t j = 0; j < dv; ++j) pred[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i) {
                const double ki = kt[i];
                const double* Si = S + i * dv;
                for (int64_t j = 0; j < dv; ++j) pred[j] += ki * Si[j];
            }
            /* 3. rank-one delta update */
            for (int64_t j = 0; j < dv; ++j) d[j] = bt * (vt[j] - pred[j]);
            for (int64_t i = 0; i < dk; ++i) {
                const double ki = kt[i];
                double* Si = S + i * dv;
                for (int64_t j = 0; j < dv; ++j) Si[j] += ki * d[j];
            }
            /* 4. output from the updated state */
            for (int64_t j = 0; j < dv; ++j) ot[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i) {
                const double qi = qt[i];
                const double* Si = S + i * dv;
                for (int64_t j = 0; j < dv; ++j) ot[j] += qi * Si[j];
            }
        }
        if (ht) memcpy(ht + bh * dk * dv, S, sizeof(double) * (size_t)(dk * dv));
        free(S);
    }
    return failed ? -2 : 0;
}

/* ------------------------------------------------------------------------------------ */
/* Chunkwise WY/UT form, written step by step.                                          */
/*                                                                                       */
/* For a chunk of L tokens starting at t0 with incoming state S0 (rows r, s in 0..L-1): */
/*   C1 gam[r][c] = sum_{s<=r} g[t0+s][c]                       (restarts every chunk)   */
/*   C2 A[r][s]   = beta_r sum_c k_rc k_sc exp(gam_rc - gam_sc)  for s < r, else 0       */
/*   C3 (I + A) X = [diag(beta) Kt | diag(beta) V],  Kt_r = exp(gam_r) * k_r             */
/*      solved by forward substitution                                                   */
/*   C4 W = X[:, :dk] (pseudo-keys), Ubar = X[:, dk:] (pseudo-values), U = Ubar - W S0   */
/*   C5 P[r][s]   = sum_c q_rc k_sc exp(gam_rc - gam_sc)        for s <= r, else 0       */
/*   C6 O = (exp(gam) * Q) S0 + P U                                                      */
/*   C7 S_L = diag(exp(gam_{L-1})) S0 + (exp(gam_{L-1} - gam) * K)^T U                   */
/* Optional exports, each [B][HV][NC][C][*] with rows >= L of the last chunk set to 0:  */
/*   A_out, P_out [..][C][C]; W_out [..][C][dk]; Ubar_out, U_out [..][C][dv];            */
/*   gam_out [..][C][dk].                                                                */
/* ------------------------------------------------------------------------------------ */
int oracle_gdr_chunked(int64_t B, int64_t T, int64_t HK, int64_t HV, int64_t dk, int64_t dv,
                       int64_t C, const double* q, const double* k, const double* v,
                       const double* g, const double* beta, const double* h0, double* o,
                       double* ht, double* A_out, double* P_out, double* W_out,
                       double* Ubar_out, double* U_out, double* gam_out, int nthreads) {
    if (!dims_ok(B, T, HK, HV, dk, dv) || C < 1) return -1;
    set_threads(nthreads);
    const int64_t G = HV / HK;
    const int64_t NC = (T + C - 1) / C;
    const int64_t RW = dk + dv; /* width of the solve's right-hand side */
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < B * HV; ++bh) {
        const int64_t b = bh / HV, h = bh % HV, kh = h / G;
        const size_t n_work = (size_t)(dk * dv      /* S */
                                       + dk * dv    /* S_next */
                                       + C * dk     /* gam */
                                       + C * C * 2  /* A, P */
                                       + C * RW     /* X */
                                       + C * dv);   /* U */
        double* S = (double*)calloc(n_work, sizeof(double));
        if (!S) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        double* Sn = S + dk * dv;
        double* gam = Sn + dk * dv;
        double* A = gam + C * dk;
        double* P = A + C * C;
        double* X = P + C * C;
        double* U = X + C * RW;
        if (h0) memcpy(S, h0 + bh * dk * dv, sizeof(double) * (size_t)(dk * dv));

        for (int64_t n = 0; n < NC; ++n) {
            const int64_t t0 = n * C;
            const int64_t L = (T - t0) < C ? (T - t0) : C;
#define KROW(r) (k + ((b * T + t0 + (r)) * HK + kh) * dk)
#define QROW(r) (q + ((b * T + t0 + (r)) * HK + kh) * dk)
#define VROW(r) (v + ((b * T + t0 + (r)) * HV + h) * dv)
#define GROW(r) (g + ((b * T + t0 + (r)) * HV + h) * dk)
#define BETA(r) (beta[(b * T + t0 + (r)) * HV + h])
            /* C1: inclusive per-channel prefix of the log-decay */
            for (int64_t c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int64_t r = 0; r < L; ++r) {
                    acc += GROW(r)[c];
                    gam[r * dk + c] = acc;
                }
            }
            /* C2 and C5: gram terms */
            for (int64_t r = 0; r < L; ++r) {
                for (int64_t s = 0; s < L; ++s) {
                    double a = 0.0, p = 0.0;
                    if (s <= r) {
                        for (int64_t c = 0; c < dk; ++c) {
                            const double f = exp(gam[r * dk + c] - gam[s * dk + c]);
                            a += KROW(r)[c] * KROW(s)[c] * f;
                            p += QROW(r)[c] * KROW(s)[c] * f;
                        }
                    }
                    A[r * C + s] = (s < r) ? BETA(r) * a : 0.0;
                    P[r * C + s] = (s <= r) ? p : 0.0;
                }
            }
            /* C3: right-hand side, then forward substitution (I + A) X = RHS */
            for (int64_t r = 0; r < L; ++r) {
                const double br = BETA(r);
                for (int64_t c = 0; c < dk; ++c)
                    X[r * RW + c] = br * exp(gam[r * dk + c]) * KROW(r)[c];
                for (int64_t j = 0; j < dv; ++j) X[r * RW + dk + j] = br * VROW(r)[j];
            }
            for (int64_t r = 0; r < L; ++r)
                for (int64_t s = 0; s < r; ++s) {
                    const double a = A[r * C + s];
                    for (int64_t x = 0; x < RW; ++x) X[r * RW + x] -= a * X[s * RW + x];
                }
            /* C4: U = Ubar - W S0 */
            for (int64_t r = 0; r < L; ++r) {
                for (int64_t j = 0; j < dv; ++j) U[r * dv + j] = X[r * RW + dk + j];
                for (int64_t c = 0; c < dk; ++c) {
                    const double w = X[r * RW + c];
                    for (int64_t j = 0; j < dv; ++j) U[r * dv + j] -= w * S[c * dv + j];
                }
            }
            /* C6: outputs */
            for (int64_t r = 0; r < L; ++r) {
                double* orow = o + ((b * T + t0 + r) * HV + h) * dv;
                for (int64_t j = 0; j < dv; ++j) orow[j] = 0.0;
                for (int64_t c = 0; c < dk; ++c) {
                    const double qd = exp(gam[r * dk + c]) * QROW(r)[c];
                    for (int64_t j = 0; j < dv; ++j) orow[j] += qd * S[c * dv + j];
                }
                for (int64_t s = 0; s <= r; ++s) {
                    const double p = P[r * C + s];
                    for (int64_t j = 0; j < dv; ++j) orow[j] += p * U[s * dv + j];
                }
            }
            /* C7: state carry */
            for (int64_t c = 0; c < dk; ++c) {
                const double gl = gam[(L - 1) * dk + c];
                const double el = exp(gl);
                for (int64_t j = 0; j < dv; ++j) Sn[c * dv + j] = el * S[c * dv + j];
                for (int64_t r = 0; r < L; ++r) {
                    const double kb = exp(gl - gam[r * dk + c]) * KROW(r)[c];
                    for (int64_t j = 0; j < dv; ++j) Sn[c * dv + j] += kb * U[r * dv + j];
                }
            }
            memcpy(S, Sn, sizeof(double) * (size_t)(dk * dv));
            /* optional exports */
            const int64_t base = (bh * NC + n) * C;
            for (int64_t r = 0; r < C; ++r) {
                const int live = r < L;
                if (A_out)
                    for (int64_t s = 0; s < C; ++s)
                        A_out[(base + r) * C + s] = live && s < L ? A[r * C + s] : 0.0;
                if (P_out)
                    for (int64_t s = 0; s < C; ++s)
                        P_out[(base + r) * C + s] = live && s < L ? P[r * C + s] : 0.0;
                if (W_out)
                    for (int64_t c = 0; c < dk; ++c)
                        W_out[(base + r) * dk + c] = live ? X[r * RW + c] : 0.0;
                if (Ubar_out)
                    for (int64_t j = 0; j < dv; ++j)
                        Ubar_out[(base + r) * dv + j] = live ? X[r * RW + dk + j] : 0.0;
                if (U_out)
                    for (int64_t j = 0; j < dv; ++j)
                        U_out[(base + r) * dv + j] = live ? U[r * dv + j] : 0.0;
                if (gam_out)
                    for (int64_t c = 0; c < dk; ++c)
                        gam_out[(base + r) * dk + c] = live ? gam[r * dk + c] : 0.0;
            }
#undef KROW
#undef QROW
#undef VROW
#undef GROW
#undef BETA
        }
        if (ht) memcpy(ht + bh * dk * dv, S, sizeof(double) * (size_t)(dk * dv));
        free(S);
    }
    return failed ? -2 : 0;
}

/* ------------------------------------------------------------------------------------ */
/* Token recurrence over a tree: every node continues from its parent's state.           */
/* ------------------------------------------------------------------------------------ */
int oracle_gdr_tree(int64_t B, int64_t T, int64_t HK, int64_t HV, int64_t dk, int64_t dv,
                    const double* q, const double* k, const double* v, const double* g,
                    const double* beta, const double* h0, const int32_t* parent, double* o,
                    int nthreads) {
    if (!dims_ok(B, T, HK, HV, dk, dv) || !parent) return -1;
    for (int64_t i = 0; i < B * T; ++i)
        if (parent[i] < -1 || parent[i] >= i % T) return -3;
    set_threads(nthreads);
    const int64_t G = HV / HK;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < B * HV; ++bh) {
        const int64_t b = bh / HV, h = bh % HV, kh = h / G;
        /* the state every node reached, then two dv scratch rows */
        double* states = (double*)malloc(sizeof(double) * (size_t)(T * dk * dv + 2 * dv));
        if (!states) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        double* pred = states + T * dk * dv;
        double* d = pred + dv;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t p = parent[b * T + t];
            double* S = states + t * dk * dv;
            if (p >= 0)
                memcpy(S, states + p * dk * dv, sizeof(double) * (size_t)(dk * dv));
            else if (h0)
                memcpy(S, h0 + bh * dk * dv, sizeof(double) * (size_t)(dk * dv));
            else
                memset(S, 0, sizeof(double) * (size_t)(dk * dv));
            const double* kt = k + ((b * T + t) * HK + kh) * dk;
            const double* qt = q + ((b * T + t) * HK + kh) * dk;
            const double* vt = v + ((b * T + t) * HV + h) * dv;
            const double* gt = g + ((b * T + t) * HV + h) * dk;
            const double bt = beta[(b * T + t) * HV + h];
            double* ot = o + ((b * T + t) * HV + h) * dv;
            /* decay */
            for (int64_t i = 0; i < dk; ++i) {
                const double e = exp(gt[i]);
                double* Si = S + i * dv;
                for (int64_t j = 0; j < dv; ++j) Si[j] *= e;
            }
            /* predict from the decayed state */
            for (int64_t j = 0; j < dv; ++j) pred[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i) {
                const double ki = kt[i];
                const double* Si = S + i * dv;
                for (int64_t j = 0; j < dv; ++j) pred[j] += ki * Si[j];
            }
            /* rank-one delta update */
            for (int64_t j = 0; j < dv; ++j) d[j] = bt * (vt[j] - pred[j]);
            for (int64_t i = 0; i < dk; ++i) {
                const double ki = kt[i];
                double* Si = S + i * dv;
                for (int64_t j = 0; j < dv; ++j) Si[j] += ki * d[j];
            }
            /* output from the node's updated state */
            for (int64_t j = 0; j < dv; ++j) ot[j] = 0.0;
            for (int64_t i = 0; i < dk; ++i) {
                const double qi = qt[i];
                const double* Si = S + i * dv;
                for (int64_t j = 0; j < dv; ++j) ot[j] += qi * Si[j];
            }
        }
        free(states);
    }
    return failed ? -2 : 0;
}
