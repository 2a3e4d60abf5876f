/* oracle_checks.c -- drives the C oracle (oracle/gdn_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer (test infrastructure): packed sequences with empty and one-token
 * members, a unit mask, grouped heads, the backward pass, and rejected arguments. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int gdn_oracle_forward(const double* q, const double* k, const double* v, const double* g, const double* beta,
                       const double* initial_state, const int32_t* cu_seqlens, int B, int T, int Hk, int Hv,
                       int dk, int dv, int N, const unsigned char* unit_mask, int threads, double* o,
                       double* final_state);
int gdn_oracle_backward(const double* q, const double* k, const double* v, const double* g, const double* beta,
                        const double* initial_state, const int32_t* cu_seqlens, int B, int T, int Hk, int Hv,
                        int dk, int dv, int N, const double* d_o, const double* dfinal, int threads, double* dq,
                        double* dkk, double* dvv, double* dg, double* dbeta, double* ds0);

static double* fill(size_t n, unsigned* seed, double lo, double hi) {
    double* x = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) x[i] = lo + (hi - lo) * (rand_r(seed) / (double)RAND_MAX);
    return x;
}

static int finite_all(const double* x, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

int main(void) {
    unsigned seed = 7;
    const int Hk = 2, Hv = 4, dk = 8, dv = 4, N = 4;
    const int32_t cu[5] = {0, 0, 1, 70, 133};  /* empty, one token, 69, 63 */
    const int T = 133;
    double *q = fill((size_t)T * Hk * dk, &seed, -0.3, 0.3), *k = fill((size_t)T * Hk * dk, &seed, -0.3, 0.3);
    double *v = fill((size_t)T * Hv * dv, &seed, -1, 1), *g = fill((size_t)T * Hv, &seed, -1, 0);
    double *beta = fill((size_t)T * Hv, &seed, 0, 1), *s0 = fill((size_t)N * Hv * dk * dv, &seed, -0.1, 0.1);
    double *o = calloc((size_t)T * Hv * dv, sizeof(double)), *fs = calloc((size_t)N * Hv * dk * dv, sizeof(double));
    int fails = 0;
    if (gdn_oracle_forward(q, k, v, g, beta, s0, cu, 1, T, Hk, Hv, dk, dv, N, NULL, 3, o, fs) != 0 ||
        !finite_all(o, (size_t)T * Hv * dv) || !finite_all(fs, (size_t)N * Hv * dk * dv)) {
        fprintf(stderr, "FAIL packed forward\n");
        ++fails;
    }
    unsigned char mask[16] = {1, 0, 1, 0, 0, 1, 1, 0, 1, 1, 1, 1, 0, 0, 0, 1};
    if (gdn_oracle_forward(q, k, v, g, beta, NULL, cu, 1, T, Hk, Hv, dk, dv, N, mask, 2, o, fs) != 0) {
        fprintf(stderr, "FAIL masked forward\n");
        ++fails;
    }
    double *dq = calloc((size_t)T * Hk * dk, sizeof(double)), *dkk = calloc((size_t)T * Hk * dk, sizeof(double));
    double *dvv = calloc((size_t)T * Hv * dv, sizeof(double)), *dg = calloc((size_t)T * Hv, sizeof(double));
    double *db = calloc((size_t)T * Hv, sizeof(double)), *ds0 = calloc((size_t)N * Hv * dk * dv, sizeof(double));
    double *d_o = fill((size_t)T * Hv * dv, &seed, -1, 1), *dfin = fill((size_t)N * Hv * dk * dv, &seed, -1, 1);
    if (gdn_oracle_backward(q, k, v, g, beta, s0, cu, 1, T, Hk, Hv, dk, dv, N, d_o, dfin, 3, dq, dkk, dvv, dg, db,
                            ds0) != 0 || !finite_all(dq, (size_t)T * Hk * dk) || !finite_all(ds0, (size_t)N * Hv * dk * dv)) {
        fprintf(stderr, "FAIL packed backward\n");
        ++fails;
    }
    /* unpacked, T = 0, and malformed offsets (rejected, nothing written) */
    if (gdn_oracle_forward(q, k, v, g, beta, s0, NULL, 1, 0, Hk, Hv, dk, dv, 1, NULL, 1, o, fs) != 0) {
        fprintf(stderr, "FAIL T = 0\n");
        ++fails;
    }
    const int32_t bad1[5] = {0, 50, 20, 70, 133}, bad2[5] = {0, 0, 1, 70, 140}, bad3[5] = {-5, 0, 1, 70, 133};
    const int32_t* bads[3] = {bad1, bad2, bad3};
    for (int i = 0; i < 3; ++i)
        if (gdn_oracle_forward(q, k, v, g, beta, s0, bads[i], 1, T, Hk, Hv, dk, dv, N, NULL, 1, o, fs) == 0 ||
            gdn_oracle_backward(q, k, v, g, beta, s0, bads[i], 1, T, Hk, Hv, dk, dv, N, d_o, dfin, 1, dq, dkk, dvv,
                                dg, db, ds0) == 0) {
            fprintf(stderr, "FAIL malformed offsets %d accepted\n", i);
            ++fails;
        }
    if (gdn_oracle_forward(q, k, v, g, beta, s0, NULL, 1, T, 3, Hv, dk, dv, 1, NULL, 1, o, fs) == 0) {
        fprintf(stderr, "FAIL Hv %% Hk != 0 accepted\n");
        ++fails;
    }
    free(q); free(k); free(v); free(g); free(beta); free(s0); free(o); free(fs);
    free(dq); free(dkk); free(dvv); free(dg); free(db); free(ds0); free(d_o); free(dfin);
    if (fails) return 1;
    printf("oracle checks passed\n");
    return 0;
}
