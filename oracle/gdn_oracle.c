/*
 * gdn_oracle.c -- the gated delta rule, written out token by token in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the GPU path is
 * checked against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header or constant with
 * the HIP library, and the library never calls it.
 *
 * What it computes (the plain definition, no chunking, no reordering):
 *
 *   Qwen3.5 Gated DeltaNet core-mechanism write-up (wanger-sjtu.github.io),
 *   flowchart node "Delta Rule State Update and Retrieval" and the section
 *   "Core mechanism: Gated DeltaNet": the state is not simply accumulated as
 *   in linear attention; it is corrected along the current key.  With the
 *   gates of the same flowchart (beta = sigmoid(b) is the write strength,
 *   g <= 0 is the log-decay), the correction written out per token t is
 *
 *       S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *       o_t = S_t^T q_t
 *
 *   evaluated in the equivalent order "decay, predict, correct, read":
 *
 *       S  <- exp(g_t) S
 *       p  <- S^T k_t                  (what the decayed state recalls for k_t)
 *       u  <- beta_t (v_t - p)          (the delta, scaled by the write strength)
 *       S  <- S + k_t u^T
 *       o_t <- S^T q_t                  (read-out after this token's update)
 *
 *   The two entry points named in the Qwen3-Next Gated DeltaNet article
 *   (jsqmd.com, section 2.2 "chunked parallel computation") are both this
 *   recurrence: chunk_gated_delta_rule over a whole segment with an optional
 *   initial state, recurrent_gated_delta_rule for one token against a cached
 *   state.  Both are served by gdn_oracle_forward below (a decode step is a
 *   batch of length-1 sequences).
 *
 * Readings where the pages are silent:
 *   - no query scale (o_t = S_t^T q_t exactly);
 *   - v-head h reads q/k head floor(h / (Hv / Hk)) (contiguous grouping);
 *   - a missing initial state means zeros (the article's segment loop passes
 *     None for the first segment);
 *   - packed sequences never interact; a zero-length sequence returns its
 *     initial state unchanged.
 *
 * Layouts (all row-major, innermost index last):
 *   q, k  [B, T, Hk, dk]      v, o [B, T, Hv, dv]      g, beta [B, T, Hv]
 *   initial_state, final_state [N, Hv, dk, dv]
 *   cu_seqlens [N+1] (int32, only with B == 1) or NULL (then N == B and
 *   sequence n is batch row n, all T tokens).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARGS 1
#define ORACLE_NO_MEMORY 2

/* One (sequence, v-head) unit: tokens [t0, t1) of batch row b. */
static void oracle_unit(const double* q, const double* k, const double* v,
                        const double* g, const double* beta,
                        const double* s0, int b, int t0, int t1, int h,
                        int T, int Hk, int Hv, int dk, int dv,
                        double* S, double* p, double* u,
                        double* o, double* s_out)
{
    const int kh = h / (Hv / Hk);
    const size_t SS = (size_t)dk * dv;
    if (s0) memcpy(S, s0, SS * sizeof(double));
    else memset(S, 0, SS * sizeof(double));

    for (int t = t0; t < t1; ++t) {
        const size_t row = (size_t)b * T + t;                 /* token index */
        const double* qt = q + (row * Hk + kh) * dk;
        const double* kt = k + (row * Hk + kh) * dk;
        const double* vt = v + (row * Hv + h) * dv;
        const double gt = g[row * Hv + h];
        const double bt = beta[row * Hv + h];
        double* ot = o + (row * Hv + h) * dv;

        /* decay */
        const double a = exp(gt);
        for (size_t e = 0; e < SS; ++e) S[e] *= a;

        /* predict: p = S^T k */
        for (int j = 0; j < dv; ++j) p[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double ki = kt[i];
            const double* Si = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j) p[j] += Si[j] * ki;
        }

        /* delta: u = beta (v - p) */
        for (int j = 0; j < dv; ++j) u[j] = bt * (vt[j] - p[j]);

        /* correct: S += k u^T */
        for (int i = 0; i < dk; ++i) {
            const double ki = kt[i];
            double* Si = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j) Si[j] += ki * u[j];
        }

        /* read out: o = S^T q */
        for (int j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double qi = qt[i];
            const double* Si = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j) ot[j] += Si[j] * qi;
        }
    }
    memcpy(s_out, S, SS * sizeof(double));
}

/*
 * Runs the recurrence for every (sequence, v-head) unit.  `unit_mask`, when
 * not NULL, holds N*Hv bytes; units whose byte is zero are skipped (their o
 * rows and final state are left untouched), which lets a caller evaluate a
 * sample of a large workload.  `threads` <= 0 lets OpenMP choose.
 */
int gdn_oracle_forward(const double* q, const double* k, const double* v,
                       const double* g, const double* beta,
                       const double* initial_state, const int32_t* cu_seqlens,
                       int B, int T, int Hk, int Hv, int dk, int dv, int N,
                       const unsigned char* unit_mask, int threads,
                       double* o, double* final_state)
{
    if (B < 1 || T < 0 || Hk < 1 || Hv < 1 || dk < 1 || dv < 1 || N < 1)
        return ORACLE_BAD_ARGS;
    if (Hv % Hk != 0) return ORACLE_BAD_ARGS;
    if (cu_seqlens) {
        if (B != 1 || cu_seqlens[0] != 0 || cu_seqlens[N] != T) return ORACLE_BAD_ARGS;
        for (int n = 0; n < N; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return ORACLE_BAD_ARGS;
    } else if (N != B) {
        return ORACLE_BAD_ARGS;
    }

    const size_t SS = (size_t)dk * dv;
    const long units = (long)N * Hv;
    const int nthreads = threads > 0 ? threads : omp_get_max_threads();
    const size_t per_thread = SS + 2 * (size_t)dv;
    double* scratch = (double*)malloc((size_t)nthreads * per_thread * sizeof(double));
    if (!scratch) return ORACLE_NO_MEMORY;

#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (long w = 0; w < units; ++w) {
        if (unit_mask && !unit_mask[w]) continue;
        double* S = scratch + (size_t)omp_get_thread_num() * per_thread;
        const int n = (int)(w / Hv), h = (int)(w % Hv);
        const int b = cu_seqlens ? 0 : n;
        const int t0 = cu_seqlens ? cu_seqlens[n] : 0;
        const int t1 = cu_seqlens ? cu_seqlens[n + 1] : T;
        const double* s0 = initial_state ? initial_state + (size_t)w * SS : NULL;
        oracle_unit(q, k, v, g, beta, s0, b, t0, t1, h, T, Hk, Hv, dk, dv,
                    S, S + SS, S + SS + dv, o, final_state + (size_t)w * SS);
    }
    free(scratch);
    return ORACLE_OK;
}

/* The number of threads gdn_oracle_forward uses when `threads` <= 0. */
int gdn_oracle_default_threads(void) { return omp_get_max_threads(); }
