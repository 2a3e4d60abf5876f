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

/*
 * ---------------------------------------------------------------------------
 * Backward pass: the gradients of a scalar loss L with respect to every input
 * of gdn_oracle_forward, given dL/do (do) and dL/dS_T (dfinal, NULL = zero).
 *
 * This is reverse-mode differentiation of the same per-token steps, taken in
 * reverse token order.  With D = dL/dS_t (everything downstream of S_t):
 *
 *   read-out     o = S_t^T q       D += q do^T            dq += S_t do
 *   correct      S_t = S~ + k u^T  du = D^T k             dk += D u
 *   delta        u = beta (v - p)  dv = beta du           dbeta = du . (v - p)
 *                                  dp = -beta du
 *   predict      p = S~^T k        dS~ = D + k dp^T       dk += S~ dp
 *   decay        S~ = e^g S_{t-1}  dg = <S~, dS~>          D <- e^g dS~
 *
 * where S~ is the decayed state before token t's correction.  After the first
 * token of a sequence, D is dL/dS_0.  The states S_{t-1} the reverse sweep
 * needs are recomputed: the forward pass keeps the state at every 64-token
 * boundary and each 64-token piece is re-run from its boundary state before
 * it is swept backwards.  dq and dk sum over the v-heads that share a q/k
 * head; sequences are independent.
 *
 * Layouts as in gdn_oracle_forward; dq, dk [B,T,Hk,dk], dv [B,T,Hv,dv],
 * dg, dbeta [B,T,Hv], dS0 [N,Hv,dk,dv].  Rows of tokens outside every sequence
 * are left untouched; the dq/dk rows of every sequence are overwritten.
 * ---------------------------------------------------------------------------
 */
#define ORACLE_PIECE 64

/* Forward over tokens [t0, t1) of (row b, v-head h) from state S (updated in place); if `keep` is
 * not NULL, the state after token t0 + i is stored at keep + i * dk * dv. */
static void oracle_run(const double* q, const double* k, const double* v, const double* g,
                       const double* beta, int b, int t0, int t1, int h, int T, int Hk, int Hv,
                       int dk, int dv, double* S, double* p, double* keep)
{
    const int kgrp = h / (Hv / Hk);
    const size_t SS = (size_t)dk * dv;
    (void)q;
    for (int t = t0; t < t1; ++t) {
        const size_t row = (size_t)b * T + t;
        const double* kt = k + (row * Hk + kgrp) * dk;
        const double* vt = v + (row * Hv + h) * dv;
        const double a = exp(g[row * Hv + h]), bt = beta[row * Hv + h];
        for (size_t e = 0; e < SS; ++e) S[e] = a * S[e];
        for (int j = 0; j < dv; ++j) p[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) p[j] += S[(size_t)i * dv + j] * kt[i];
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += kt[i] * bt * (vt[j] - p[j]);
        if (keep) memcpy(keep + (size_t)(t - t0) * SS, S, SS * sizeof(double));
    }
}

int gdn_oracle_backward(const double* q, const double* k, const double* v,
                        const double* g, const double* beta,
                        const double* initial_state, const int32_t* cu_seqlens,
                        int B, int T, int Hk, int Hv, int dk, int dv, int N,
                        const double* d_o, const double* dfinal, int threads,
                        double* dq, double* dkk, double* dvv, double* dg, double* dbeta,
                        double* ds0)
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
    const int G = Hv / Hk;
    const size_t SS = (size_t)dk * dv;
    const int pieces = (T + ORACLE_PIECE - 1) / ORACLE_PIECE;
    /* per thread: checkpoints, one piece of states, the working state, D, dS~, and vectors */
    const size_t per_thread = (size_t)(pieces + 1) * SS + (size_t)ORACLE_PIECE * SS + 3 * SS + 6 * (size_t)dv;
    const int nthreads = threads > 0 ? threads : omp_get_max_threads();
    double* scratch = (double*)malloc((size_t)nthreads * per_thread * sizeof(double));
    if (!scratch) return ORACLE_NO_MEMORY;
    const long groups = (long)N * Hk;

#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (long w = 0; w < groups; ++w) {
        double* ck = scratch + (size_t)omp_get_thread_num() * per_thread;  /* checkpoints */
        double* piece = ck + (size_t)(pieces + 1) * SS;                     /* one piece's states */
        double* S = piece + (size_t)ORACLE_PIECE * SS;
        double* D = S + SS;
        double* dS = D + SS;
        double* p = dS + SS;
        double* u = p + dv;
        double* du = u + dv;
        double* dp = du + dv;
        double* pv = dp + dv;
        const int n = (int)(w / Hk), kh = (int)(w % Hk);
        const int b = cu_seqlens ? 0 : n;
        const int sb = cu_seqlens ? cu_seqlens[n] : 0;
        const int se = cu_seqlens ? cu_seqlens[n + 1] : T;
        for (int t = sb; t < se; ++t) {
            const size_t row = (size_t)b * T + t;
            memset(dq + (row * Hk + kh) * dk, 0, dk * sizeof(double));
            memset(dkk + (row * Hk + kh) * dk, 0, dk * sizeof(double));
        }
        for (int h = kh * G; h < (kh + 1) * G; ++h) {
            const size_t unit = (size_t)n * Hv + h;
            /* forward: the state at every piece boundary */
            if (initial_state) memcpy(S, initial_state + unit * SS, SS * sizeof(double));
            else memset(S, 0, SS * sizeof(double));
            const int np = (se - sb + ORACLE_PIECE - 1) / ORACLE_PIECE;
            for (int c = 0; c < np; ++c) {
                memcpy(ck + (size_t)c * SS, S, SS * sizeof(double));
                const int a0 = sb + c * ORACLE_PIECE;
                const int a1 = a0 + ORACLE_PIECE < se ? a0 + ORACLE_PIECE : se;
                oracle_run(q, k, v, g, beta, b, a0, a1, h, T, Hk, Hv, dk, dv, S, p, NULL);
            }
            /* reverse sweep */
            if (dfinal) memcpy(D, dfinal + unit * SS, SS * sizeof(double));
            else memset(D, 0, SS * sizeof(double));
            for (int c = np - 1; c >= 0; --c) {
                const int a0 = sb + c * ORACLE_PIECE;
                const int a1 = a0 + ORACLE_PIECE < se ? a0 + ORACLE_PIECE : se;
                memcpy(S, ck + (size_t)c * SS, SS * sizeof(double));
                oracle_run(q, k, v, g, beta, b, a0, a1, h, T, Hk, Hv, dk, dv, S, p, piece);
                for (int t = a1 - 1; t >= a0; --t) {
                    const size_t row = (size_t)b * T + t;
                    const double* qt = q + (row * Hk + kh) * dk;
                    const double* kt = k + (row * Hk + kh) * dk;
                    const double* vt = v + (row * Hv + h) * dv;
                    const double* dot = d_o + (row * Hv + h) * dv;
                    const double a = exp(g[row * Hv + h]), bt = beta[row * Hv + h];
                    const double* St = piece + (size_t)(t - a0) * SS;                 /* S_t */
                    const double* Sp = t > a0 ? St - SS : ck + (size_t)c * SS;        /* S_{t-1} */
                    double* dqt = dq + (row * Hk + kh) * dk;
                    double* dkt = dkk + (row * Hk + kh) * dk;
                    /* read-out */
                    for (int i = 0; i < dk; ++i)
                        for (int j = 0; j < dv; ++j) {
                            D[(size_t)i * dv + j] += qt[i] * dot[j];
                            dqt[i] += St[(size_t)i * dv + j] * dot[j];
                        }
                    /* the forward quantities of this token: p = (a S_{t-1})^T k, u */
                    for (int j = 0; j < dv; ++j) p[j] = 0.0;
                    for (int i = 0; i < dk; ++i)
                        for (int j = 0; j < dv; ++j) p[j] += a * Sp[(size_t)i * dv + j] * kt[i];
                    for (int j = 0; j < dv; ++j) {
                        pv[j] = vt[j] - p[j];
                        u[j] = bt * pv[j];
                    }
                    /* correct */
                    for (int j = 0; j < dv; ++j) du[j] = 0.0;
                    for (int i = 0; i < dk; ++i)
                        for (int j = 0; j < dv; ++j) {
                            du[j] += D[(size_t)i * dv + j] * kt[i];
                            dkt[i] += D[(size_t)i * dv + j] * u[j];
                        }
                    /* delta */
                    double db = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        dvv[(row * Hv + h) * dv + j] = bt * du[j];
                        db += du[j] * pv[j];
                        dp[j] = -bt * du[j];
                    }
                    dbeta[row * Hv + h] = db;
                    /* predict and decay */
                    double dgt = 0.0;
                    for (int i = 0; i < dk; ++i)
                        for (int j = 0; j < dv; ++j) {
                            const size_t e = (size_t)i * dv + j;
                            const double st = a * Sp[e];
                            dS[e] = D[e] + kt[i] * dp[j];
                            dkt[i] += st * dp[j];
                            dgt += st * dS[e];
                        }
                    dg[row * Hv + h] = dgt;
                    for (size_t e = 0; e < SS; ++e) D[e] = a * dS[e];
                }
            }
            memcpy(ds0 + unit * SS, D, SS * sizeof(double));
        }
    }
    free(scratch);
    return ORACLE_OK;
}
