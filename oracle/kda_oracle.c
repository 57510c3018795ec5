/*
 * Plain float64 CPU oracle for the bounded-decay KDA (delta-rule) forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or constant with the GPU library.
 *
 * What it computes (the definition, token by token, no chunking):
 *
 *   gate (per token t, key channel c):
 *     bounded     g = g_min * sigmoid(a)         "Trillion-Scale MoE Multimodal
 *                                                Models: Practical Techniques ...",
 *                                                sec. 3.2 (first displayed formula,
 *                                                g_min = -5); "Breaking Through
 *                                                Trillion-Parameter Multimodal MoE",
 *                                                sec. 2.1 (g_t = g_min * sigma(.)).
 *     logsigmoid  g = log sigmoid(a) = -softplus(-a)   the unbounded form the
 *                                                same sections replace (used only
 *                                                for the ablation).
 *
 *   state S (dv x dk, row i = value channel, column j = key channel), S_0 = 0
 *   or a caller-given initial state; for each token t:
 *     S <- S * diag(exp g_t)                      decay of every key column
 *     S <- S - beta_t * (S k_t) k_t^T             erase along k_t  (delta rule,
 *                                                "Delta Net" in sec. 2.1 of the
 *                                                third page)
 *     S <- S + beta_t * v_t k_t^T                 write
 *     o_t = S q_t                                 read
 *   so S_t = S_{t-1} diag(exp g_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T.
 *
 * Row i of S only ever touches row i, so rows are computed independently (and
 * in parallel with OpenMP); within a row the four steps above are written out
 * literally.  erase = 0 drops the erase step (plain decayed linear attention);
 * it exists only for the oracle's self-checks.
 *
 * Layouts: q, k, a: [B][H][T][dk]; v, out: [B][H][T][dv]; beta: [B][H][T];
 * S0 and final_state: [B][H][dv][dk].  All arrays are float64, row-major.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_GATE_BOUNDED = 0, ORACLE_GATE_LOGSIGMOID = 1 };

static double oracle_gate(double a, double g_min, int mode)
{
    if (mode == ORACLE_GATE_BOUNDED)
        return g_min / (1.0 + exp(-a));
    /* log(sigmoid(a)) = -(max(-a, 0) + log1p(exp(-|a|))): no overflow for any a */
    return -(fmax(-a, 0.0) + log1p(exp(-fabs(a))));
}

int kda_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Returns 0 on success, -1 on bad arguments, -2 on allocation failure. */
int kda_oracle_recurrent(const double *q, const double *k, const double *v,
                         const double *a, const double *beta,
                         long B, long H, long T, long dk, long dv,
                         double g_min, int gate_mode, int erase,
                         const double *S0, double *out, double *final_state)
{
    if (!q || !k || !v || !a || !beta || !out) return -1;
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) return -1;
    if (gate_mode != ORACLE_GATE_BOUNDED && gate_mode != ORACLE_GATE_LOGSIGMOID) return -1;

    const long TB = 256; /* tokens whose decay factors are computed together */
    double *decay = (double *)malloc(sizeof(double) * (size_t)TB * (size_t)dk);
    double *S = (double *)malloc(sizeof(double) * (size_t)dv * (size_t)dk);
    if (!decay || !S) { free(decay); free(S); return -2; }

    for (long bh = 0; bh < B * H; ++bh) {
        const double *qh = q + bh * T * dk, *kh = k + bh * T * dk, *ah = a + bh * T * dk;
        const double *vh = v + bh * T * dv, *bth = beta + bh * T;
        double *oh = out + bh * T * dv;

        if (S0) memcpy(S, S0 + bh * dv * dk, sizeof(double) * (size_t)(dv * dk));
        else memset(S, 0, sizeof(double) * (size_t)(dv * dk));

        for (long t0 = 0; t0 < T; t0 += TB) {
            long nt = (T - t0 < TB) ? (T - t0) : TB;
            #pragma omp parallel for schedule(static)
            for (long x = 0; x < nt * dk; ++x)
                decay[x] = exp(oracle_gate(ah[t0 * dk + x], g_min, gate_mode));

            #pragma omp parallel for schedule(static)
            for (long i = 0; i < dv; ++i) {
                double *row = S + i * dk; /* S[i][:] */
                for (long tt = 0; tt < nt; ++tt) {
                    long t = t0 + tt;
                    const double *kt = kh + t * dk, *qt = qh + t * dk, *dt = decay + tt * dk;
                    const double bt = bth[t];
                    /* decay: S[i][j] *= exp(g_t[j]) */
                    for (long j = 0; j < dk; ++j) row[j] *= dt[j];
                    /* erase: S[i][:] -= beta_t * (S[i][:] . k_t) * k_t */
                    if (erase) {
                        double sk = 0.0;
                        for (long j = 0; j < dk; ++j) sk += row[j] * kt[j];
                        for (long j = 0; j < dk; ++j) row[j] -= bt * sk * kt[j];
                    }
                    /* write: S[i][:] += beta_t * v_t[i] * k_t */
                    const double w = bt * vh[t * dv + i];
                    for (long j = 0; j < dk; ++j) row[j] += w * kt[j];
                    /* read: o_t[i] = S[i][:] . q_t */
                    double o = 0.0;
                    for (long j = 0; j < dk; ++j) o += row[j] * qt[j];
                    oh[t * dv + i] = o;
                }
            }
        }
        if (final_state) memcpy(final_state + bh * dv * dk, S, sizeof(double) * (size_t)(dv * dk));
    }
    free(decay);
    free(S);
    return 0;
}
