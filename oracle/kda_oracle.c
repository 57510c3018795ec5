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

/* Threads of the calls that follow (n >= 1; for timing the oracle on one core).  Returns the
 * previous count. */
int kda_oracle_set_threads(int n)
{
    const int old = kda_oracle_threads();
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#endif
    return old;
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

/*
 * Gradients of the same recurrence (reverse mode, written out by hand), for the
 * backward pass of training ("zero-intrusion to upper-layer training scripts",
 * "Breaking Through Trillion-Parameter Multimodal MoE", sec. 2.1: the operator
 * must give the gradients of exactly the forward above).
 *
 * The scalar objective is L = sum_t dout_t . o_t + <dfinal, S_T>, so dout and
 * dfinal (NULL: zero) are the incoming gradients of out and final_state.  With
 * the forward of one token written as
 *     St = S_{t-1} diag(d_t),  d_t = exp(g_t)     (decay)
 *     y  = St k_t,  e = beta_t (v_t - y)          (erase coefficient and write)
 *     S_t = St + e k_t^T,  o_t = S_t q_t,
 * the adjoint runs t = T .. 1 carrying dS = dL/dS_t:
 *     dS += dout_t q_t^T;        dq_t = S_t^T dout_t
 *     de = dS k_t;               dk_t  = dS^T e            (from S_t = St + e k^T)
 *     dbeta_t = de . (v_t - y);  dv_t  = beta_t de;  dy = -beta_t de
 *     dSt = dS + dy k_t^T;       dk_t += St^T dy           (from y = St k)
 *     dg_t[c] = sum_i dSt[i][c] St[i][c]                   (from St = S_{t-1} diag(e^g))
 *     dS = dSt diag(d_t)                                   (dL/dS_{t-1})
 * and da = dg * dg/da: g_min sigmoid(a) (1 - sigmoid(a)) for the bounded gate,
 * 1 - sigmoid(a) for log sigmoid(a).  dS0 = dS after t = 1.
 *
 * Rows of S stay independent, so each row's trajectory is recomputed block by
 * block from per-row checkpoints (every 64 tokens) and run backwards; dq, dk,
 * dbeta and dg are sums over rows (OpenMP reductions per block).
 * Layouts as the forward; dq, dk, da: [B][H][T][dk]; dv: [B][H][T][dv];
 * dbeta: [B][H][T]; dS0 (NULL: not wanted): [B][H][dv][dk].
 */
static double oracle_dgate(double a, double g_min, int mode)
{
    const double s = 1.0 / (1.0 + exp(-a));
    if (mode == ORACLE_GATE_BOUNDED) return g_min * s * (1.0 - s);
    return 1.0 - s;
}

int kda_oracle_backward(const double *q, const double *k, const double *v,
                        const double *a, const double *beta,
                        long B, long H, long T, long dk, long dv,
                        double g_min, int gate_mode, const double *S0,
                        const double *dout, const double *dfinal,
                        double *dq, double *dk_out, double *dv_out, double *da,
                        double *dbeta, double *dS0)
{
    if (!q || !k || !v || !a || !beta || !dout || !dq || !dk_out || !dv_out || !da || !dbeta) return -1;
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) return -1;
    if (gate_mode != ORACLE_GATE_BOUNDED && gate_mode != ORACLE_GATE_LOGSIGMOID) return -1;

    const long TB = 64;
    const long NB = (T + TB - 1) / TB;
    double *decay = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * (size_t)dk);
    double *ck = (double *)malloc(sizeof(double) * (size_t)(NB > 0 ? NB : 1) * (size_t)dv * (size_t)dk);
    double *dS = (double *)malloc(sizeof(double) * (size_t)dv * (size_t)dk);
    double *bq = (double *)malloc(sizeof(double) * (size_t)TB * (size_t)dk);
    double *bk = (double *)malloc(sizeof(double) * (size_t)TB * (size_t)dk);
    double *bg = (double *)malloc(sizeof(double) * (size_t)TB * (size_t)dk);
    double *bb = (double *)malloc(sizeof(double) * (size_t)TB);
    if (!decay || !ck || !dS || !bq || !bk || !bg || !bb) {
        free(decay); free(ck); free(dS); free(bq); free(bk); free(bg); free(bb);
        return -2;
    }
    int rc = 0;
    for (long bh = 0; bh < B * H && rc == 0; ++bh) {
        const double *qh = q + bh * T * dk, *kh = k + bh * T * dk, *ah = a + bh * T * dk;
        const double *vh = v + bh * T * dv, *bth = beta + bh * T, *doh = dout + bh * T * dv;

        #pragma omp parallel for schedule(static)
        for (long x = 0; x < T * dk; ++x) decay[x] = exp(oracle_gate(ah[x], g_min, gate_mode));

        /* per-row forward, keeping S at the start of every block */
        #pragma omp parallel for schedule(static)
        for (long i = 0; i < dv; ++i) {
            double *row = (double *)malloc(sizeof(double) * (size_t)dk);
            if (!row) continue;
            for (long j = 0; j < dk; ++j) row[j] = S0 ? S0[(bh * dv + i) * dk + j] : 0.0;
            for (long t = 0; t < T; ++t) {
                if (t % TB == 0) memcpy(ck + ((t / TB) * dv + i) * dk, row, sizeof(double) * (size_t)dk);
                const double *kt = kh + t * dk, *dt = decay + t * dk;
                double y = 0.0;
                for (long j = 0; j < dk; ++j) { row[j] *= dt[j]; y += row[j] * kt[j]; }
                const double e = bth[t] * (vh[t * dv + i] - y);
                for (long j = 0; j < dk; ++j) row[j] += e * kt[j];
            }
            free(row);
        }

        for (long x = 0; x < dv * dk; ++x) dS[x] = dfinal ? dfinal[bh * dv * dk + x] : 0.0;

        for (long nb = NB - 1; nb >= 0; --nb) {
            const long t0 = nb * TB, n = (T - t0 < TB) ? (T - t0) : TB;
            memset(bq, 0, sizeof(double) * (size_t)(n * dk));
            memset(bk, 0, sizeof(double) * (size_t)(n * dk));
            memset(bg, 0, sizeof(double) * (size_t)(n * dk));
            memset(bb, 0, sizeof(double) * (size_t)n);
            const long nd = n * dk;
            int failed = 0;
            #pragma omp parallel reduction(+ : bq[:nd], bk[:nd], bg[:nd], bb[:n]) reduction(| : failed)
            {
                double *St = (double *)malloc(sizeof(double) * (size_t)nd);  /* S_{t-1} diag(d_t), row i */
                double *Sn = (double *)malloc(sizeof(double) * (size_t)nd);  /* S_t, row i */
                double *yv = (double *)malloc(sizeof(double) * (size_t)n);
                double *ev = (double *)malloc(sizeof(double) * (size_t)n);
                double *ds = (double *)malloc(sizeof(double) * (size_t)dk);
                if (!St || !Sn || !yv || !ev || !ds) failed = 1;
                #pragma omp for schedule(static)
                for (long i = 0; i < dv; ++i) {
                    if (failed) continue;
                    /* recompute the row over the block */
                    const double *c0 = ck + (nb * dv + i) * dk;
                    for (long tt = 0; tt < n; ++tt) {
                        const long t = t0 + tt;
                        const double *kt = kh + t * dk, *dt = decay + t * dk;
                        const double *prev = tt ? Sn + (tt - 1) * dk : c0;
                        double *st = St + tt * dk, *sn = Sn + tt * dk;
                        double y = 0.0;
                        for (long j = 0; j < dk; ++j) { st[j] = prev[j] * dt[j]; y += st[j] * kt[j]; }
                        const double e = bth[t] * (vh[t * dv + i] - y);
                        for (long j = 0; j < dk; ++j) sn[j] = st[j] + e * kt[j];
                        yv[tt] = y;
                        ev[tt] = e;
                    }
                    /* and backwards */
                    memcpy(ds, dS + i * dk, sizeof(double) * (size_t)dk);
                    for (long tt = n - 1; tt >= 0; --tt) {
                        const long t = t0 + tt;
                        const double *kt = kh + t * dk, *qt = qh + t * dk, *dt = decay + t * dk;
                        const double *st = St + tt * dk, *sn = Sn + tt * dk;
                        const double bt = bth[t], dot = doh[t * dv + i];
                        double de = 0.0;
                        for (long j = 0; j < dk; ++j) {
                            ds[j] += dot * qt[j];
                            bq[tt * dk + j] += dot * sn[j];
                            de += ds[j] * kt[j];
                        }
                        for (long j = 0; j < dk; ++j) bk[tt * dk + j] += ev[tt] * ds[j];
                        bb[tt] += de * (vh[t * dv + i] - yv[tt]);
                        dv_out[bh * T * dv + t * dv + i] = bt * de;
                        const double dy = -bt * de;
                        for (long j = 0; j < dk; ++j) {
                            ds[j] += dy * kt[j];
                            bk[tt * dk + j] += dy * st[j];
                            bg[tt * dk + j] += ds[j] * st[j];
                            ds[j] *= dt[j];
                        }
                    }
                    memcpy(dS + i * dk, ds, sizeof(double) * (size_t)dk);
                }
                free(St); free(Sn); free(yv); free(ev); free(ds);
            }
            if (failed) { rc = -2; break; }
            for (long tt = 0; tt < n; ++tt) {
                const long t = t0 + tt;
                for (long j = 0; j < dk; ++j) {
                    dq[bh * T * dk + t * dk + j] = bq[tt * dk + j];
                    dk_out[bh * T * dk + t * dk + j] = bk[tt * dk + j];
                    da[bh * T * dk + t * dk + j] = bg[tt * dk + j] * oracle_dgate(ah[t * dk + j], g_min, gate_mode);
                }
                dbeta[bh * T + t] = bb[tt];
            }
        }
        if (dS0) memcpy(dS0 + bh * dv * dk, dS, sizeof(double) * (size_t)(dv * dk));
    }
    free(decay); free(ck); free(dS); free(bq); free(bk); free(bg); free(bb);
    return rc;
}
