/*
 * attn_bwd_oracle.c -- plain fp64 CPU oracle for the gradients of causal
 * grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests and the bench use it.  It shares no code
 * with the HIP library.
 *
 * What it computes.  The pages say the fused attention backward is missing
 * (page "Tessera: a from-scratch distillation and serving stack in one
 * repository", section "The kernel set and its torch fallback", and the
 * Status list of the README excerpts); the backward of the forward pass in
 * attn_oracle.c is the plain reading.  Given the output gradient dO, with
 * P the softmax weights of the forward pass (query row i, visible keys j):
 *
 *   dP_ij  = dO_i . v_j
 *   Delta_i = sum_j P_ij dP_ij
 *   dS_ij  = P_ij (dP_ij - Delta_i)
 *   dq_i   = scale * sum_j dS_ij k_j
 *   dk_j   = scale * sum over query heads of the group, sum_i dS_ij q_i
 *   dv_j   = sum over query heads of the group, sum_i P_ij dO_i
 *
 * P comes from the oracle's own exact softmax (two passes per row, fp64);
 * no forward output of the GPU enters.  Rows are processed one at a time, so
 * nothing of size T x T is stored.  Every input is widened exactly to double
 * (bf16: its 16 bits in the top half of an fp32 word).  Layouts: q, dO, dq
 * [B,Hq,T,D]; k, v, dk, dv [B,Hkv,T,D]; outputs fp64; Delta [B,Hq,T] fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double wide(const uint16_t *p, int64_t idx)
{
    uint32_t bits = (uint32_t)p[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

int tessera_oracle_attn_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            const uint16_t *dout, int B, int Hq, int Hkv, int T, int D,
                            int causal, double scale, double *dq, double *dk, double *dv,
                            double *delta)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv || !delta) return 1;
    if (B < 1 || Hq < 1 || Hkv < 1 || T < 1 || D < 1 || Hq % Hkv != 0) return 2;
    if (causal != 0 && causal != 1) return 3;
    const int G = Hq / Hkv;
    int failed = 0;
    memset(dk, 0, sizeof(double) * (size_t)B * Hkv * T * D);
    memset(dv, 0, sizeof(double) * (size_t)B * Hkv * T * D);
#pragma omp parallel for collapse(2) schedule(dynamic, 1) reduction(| : failed)
    for (int b = 0; b < B; ++b) {
        for (int g = 0; g < Hkv; ++g) {
            double *s = (double *)malloc(sizeof(double) * (size_t)T);
            double *dp = (double *)malloc(sizeof(double) * (size_t)T);
            if (!s || !dp) {
                failed = 1;
                free(s);
                free(dp);
                continue;
            }
            const int64_t kv0 = ((int64_t)b * Hkv + g) * T * D;
            for (int h = g * G; h < (g + 1) * G; ++h) {
                for (int i = 0; i < T; ++i) {
                    const int64_t qi = (((int64_t)b * Hq + h) * T + i) * D;
                    const int n = causal ? i + 1 : T;
                    /* softmax weights of row i */
                    double m = -INFINITY;
                    for (int j = 0; j < n; ++j) {
                        double dot = 0.0;
                        for (int d = 0; d < D; ++d)
                            dot += wide(q, qi + d) * wide(k, kv0 + (int64_t)j * D + d);
                        s[j] = scale * dot;
                        if (s[j] > m) m = s[j];
                    }
                    double Z = 0.0;
                    for (int j = 0; j < n; ++j) {
                        s[j] = exp(s[j] - m);
                        Z += s[j];
                    }
                    /* s[j] becomes P_ij; dP_ij and Delta_i */
                    double dl = 0.0;
                    for (int j = 0; j < n; ++j) {
                        s[j] /= Z;
                        double dot = 0.0;
                        for (int d = 0; d < D; ++d)
                            dot += wide(dout, qi + d) * wide(v, kv0 + (int64_t)j * D + d);
                        dp[j] = dot;
                        dl += s[j] * dot;
                    }
                    delta[((int64_t)b * Hq + h) * T + i] = dl;
                    for (int d = 0; d < D; ++d) dq[qi + d] = 0.0;
                    for (int j = 0; j < n; ++j) {
                        const double ds = s[j] * (dp[j] - dl);
                        const int64_t kj = kv0 + (int64_t)j * D;
                        for (int d = 0; d < D; ++d) {
                            dq[qi + d] += scale * ds * wide(k, kj + d);
                            dk[kj + d] += scale * ds * wide(q, qi + d);
                            dv[kj + d] += s[j] * wide(dout, qi + d);
                        }
                    }
                }
            }
            free(s);
            free(dp);
        }
    }
    return failed ? -1 : 0;
}

/* Softmax statistics of query row i of head (b, h): its log-sum-exp and
 * Delta_i = sum_j P_ij (dO_i . v_j), from the row's own scores. */
static void row_stats(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                      const uint16_t *dout, int Hq, int Hkv, int T, int D, int causal,
                      double scale, int b, int h, int i, double *s, double *lse_out,
                      double *delta_out)
{
    const int G = Hq / Hkv;
    const int64_t qi = (((int64_t)b * Hq + h) * T + i) * D;
    const int64_t kv0 = ((int64_t)b * Hkv + h / G) * T * D;
    const int n = causal ? i + 1 : T;
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += wide(q, qi + d) * wide(k, kv0 + (int64_t)j * D + d);
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
    }
    double Z = 0.0;
    for (int j = 0; j < n; ++j) Z += exp(s[j] - m);
    const double lse = m + log(Z);
    double dl = 0.0;
    for (int j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += wide(dout, qi + d) * wide(v, kv0 + (int64_t)j * D + d);
        dl += exp(s[j] - lse) * dot;
    }
    *lse_out = lse;
    *delta_out = dl;
}

/* The same gradients for selected rows only, each from the definitions
 * above: dq and Delta of query rows qrows[] (flat index (b*Hq + h)*T + i)
 * and dk, dv of key rows krows[] (flat index (b*Hkv + g)*T + j).  A key
 * row's gradients need the log-sum-exp and Delta of every query row of its
 * group, which are computed once per (b, query head) that a key row needs.
 * Outputs: dq_rows [nq, D], delta_rows [nq], dk_rows and dv_rows [nk, D]. */
int tessera_oracle_attn_bwd_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                 const uint16_t *dout, int B, int Hq, int Hkv, int T, int D,
                                 int causal, double scale, const int64_t *qrows, int64_t nq,
                                 const int64_t *krows, int64_t nk, double *dq_rows,
                                 double *delta_rows, double *dk_rows, double *dv_rows)
{
    if (!q || !k || !v || !dout || (nq && (!qrows || !dq_rows || !delta_rows)) ||
        (nk && (!krows || !dk_rows || !dv_rows)))
        return 1;
    if (B < 1 || Hq < 1 || Hkv < 1 || T < 1 || D < 1 || Hq % Hkv != 0 || nq < 0 || nk < 0)
        return 2;
    if (causal != 0 && causal != 1) return 3;
    for (int64_t r = 0; r < nq; ++r)
        if (qrows[r] < 0 || qrows[r] >= (int64_t)B * Hq * T) return 4;
    for (int64_t r = 0; r < nk; ++r)
        if (krows[r] < 0 || krows[r] >= (int64_t)B * Hkv * T) return 4;
    const int G = Hq / Hkv;
    int failed = 0;

    /* query rows */
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int64_t r = 0; r < nq; ++r) {
        double *s = (double *)malloc(sizeof(double) * (size_t)T);
        if (!s) {
            failed = 1;
            continue;
        }
        const int i = (int)(qrows[r] % T);
        const int h = (int)((qrows[r] / T) % Hq);
        const int b = (int)(qrows[r] / ((int64_t)T * Hq));
        double lse, dl;
        row_stats(q, k, v, dout, Hq, Hkv, T, D, causal, scale, b, h, i, s, &lse, &dl);
        const int64_t qi = qrows[r] * D;
        const int64_t kv0 = ((int64_t)b * Hkv + h / G) * T * D;
        const int n = causal ? i + 1 : T;
        double *o = dq_rows + r * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        for (int j = 0; j < n; ++j) {
            double dot = 0.0;
            for (int d = 0; d < D; ++d) dot += wide(dout, qi + d) * wide(v, kv0 + (int64_t)j * D + d);
            const double ds = exp(s[j] - lse) * (dot - dl);
            for (int d = 0; d < D; ++d) o[d] += scale * ds * wide(k, kv0 + (int64_t)j * D + d);
        }
        delta_rows[r] = dl;
        free(s);
    }
    if (nk == 0 || failed) return failed ? -1 : 0;

    /* key rows: statistics of the query rows of every (b, query head) involved */
    char *need = (char *)calloc((size_t)B * Hq, 1);
    double *lse_all = (double *)malloc(sizeof(double) * (size_t)B * Hq * T);
    double *dl_all = (double *)malloc(sizeof(double) * (size_t)B * Hq * T);
    if (!need || !lse_all || !dl_all) {
        free(need);
        free(lse_all);
        free(dl_all);
        return -1;
    }
    for (int64_t r = 0; r < nk; ++r) {
        const int64_t bg = krows[r] / T;
        for (int h = (int)(bg % Hkv) * G; h < (int)(bg % Hkv + 1) * G; ++h)
            need[(bg / Hkv) * Hq + h] = 1;
    }
    for (int64_t bh = 0; bh < (int64_t)B * Hq; ++bh) {
        if (!need[bh]) continue;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : failed)
        for (int i = 0; i < T; ++i) {
            double *s = (double *)malloc(sizeof(double) * (size_t)T);
            if (!s) {
                failed = 1;
                continue;
            }
            row_stats(q, k, v, dout, Hq, Hkv, T, D, causal, scale, (int)(bh / Hq), (int)(bh % Hq),
                      i, s, &lse_all[bh * T + i], &dl_all[bh * T + i]);
            free(s);
        }
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nk; ++r) {
        const int j = (int)(krows[r] % T);
        const int64_t bg = krows[r] / T;
        const int g = (int)(bg % Hkv), b = (int)(bg / Hkv);
        const int64_t kj = krows[r] * D;
        double *ok = dk_rows + r * D, *ov = dv_rows + r * D;
        for (int d = 0; d < D; ++d) ok[d] = ov[d] = 0.0;
        for (int h = g * G; h < (g + 1) * G; ++h) {
            const int64_t bh = (int64_t)b * Hq + h;
            for (int i = causal ? j : 0; i < T; ++i) {
                const int64_t qi = (bh * T + i) * D;
                double sdot = 0.0, pdot = 0.0;
                for (int d = 0; d < D; ++d) {
                    sdot += wide(q, qi + d) * wide(k, kj + d);
                    pdot += wide(dout, qi + d) * wide(v, kj + d);
                }
                const double p = exp(scale * sdot - lse_all[bh * T + i]);
                const double ds = p * (pdot - dl_all[bh * T + i]);
                for (int d = 0; d < D; ++d) {
                    ok[d] += scale * ds * wide(q, qi + d);
                    ov[d] += p * wide(dout, qi + d);
                }
            }
        }
    }
    free(need);
    free(lse_all);
    free(dl_all);
    return failed ? -1 : 0;
}
