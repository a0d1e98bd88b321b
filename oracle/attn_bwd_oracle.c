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
