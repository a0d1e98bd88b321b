/*
 * attn_oracle.c -- plain fp64 CPU oracle for causal grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the package's smoke check and the bench's
 * CPU-baseline leg use it.  It shares no code with the HIP library.
 *
 * What it computes.  The pages ("Tessera: a from-scratch distillation and
 * serving stack in one repository", section "The kernel set and its torch
 * fallback"; and the README excerpt on topairepos.com, list "Kernels") name a
 * FlashAttention forward kernel with online softmax, causal masking and
 * grouped-query attention, checked against a plain reference.  Online softmax
 * is an exact reformulation, so the oracle computes the plain definition of
 * the result, row by row, in two passes, without any blocking:
 *
 *   G = Hq / Hkv,  query head h reads KV head g = h / G      (contiguous groups)
 *   for every (b, h, i):
 *     J      = { j : 0 <= j <= i }  if causal,  else { 0 .. T-1 }
 *     s_j    = scale * sum_d q[b,h,i,d] * k[b,g,j,d]            (j in J)
 *     m      = max_j s_j
 *     Z      = sum_j exp(s_j - m)
 *     O[b,h,i,:] = sum_j exp(s_j - m) * v[b,g,j,:] / Z
 *     lse[b,h,i] = m + log(Z)                                   (natural log)
 *
 * Subtracting m only protects fp64 from overflow; it does not change the
 * value.  Every input element is widened exactly to double: fp32 directly,
 * bf16 by placing its 16 bits in the top half of an fp32 word.  `scale` is
 * used exactly as given.  Tensors are contiguous, D innermost:
 * q [B,Hq,T,D], k and v [B,Hkv,T,D]; O [B,Hq,T,D] and lse [B,Hq,T] are fp64.
 *
 * A query row with no visible key (impossible for these shapes, since key i
 * is always visible to query i) would get O = 0 and lse = -inf.
 *
 * Continuation of a cached sequence (tessera_oracle_attn_fwd_kv).  The same
 * page, section "Serving: block-paged KV, batch recomposition, speculation",
 * holds that decoding incrementally with the KV cache gives what a full
 * forward pass gives.  With Tq query rows against Tk key rows, query row i
 * stands at sequence position i + Tk - Tq, so the causal key set becomes
 * J = { j : 0 <= j <= i + Tk - Tq } (all Tk keys when not causal); q and O
 * are [B,Hq,Tq,D], k and v [B,Hkv,Tk,D], lse [B,Hq,Tq].  Tq = Tk = T is the
 * definition above.  A causal row with i + Tk - Tq < 0 has no visible key.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_DTYPE_F32 0
#define ORACLE_DTYPE_BF16 1

/* Widen element `idx` of an fp32 or bf16 array to double, exactly. */
static double widen(const void *p, int dtype, int64_t idx)
{
    if (dtype == ORACLE_DTYPE_F32)
        return (double)((const float *)p)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)p)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int check_args(const void *q, const void *k, const void *v, int dtype,
                      int B, int Hq, int Hkv, int Tq, int Tk, int D, int causal)
{
    if (!q || !k || !v) return 1;
    if (dtype != ORACLE_DTYPE_F32 && dtype != ORACLE_DTYPE_BF16) return 2;
    if (B < 1 || Hq < 1 || Hkv < 1 || Tq < 1 || Tk < 1 || D < 1) return 3;
    if (Hq % Hkv != 0) return 4;
    if (causal != 0 && causal != 1) return 5;
    return 0;
}

/*
 * One query row of Tq against Tk keys.  `s` and `p` are caller scratch of Tk
 * doubles each.  Writes D values to `o` and one to `lse`; if `probs` is not
 * NULL it also writes the Tk softmax weights of the row (0 for masked keys).
 */
static void one_row(const void *q, const void *k, const void *v, int dtype,
                    int Hq, int Hkv, int Tq, int Tk, int D, int causal, double scale,
                    int b, int h, int i, double *s, double *p, double *o,
                    double *lse, double *probs)
{
    const int G = Hq / Hkv;
    const int g = h / G;
    const int64_t qrow = (((int64_t)b * Hq + h) * Tq + i) * D;
    const int64_t kv0 = ((int64_t)b * Hkv + g) * Tk * D;
    const int pos = i + (Tk - Tq);          /* sequence position of query row i */
    int n = causal ? pos + 1 : Tk;          /* visible keys are 0 .. n-1 */
    if (n < 0) n = 0;

    /* pass 1: scaled scores and their maximum */
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += widen(q, dtype, qrow + d) * widen(k, dtype, kv0 + (int64_t)j * D + d);
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
    }

    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (n == 0) { /* no visible key */
        *lse = -INFINITY;
        if (probs) for (int j = 0; j < Tk; ++j) probs[j] = 0.0;
        return;
    }

    /* pass 2: normaliser, then the weighted sum of value rows */
    double Z = 0.0;
    for (int j = 0; j < n; ++j) {
        p[j] = exp(s[j] - m);
        Z += p[j];
    }
    for (int j = 0; j < n; ++j) {
        const double w = p[j] / Z;
        for (int d = 0; d < D; ++d)
            o[d] += w * widen(v, dtype, kv0 + (int64_t)j * D + d);
    }
    *lse = m + log(Z);

    if (probs) {
        for (int j = 0; j < Tk; ++j) probs[j] = (j < n) ? p[j] / Z : 0.0;
    }
}

static int resolve_threads(int nthreads)
{
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/*
 * Attention over selected rows.  rows[r] is the flat row index
 * (b*Hq + h)*T + i.  O is nrows x D, lse is nrows.  Returns 0 on success,
 * a positive code for bad arguments, -1 if scratch allocation failed.
 */
int tessera_oracle_attn_rows(const void *q, const void *k, const void *v, int dtype,
                             int B, int Hq, int Hkv, int T, int D, int causal,
                             double scale, const int64_t *rows, int64_t nrows,
                             double *O, double *lse, int nthreads)
{
    int rc = check_args(q, k, v, dtype, B, Hq, Hkv, T, T, D, causal);
    if (rc) return rc;
    if (nrows < 0 || (nrows > 0 && (!rows || !O || !lse))) return 6;
    const int64_t total = (int64_t)B * Hq * T;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= total) return 7;

    int failed = 0;
    const int nt = resolve_threads(nthreads);
#pragma omp parallel num_threads(nt) reduction(| : failed)
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)T);
        double *p = (double *)malloc(sizeof(double) * (size_t)T);
        if (!s || !p) {
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t r = 0; r < nrows; ++r) {
                const int64_t flat = rows[r];
                const int i = (int)(flat % T);
                const int64_t bh = flat / T;
                const int h = (int)(bh % Hq);
                const int b = (int)(bh / Hq);
                one_row(q, k, v, dtype, Hq, Hkv, T, T, D, causal, scale, b, h, i, s, p,
                        O + r * D, lse + r, NULL);
            }
        }
        free(s);
        free(p);
    }
    return failed ? -1 : 0;
}

/* Tq query rows against Tk key rows: O [B,Hq,Tq,D], lse [B,Hq,Tq]. */
int tessera_oracle_attn_fwd_kv(const void *q, const void *k, const void *v, int dtype,
                               int B, int Hq, int Hkv, int Tq, int Tk, int D, int causal,
                               double scale, double *O, double *lse, int nthreads)
{
    int rc = check_args(q, k, v, dtype, B, Hq, Hkv, Tq, Tk, D, causal);
    if (rc) return rc;
    if (!O || !lse) return 6;
    const int64_t total = (int64_t)B * Hq * Tq;

    int failed = 0;
    const int nt = resolve_threads(nthreads);
#pragma omp parallel num_threads(nt) reduction(| : failed)
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)Tk);
        double *p = (double *)malloc(sizeof(double) * (size_t)Tk);
        if (!s || !p) {
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t flat = 0; flat < total; ++flat) {
                const int i = (int)(flat % Tq);
                const int64_t bh = flat / Tq;
                const int h = (int)(bh % Hq);
                const int b = (int)(bh / Hq);
                one_row(q, k, v, dtype, Hq, Hkv, Tq, Tk, D, causal, scale, b, h, i, s, p,
                        O + flat * D, lse + flat, NULL);
            }
        }
        free(s);
        free(p);
    }
    return failed ? -1 : 0;
}

/* Attention over every row: O [B,Hq,T,D], lse [B,Hq,T]. */
int tessera_oracle_attn_fwd(const void *q, const void *k, const void *v, int dtype,
                            int B, int Hq, int Hkv, int T, int D, int causal,
                            double scale, double *O, double *lse, int nthreads)
{
    return tessera_oracle_attn_fwd_kv(q, k, v, dtype, B, Hq, Hkv, T, T, D, causal, scale,
                                      O, lse, nthreads);
}

/* Attention plus the softmax weights P [B,Hq,T,T] (masked keys get 0). */
int tessera_oracle_attn_probs(const void *q, const void *k, const void *v, int dtype,
                              int B, int Hq, int Hkv, int T, int D, int causal,
                              double scale, double *O, double *lse, double *P)
{
    int rc = check_args(q, k, v, dtype, B, Hq, Hkv, T, T, D, causal);
    if (rc) return rc;
    if (!O || !lse || !P) return 6;
    double *s = (double *)malloc(sizeof(double) * (size_t)T);
    double *p = (double *)malloc(sizeof(double) * (size_t)T);
    if (!s || !p) {
        free(s);
        free(p);
        return -1;
    }
    const int64_t total = (int64_t)B * Hq * T;
    for (int64_t flat = 0; flat < total; ++flat) {
        const int i = (int)(flat % T);
        const int64_t bh = flat / T;
        const int h = (int)(bh % Hq);
        const int b = (int)(bh / Hq);
        one_row(q, k, v, dtype, Hq, Hkv, T, T, D, causal, scale, b, h, i, s, p,
                O + flat * D, lse + flat, P + flat * T);
    }
    free(s);
    free(p);
    return 0;
}

/* Threads an OpenMP region would use for `nthreads` (<= 0: all). */
int tessera_oracle_threads(int nthreads)
{
    return resolve_threads(nthreads);
}
