/* Runs every entry of the fp64 oracle (oracle/*.c) on small inputs, built
 * with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_sanitizers.py): ragged and one-row shapes, GQA, causal and not,
 * bf16 and fp32, rows and key rows at the ends, a paged cache with empty and
 * full sequences, and rejected arguments.  A sanitizer report or a failed
 * check ends the program with a nonzero status.  Test-side code only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int tessera_oracle_attn_fwd(const void *, const void *, const void *, int, int, int, int, int,
                            int, int, double, double *, double *, int);
int tessera_oracle_attn_fwd_kv(const void *, const void *, const void *, int, int, int, int, int,
                               int, int, int, double, double *, double *, int);
int tessera_oracle_attn_rows(const void *, const void *, const void *, int, int, int, int, int,
                             int, int, double, const int64_t *, int64_t, double *, double *, int);
int tessera_oracle_attn_probs(const void *, const void *, const void *, int, int, int, int, int,
                              int, int, double, double *, double *, double *);
int tessera_oracle_attn_bwd(const uint16_t *, const uint16_t *, const uint16_t *,
                            const uint16_t *, int, int, int, int, int, int, double, double *,
                            double *, double *, double *);
int tessera_oracle_attn_bwd_rows(const uint16_t *, const uint16_t *, const uint16_t *,
                                 const uint16_t *, int, int, int, int, int, int, double,
                                 const int64_t *, int64_t, const int64_t *, int64_t, double *,
                                 double *, double *, double *);
int tessera_oracle_paged_decode(const uint16_t *, const uint16_t *, const uint16_t *,
                                const int32_t *, const int32_t *, int, int, int, int, int, int,
                                int, int, int, double, double *, double *);
int tessera_oracle_rmsnorm(const uint16_t *, const uint16_t *, int64_t, int, double, double *);

static int failures = 0;
static void check(int ok, const char *what)
{
    if (!ok) {
        fprintf(stderr, "FAIL %s\n", what);
        ++failures;
    }
}

/* bf16 bits of a pseudo-random value in about [-2, 2) (a fixed LCG) */
static uint32_t state = 12345u;
static uint16_t rand_bf16(void)
{
    state = state * 1664525u + 1013904223u;
    float f = ((float)(state >> 8) / (float)(1u << 24)) * 4.0f - 2.0f;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static uint16_t *bf16_array(size_t n)
{
    uint16_t *a = malloc(n * sizeof *a);
    for (size_t i = 0; i < n; ++i) a[i] = rand_bf16();
    return a;
}

static int all_finite(const double *a, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(a[i])) return 0;
    return 1;
}

int main(void)
{
    const int shapes[][5] = {{1, 4, 2, 1, 32}, {2, 6, 2, 17, 64}, {1, 4, 4, 33, 128},
                             {3, 8, 1, 9, 16}};
    for (int s = 0; s < 4; ++s) {
        const int B = shapes[s][0], Hq = shapes[s][1], Hkv = shapes[s][2], T = shapes[s][3],
                  D = shapes[s][4];
        const size_t nq = (size_t)B * Hq * T * D, nk = (size_t)B * Hkv * T * D;
        const size_t nl = (size_t)B * Hq * T;
        uint16_t *q = bf16_array(nq), *k = bf16_array(nk), *v = bf16_array(nk),
                 *dout = bf16_array(nq);
        double *O = malloc(nq * 8), *lse = malloc(nl * 8), *P = malloc(nl * T * 8);
        for (int causal = 0; causal <= 1; ++causal) {
            check(tessera_oracle_attn_fwd(q, k, v, 1, B, Hq, Hkv, T, D, causal, 0.3, O, lse, 2) ==
                      0, "fwd");
            check(all_finite(O, nq) && all_finite(lse, nl), "fwd finite");
            check(tessera_oracle_attn_probs(q, k, v, 1, B, Hq, Hkv, T, D, causal, 0.3, O, lse,
                                            P) == 0, "probs");
            for (size_t r = 0; r < nl; ++r) {
                double sum = 0.0;
                for (int j = 0; j < T; ++j) sum += P[r * T + j];
                check(fabs(sum - 1.0) < 1e-12, "probs sum to one");
            }
            const int64_t rows[3] = {0, (int64_t)nl / 2, (int64_t)nl - 1};
            check(tessera_oracle_attn_rows(q, k, v, 1, B, Hq, Hkv, T, D, causal, 0.3, rows, 3, O,
                                           lse, 1) == 0, "rows");
            if (T > 1)
                check(tessera_oracle_attn_fwd_kv(q, k, v, 1, B, Hq, Hkv, T - 1, T, D, causal, 0.3,
                                                 O, lse, 2) == 0, "fwd_kv");
            double *dq = malloc(nq * 8), *dk = malloc(nk * 8), *dv = malloc(nk * 8),
                   *dl = malloc(nl * 8);
            check(tessera_oracle_attn_bwd(q, k, v, dout, B, Hq, Hkv, T, D, causal, 0.3, dq, dk, dv,
                                          dl) == 0, "bwd");
            check(all_finite(dq, nq) && all_finite(dk, nk) && all_finite(dv, nk), "bwd finite");
            const int64_t krows[2] = {0, (int64_t)(B * Hkv * T) - 1};
            check(tessera_oracle_attn_bwd_rows(q, k, v, dout, B, Hq, Hkv, T, D, causal, 0.3, rows,
                                               3, krows, 2, dq, dl, dk, dv) == 0, "bwd rows");
            free(dq);
            free(dk);
            free(dv);
            free(dl);
        }
        /* fp32 inputs */
        float *qf = malloc(nq * 4), *kf = malloc(nk * 4), *vf = malloc(nk * 4);
        for (size_t i = 0; i < nq; ++i) qf[i] = (float)(i % 7) * 0.1f - 0.3f;
        for (size_t i = 0; i < nk; ++i) kf[i] = vf[i] = (float)(i % 5) * 0.2f - 0.4f;
        check(tessera_oracle_attn_fwd(qf, kf, vf, 0, B, Hq, Hkv, T, D, 1, 0.5, O, lse, 1) == 0,
              "fwd fp32");
        free(qf);
        free(kf);
        free(vf);
        /* rejected arguments */
        if ((Hq + 1) % Hkv != 0)   /* a group size that does not divide (never reads q) */
            check(tessera_oracle_attn_fwd(q, k, v, 1, B, Hq + 1, Hkv, T, D, 1, 0.3, O, lse, 1) != 0,
                  "bad group");
        check(tessera_oracle_attn_fwd(NULL, k, v, 1, B, Hq, Hkv, T, D, 1, 0.3, O, lse, 1) != 0,
              "null");
        const int64_t bad_row = (int64_t)nl;
        check(tessera_oracle_attn_rows(q, k, v, 1, B, Hq, Hkv, T, D, 1, 0.3, &bad_row, 1, O, lse,
                                       1) != 0, "row out of range");
        free(q);
        free(k);
        free(v);
        free(dout);
        free(O);
        free(lse);
        free(P);
    }

    /* paged decode: 3 sequences (empty, ragged, full) over 16-row blocks */
    {
        const int B = 3, Hq = 4, Hkv = 2, Tq = 2, D = 32, bs = 16, maxb = 4, nblk = 9;
        uint16_t *q = bf16_array((size_t)B * Hq * Tq * D);
        uint16_t *kc = bf16_array((size_t)nblk * Hkv * bs * D);
        uint16_t *vc = bf16_array((size_t)nblk * Hkv * bs * D);
        const int32_t table[3][4] = {{-1, -1, -1, -1}, {3, 0, -1, -1}, {8, 1, 5, 2}};
        const int32_t lens[3] = {0, 20, 64};
        double *O = malloc((size_t)B * Hq * Tq * D * 8), *lse = malloc((size_t)B * Hq * Tq * 8);
        for (int causal = 0; causal <= 1; ++causal)
            check(tessera_oracle_paged_decode(q, kc, vc, &table[0][0], lens, B, Hq, Hkv, Tq, D,
                                              bs, maxb, nblk, causal, 0.2, O, lse) == 0, "paged");
        check(lse[0] == -INFINITY && O[0] == 0.0, "paged empty sequence");
        free(q);
        free(kc);
        free(vc);
        free(O);
        free(lse);
    }

    /* RMSNorm */
    {
        uint16_t *x = bf16_array(5 * 24), *w = bf16_array(24);
        double *y = malloc(5 * 24 * 8);
        check(tessera_oracle_rmsnorm(x, w, 5, 24, 1e-6, y) == 0 && all_finite(y, 5 * 24),
              "rmsnorm");
        check(tessera_oracle_rmsnorm(x, w, 0, 24, 1e-6, y) != 0, "rmsnorm rows");
        free(x);
        free(w);
        free(y);
    }

    if (failures) return 1;
    printf("oracle checks: ok\n");
    return 0;
}
