/*
 * paged_oracle.c -- plain fp64 CPU oracle for attention decode over a
 * block-paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests and the bench use it.  It shares no code
 * with the HIP library.
 *
 * What it computes.  The serving section of the page "Tessera: a
 * from-scratch distillation and serving stack in one repository" ("Serving:
 * block-paged KV, batch recomposition, speculation") describes a block-paged
 * KV cache, and the pages list a fused paged-attention decode kernel as not
 * yet done.  The pages give no block-table layout; the reading used here:
 *
 *   k_cache, v_cache [num_blocks, Hkv, block_size, D]   (bf16 patterns)
 *   block_table      [B, max_blocks]  (int32 physical block of each logical one)
 *   context_lens     [B]              (int32 tokens in the cache, new ones included)
 *
 * Token t of sequence b lives in block block_table[b, t / block_size], row
 * t % block_size.  The Tq query rows of sequence b are its last Tq tokens:
 * row i stands at position n_b - Tq + i (n_b = context_lens[b]) and, with
 * causal = 1, sees tokens 0 .. n_b - Tq + i; with causal = 0 all n_b.  The
 * result is the attention definition of attn_oracle.c over the gathered
 * rows: q, O [B,Hq,Tq,D], lse [B,Hq,Tq], KV head h / (Hq / Hkv).  A row with
 * no visible token gets O = 0 and lse = -inf.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double widen16(const uint16_t *p, int64_t idx)
{
    uint32_t bits = (uint32_t)p[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

int tessera_oracle_paged_decode(const uint16_t *q, const uint16_t *k_cache,
                                const uint16_t *v_cache, const int32_t *block_table,
                                const int32_t *context_lens, int B, int Hq, int Hkv, int Tq,
                                int D, int block_size, int max_blocks, int num_blocks,
                                int causal, double scale, double *O, double *lse)
{
    if (!q || !k_cache || !v_cache || !block_table || !context_lens || !O || !lse) return 1;
    if (B < 1 || Hq < 1 || Hkv < 1 || Tq < 1 || D < 1 || block_size < 1 || max_blocks < 1 ||
        num_blocks < 1 || Hq % Hkv != 0)
        return 2;
    for (int b = 0; b < B; ++b) {
        const int n = context_lens[b];
        if (n < 0 || n > max_blocks * block_size) return 3;
        for (int t = 0; t < n; t += block_size) {
            const int blk = block_table[(int64_t)b * max_blocks + t / block_size];
            if (blk < 0 || blk >= num_blocks) return 4;
        }
    }
    const int G = Hq / Hkv;
    int failed = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1) reduction(| : failed)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hq; ++h) {
            const int n = context_lens[b];
            const int g = h / G;
            double *s = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
            if (!s) {
                failed = 1;
                continue;
            }
            for (int i = 0; i < Tq; ++i) {
                const int64_t qi = (((int64_t)b * Hq + h) * Tq + i) * D;
                double *o = O + qi;
                for (int d = 0; d < D; ++d) o[d] = 0.0;
                int vis = causal ? n - Tq + i + 1 : n;   /* tokens 0 .. vis-1 */
                if (vis > n) vis = n;
                if (vis <= 0) {
                    lse[((int64_t)b * Hq + h) * Tq + i] = -INFINITY;
                    continue;
                }
                double m = -INFINITY;
                for (int t = 0; t < vis; ++t) {
                    const int64_t blk = block_table[(int64_t)b * max_blocks + t / block_size];
                    const int64_t row = ((blk * Hkv + g) * block_size + t % block_size) * D;
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d)
                        dot += widen16(q, qi + d) * widen16(k_cache, row + d);
                    s[t] = scale * dot;
                    if (s[t] > m) m = s[t];
                }
                double Z = 0.0;
                for (int t = 0; t < vis; ++t) {
                    s[t] = exp(s[t] - m);
                    Z += s[t];
                }
                for (int t = 0; t < vis; ++t) {
                    const int64_t blk = block_table[(int64_t)b * max_blocks + t / block_size];
                    const int64_t row = ((blk * Hkv + g) * block_size + t % block_size) * D;
                    const double w = s[t] / Z;
                    for (int d = 0; d < D; ++d) o[d] += w * widen16(v_cache, row + d);
                }
                lse[((int64_t)b * Hq + h) * Tq + i] = m + log(Z);
            }
            free(s);
        }
    }
    return failed ? -1 : 0;
}
