/*
 * rmsnorm_oracle.c -- plain fp64 CPU oracle for RMSNorm.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests and the bench use it.  It shares no code
 * with the HIP library.
 *
 * What it computes.  The pages list a fused RMSNorm in the kernel set (page
 * "Tessera: a from-scratch distillation and serving stack in one
 * repository", section "The kernel set and its torch fallback") and an
 * RMSNorm decoder (README excerpt on topairepos.com, "What's in it"), with no
 * formula.  The plain reading is root-mean-square normalisation with a
 * per-feature gain, row by row:
 *
 *     ms      = (1/n) * sum_c x[r,c]^2
 *     y[r,c]  = x[r,c] / sqrt(ms + eps) * w[c]
 *
 * in double precision, every bf16 input widened exactly (its 16 bits in the
 * top half of an fp32 word).  x [rows, n] and w [n] are uint16 bf16 patterns;
 * y [rows, n] is fp64.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static double widen_bf16(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

int tessera_oracle_rmsnorm(const uint16_t *x, const uint16_t *w, int64_t rows, int n,
                           double eps, double *y)
{
    if (!x || !w || !y) return 1;
    if (rows < 1 || n < 1) return 2;
    if (!(eps >= 0.0)) return 3;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *xr = x + r * n;
        double ss = 0.0;
        for (int c = 0; c < n; ++c) {
            const double v = widen_bf16(xr[c]);
            ss += v * v;
        }
        const double ms = ss / n;
        const double inv = 1.0 / sqrt(ms + eps);
        for (int c = 0; c < n; ++c)
            y[r * n + c] = widen_bf16(xr[c]) * inv * widen_bf16(w[c]);
    }
    return 0;
}
