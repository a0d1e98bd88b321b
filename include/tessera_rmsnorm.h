/*
 * tessera_rmsnorm.h -- C ABI of the fused RMSNorm forward in the MI355X
 * (gfx950) library (libtessera_attn.so, which also holds the attention
 * entry points of tessera_attn.h; the status codes and error functions are
 * those declared there).
 *
 * The operation.  The pages list a fused RMSNorm among the kernels (page
 * "Tessera: a from-scratch distillation and serving stack in one
 * repository", section "The kernel set and its torch fallback") and an
 * RMSNorm decoder (README excerpt on topairepos.com, "What's in it").  They
 * print no formula; the plain reading is root-mean-square normalisation
 * with a learned per-feature gain, in one pass over each row:
 *
 *     y[r, c] = x[r, c] / sqrt(mean_c' x[r, c']^2 + eps) * w[c]
 *
 * Layout.  x and y are contiguous [rows, n] bfloat16 (16-bit patterns), w is
 * [n] bfloat16.  The mean of squares and the product are taken in fp32 and
 * y is rounded once to bf16 (nearest even).
 *
 * Arguments.  rows >= 1; 8 <= n <= 65536 and n % 8 == 0; eps finite and
 * >= 0; x, w, y 16-byte aligned.  y may be x itself (in place) but may not
 * otherwise overlap x or w.  Ownership, streams and errors are as in
 * tessera_attn.h: nothing is allocated or kept, work goes on `stream`, and
 * every check runs before anything is enqueued.
 */
#ifndef TESSERA_RMSNORM_H
#define TESSERA_RMSNORM_H

#include "tessera_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Statuses: TESSERA_ERR_NULL, TESSERA_ERR_SHAPE (rows < 1 or n < 8),
 * TESSERA_ERR_UNSUPPORTED (n % 8 != 0 or n > 65536), TESSERA_ERR_EPS,
 * TESSERA_ERR_ALIGN, TESSERA_ERR_ALIAS, TESSERA_ERR_TOO_LARGE (rows * n past
 * 2^62), TESSERA_ERR_LAUNCH.
 */
int tessera_rmsnorm_fwd(const void *x, const void *w, void *y, long long rows, int n, float eps,
                        void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TESSERA_RMSNORM_H */
