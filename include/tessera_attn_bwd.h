/*
 * tessera_attn_bwd.h -- C ABI of the attention backward pass in the MI355X
 * (gfx950) library (libtessera_attn.so; status codes and error functions as
 * declared in tessera_attn.h).
 *
 * The operation.  The page "Tessera: a from-scratch distillation and serving
 * stack in one repository" (section "The kernel set and its torch fallback")
 * and the Status lists of the README excerpts name a fused attention
 * backward as not yet done.  This is the gradient of tessera_attn_fwd's
 * result O for an output gradient dO.  With P the forward's softmax weights
 * (rebuilt from its lse), for every batch b, query head h, KV head
 * g = h / (Hq / Hkv), query row i and visible key j:
 *
 *     dP_ij   = dO_i . v_j          Delta_i = sum_d dO_id O_id
 *     dS_ij   = P_ij (dP_ij - Delta_i)
 *     dq_i    = scale * sum_j dS_ij k_j
 *     dk_j    = scale * sum over the query heads of g, sum_i dS_ij q_i
 *     dv_j    = sum over the query heads of g, sum_i P_ij dO_i
 *
 * Inputs.  q, k, v, causal, scale exactly as given to tessera_attn_fwd, and
 * its results out and lse; dout like out.  All bf16 tensors are bfloat16
 * bit patterns, contiguous, D innermost: q, out, dout, dq [B,Hq,T,D];
 * k, v, dk, dv [B,Hkv,T,D]; lse and delta [B,Hq,T] float32.
 *
 * Outputs.  dq, dk, dv (bf16, accumulated in fp32 and rounded once), and
 * delta: Delta_i above, written as a by-product (the second kernel of the
 * call reads it).  P and dS are rounded to bf16 for the matrix cores.
 *
 * Ownership, streams, errors: as in tessera_attn.h.  No output may overlap
 * an input or another output.  The result does not depend on scheduling
 * (no atomics).
 */
#ifndef TESSERA_ATTN_BWD_H
#define TESSERA_ATTN_BWD_H

#include "tessera_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

int tessera_attn_bwd(const void *q, const void *k, const void *v, const void *out,
                     const void *dout, const float *lse, void *dq, void *dk, void *dv,
                     float *delta, int B, int Hq, int Hkv, int T, int D, int causal, float scale,
                     void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TESSERA_ATTN_BWD_H */
