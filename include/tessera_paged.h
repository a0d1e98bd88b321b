/*
 * tessera_paged.h -- C ABI of attention decode over a block-paged KV cache in
 * the MI355X (gfx950) library (libtessera_attn.so; status codes and error
 * functions as declared in tessera_attn.h).
 *
 * The operation.  The page "Tessera: a from-scratch distillation and serving
 * stack in one repository" (section "Serving: block-paged KV, batch
 * recomposition, speculation") describes a KV cache held in fixed-size blocks
 * that sequences reference through a ref-counted allocator, and the Status
 * lists of the pages name a fused paged-attention decode kernel as not yet
 * done.  This is that kernel: for each sequence b with n = context_lens[b]
 * cached tokens (the new ones included), its Tq newest tokens attend to its
 * cached tokens.  Query row i stands at position n - Tq + i; with causal = 1
 * it sees tokens 0 .. n - Tq + i, with causal = 0 all n.  For every query
 * head h (KV head g = h / (Hq / Hkv)):
 *
 *     s_it        = scale * sum_d q[b,h,i,d] * K_b[g,t,d]
 *     out[b,h,i]  = sum_t softmax_t(s_it) * V_b[g,t,:]
 *     lse[b,h,i]  = ln sum_t exp(s_it)
 *
 * over the visible tokens t.  A row that sees no token (n = 0, or n < Tq
 * under the causal mask) gets out = 0 and lse = -inf.  With the cache
 * gathered into contiguous K/V this is tessera_attn_fwd_kv with Tk = n.
 *
 * Layout (the pages give none; this is the library's reading).  Token t of
 * sequence b lives in physical block block_table[b, t / block_size], row
 * t % block_size:
 *     q            [B, Hq, Tq, D]                      bf16
 *     k_cache      [num_blocks, Hkv, block_size, D]    bf16
 *     v_cache      [num_blocks, Hkv, block_size, D]    bf16
 *     block_table  [B, max_blocks]                     int32
 *     context_lens [B]                                 int32
 *     out          [B, Hq, Tq, D]                      bf16
 *     lse          [B, Hq, Tq]                         float32, natural log
 * so the rows of one KV head within a block are contiguous.  Only the
 * table entries of blocks that hold one of a sequence's n tokens are read.
 *
 * Limits: D is 32, 64 or 128; (Hq / Hkv) * Tq <= 32 (the query rows that
 * share a KV head); block_size is a multiple of 16.
 *
 * Bad device data.  The lengths and the table live in device memory, so they
 * cannot be checked before the launch.  A length outside
 * [0, max_blocks * block_size], or a table entry in use outside
 * [0, num_blocks), is not followed: no memory outside the caches is read
 * through it, and every out and lse value of that sequence becomes NaN.
 *
 * Workspace.  The 32-key tiles of each KV head, over all sequences, are
 * shared out in equal contiguous parts among a fixed set of waves (1536 in
 * all, 2048 at D = 32, fewer for small calls), so a sequence may be cut into pieces held by
 * several waves; their partial results are merged through their lse.  The
 * caller passes a device workspace of at least
 * tessera_paged_decode_workspace(...) bytes (always more than 0), 16-byte
 * aligned.  Its contents on entry do not matter; two calls must not use one
 * workspace at the same time.
 *
 * Ownership, streams and errors: as in tessera_attn.h (scale any finite
 * float, causal 0 or 1; no output may overlap an input, the workspace or the
 * other output).  TESSERA_ERR_WORKSPACE: the workspace is NULL or smaller
 * than required.
 */
#ifndef TESSERA_PAGED_H
#define TESSERA_PAGED_H

#include "tessera_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of workspace tessera_paged_decode needs for these sizes (more than
 * 0), or -status (a negative tessera_attn_status) when the sizes are invalid
 * or unsupported. */
long long tessera_paged_decode_workspace(int B, int Hq, int Hkv, int Tq, int D, int block_size,
                                         int max_blocks);

int tessera_paged_decode(const void *q, const void *k_cache, const void *v_cache,
                         const int *block_table, const int *context_lens, void *out, float *lse,
                         int B, int Hq, int Hkv, int Tq, int D, int num_blocks, int block_size,
                         int max_blocks, int causal, float scale, void *workspace,
                         long long workspace_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * decode as tessera_paged_decode, with the same arguments except the
 * workspace, and identical results.  The partial results go to a fixed
 * scratch buffer of tessera_paged_decode_scratch_limit() bytes (32 MiB) that
 * the library holds in each GPU's memory from its first use on that GPU until
 * the process ends; the call itself allocates nothing.  Sizes whose workspace
 * (tessera_paged_decode_workspace) exceeds that limit return
 * TESSERA_ERR_SCRATCH with nothing launched.  Every call on one GPU uses
 * that GPU's one buffer: calls that overlap in time on one GPU (other
 * streams or threads) race on it, so the caller serialises them, for
 * example by issuing them on one stream.
 */
int tessera_paged_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                 const int *block_table, const int *context_lens, void *out,
                                 float *lse, int B, int Hq, int Hkv, int Tq, int D,
                                 int num_blocks, int block_size, int max_blocks, int causal,
                                 float scale, void *stream);

/* Bytes of the fixed scratch buffer behind tessera_paged_decode_noalloc. */
long long tessera_paged_decode_scratch_limit(void);

#ifdef __cplusplus
}
#endif

#endif /* TESSERA_PAGED_H */
