/*
 * tessera_attn.h -- C ABI of the MI355X (gfx950) attention forward library.
 *
 * The operation.  The FlashAttention forward pass named on the page "Tessera:
 * a from-scratch distillation and serving stack in one repository" (section
 * "The kernel set and its torch fallback", and the README excerpt's
 * "Kernels" list on topairepos.com): attention with an online softmax,
 * causal masking and grouped-query attention.  For every batch b, query head
 * h and query row i, with G = Hq / Hkv and KV head g = h / G:
 *
 *     s_ij       = scale * sum_d q[b,h,i,d] * k[b,g,j,d]
 *     out[b,h,i] = sum_j softmax_j(s_ij) * v[b,g,j,:]
 *     lse[b,h,i] = ln sum_j exp(s_ij)
 *
 * over keys j <= i when causal = 1, over all T keys when causal = 0.  The
 * online softmax is an exact reformulation; results match the plain
 * definition up to rounding.
 *
 * Layout.  Every tensor is contiguous and row-major with D innermost:
 *     q   [B, Hq,  T, D]      k, v [B, Hkv, T, D]
 *     out [B, Hq,  T, D]      (same dtype as q)
 *     lse [B, Hq,  T]         float32, natural log
 *
 * Ownership and streams.  All pointers are device memory owned by the caller
 * on the device current at the call.  The library allocates nothing, keeps
 * no pointer after the call, never synchronises and never changes the
 * current device.  Work is enqueued on `stream` (a hipStream_t; NULL is the
 * default stream) and is complete when that stream reaches it; the caller
 * keeps every buffer alive until then.  `out` and `lse` must not overlap
 * q, k, v or each other.
 *
 * Work queues.  A bf16 call with at least four work items (query tiles times
 * KV heads) per workgroup the GPU holds at once runs as a persistent launch:
 * its workgroups pull items from queues, so that the GPU's dies, which do not
 * all run at one speed, finish together.  The queue counters live in a small
 * block of device memory that belongs to the library (part of its loaded
 * code, zero at load; every such launch leaves it at zero again).  Each
 * stream gets a block of its own on its first such call, up to 64 streams
 * per device; calls on further streams, and calls on a stream that is being
 * captured into a graph, run as plain grids without counters.  Results are
 * the same bits either way.
 *
 * Errors.  Every argument is checked before anything is enqueued; a failed
 * check returns its status with no buffer touched and nothing launched.
 * TESSERA_ERR_LAUNCH means the HIP launch itself failed; the HIP error text
 * is then available from tessera_attn_last_error() on the calling thread.
 * No C++ exception crosses this interface and nothing is printed.
 * The functions may be called from several threads; the only state they keep
 * is the stream-to-queue-block table above, updated under a lock.
 */
#ifndef TESSERA_ATTN_H
#define TESSERA_ATTN_H

#ifdef __cplusplus
extern "C" {
#endif

enum tessera_attn_status {
    TESSERA_OK = 0,
    TESSERA_ERR_NULL = 1,        /* a pointer argument is NULL */
    TESSERA_ERR_SHAPE = 2,       /* B, Hq, Hkv or a row count < 1, Hq % Hkv != 0, or a
                                    causal tessera_attn_fwd_kv call with Tq > Tk */
    TESSERA_ERR_UNSUPPORTED = 3, /* D is not 32, 64 or 128, or another size limit of the
                                    called function is exceeded */
    TESSERA_ERR_CAUSAL = 4,      /* causal is neither 0 nor 1 */
    TESSERA_ERR_SCALE = 5,       /* scale is NaN or infinite */
    TESSERA_ERR_ALIGN = 6,       /* q, k, v, out not 16-byte or lse not 4-byte aligned */
    TESSERA_ERR_ALIAS = 7,       /* out or lse overlaps an input or each other */
    TESSERA_ERR_TOO_LARGE = 8,   /* the launch grid would exceed 2^31 - 1 workgroups */
    TESSERA_ERR_LAUNCH = 9,      /* the HIP kernel launch failed */
    TESSERA_ERR_EPS = 10,        /* RMSNorm eps is NaN, infinite or negative */
    TESSERA_ERR_WORKSPACE = 11,  /* paged decode workspace NULL or too small */
    TESSERA_ERR_SCRATCH = 12     /* the allocation-free paged decode needs more than the
                                    library's fixed scratch buffer holds */
};

/*
 * bf16 attention forward.  q, k, v and out hold bfloat16 values (16-bit
 * patterns); products are accumulated in fp32 and out is rounded once to
 * bf16 (nearest even).  The softmax weights enter the P.V product as bf16,
 * and the row sums that normalise out add those same rounded weights, so the
 * weights of a row sum to one exactly as used.  lse is fp32 (natural log).
 * scale is any finite float (0 and
 * negative values included); it multiplies q.k before the mask and softmax.
 * Returns a tessera_attn_status.
 */
int tessera_attn_fwd(const void *q, const void *k, const void *v, void *out, float *lse,
                     int B, int Hq, int Hkv, int T, int D, int causal, float scale,
                     void *stream);

/*
 * bf16 attention forward of Tq query rows against Tk key rows (Tq <= Tk when
 * causal): the continuation of a sequence whose first Tk - Tq positions are
 * already in the K/V cache, as in chunked prefill or decoding a few tokens.
 * The page "Tessera: a from-scratch distillation and serving stack in one
 * repository" (section "Serving: block-paged KV, batch recomposition,
 * speculation") states the property this serves: decoding incrementally with
 * the KV cache gives what a full forward pass gives.  Query row i stands at
 * sequence position i + Tk - Tq, so with causal = 1 it sees keys
 * j <= i + Tk - Tq (the causal mask aligned to the last key); with causal = 0
 * it sees all Tk keys, and any Tq, Tk >= 1 is accepted.  Row i of the result
 * equals row i + Tk - Tq of tessera_attn_fwd run on the full sequence.
 *     q   [B, Hq,  Tq, D]     k, v [B, Hkv, Tk, D]
 *     out [B, Hq,  Tq, D]     lse  [B, Hq,  Tq]
 * Everything else (dtypes, scale, ownership, streams, errors) is as for
 * tessera_attn_fwd; tessera_attn_fwd(..., T, ...) is this call with
 * Tq = Tk = T.
 */
int tessera_attn_fwd_kv(const void *q, const void *k, const void *v, void *out, float *lse,
                        int B, int Hq, int Hkv, int Tq, int Tk, int D, int causal, float scale,
                        void *stream);

/*
 * Tile configuration of the bf16 forward (the "autotuned tile sizes" of the
 * kernel set on the page "Tessera: a from-scratch distillation and serving
 * stack in one repository", section "The kernel set and its torch
 * fallback").  A workgroup is eight waves that share each staged 64-key K/V
 * tile; the configuration sets how its work is cut:
 *   heads_per_workgroup  1, 2 or 4 query heads of one GQA group per
 *                        workgroup (must divide Hq / Hkv); the workgroup's
 *                        query tile then spans 8 / heads_per_workgroup
 *                        blocks of query_rows_per_wave rows
 *   query_rows_per_wave  32 or 64 (64: D <= 64 only)
 *   workgroups_per_cu    1 or 2 (2: D <= 64, 32 rows per wave, and the key
 *                        count a multiple of 64)
 *   persistent           0: one workgroup per work item; 1: as many
 *                        workgroups as the GPU holds at once, taking items
 *                        from work queues (workgroups_per_cu = 1 only)
 * Every configuration computes the same result up to rounding.  The library
 * picks one from a static table built by an offline sweep on MI355X (per
 * head size, causal or not, and problem size); tessera_attn_fwd and
 * tessera_attn_fwd_kv use that pick.
 */
typedef struct tessera_attn_tile_config {
    int heads_per_workgroup;
    int query_rows_per_wave;
    int workgroups_per_cu;
    int persistent;
} tessera_attn_tile_config;

/*
 * The configuration the library's table picks for these sizes (arguments as
 * for tessera_attn_fwd_kv; no pointer is read except `config`, which
 * receives it).  Returns TESSERA_OK, or TESSERA_ERR_NULL / TESSERA_ERR_SHAPE
 * / TESSERA_ERR_UNSUPPORTED / TESSERA_ERR_CAUSAL for bad arguments.
 */
int tessera_attn_fwd_tile_config(int B, int Hq, int Hkv, int Tq, int Tk, int D, int causal,
                                 tessera_attn_tile_config *config);

/*
 * tessera_attn_fwd_kv with the tile configuration given explicitly (the
 * sweep that builds the table times every configuration through this).  A
 * configuration that these sizes do not allow returns
 * TESSERA_ERR_UNSUPPORTED before anything is launched; `config` NULL is
 * TESSERA_ERR_NULL.  Everything else is as for tessera_attn_fwd_kv.
 */
int tessera_attn_fwd_with_config(const void *q, const void *k, const void *v, void *out,
                                 float *lse, int B, int Hq, int Hkv, int Tq, int Tk, int D,
                                 int causal, float scale, const tessera_attn_tile_config *config,
                                 void *stream);

/*
 * fp32 attention forward: the same operation and arguments with float32
 * q, k, v and out, computed in fp32 throughout.
 */
int tessera_attn_fwd_f32(const float *q, const float *k, const float *v, float *out, float *lse,
                         int B, int Hq, int Hkv, int T, int D, int causal, float scale,
                         void *stream);

/* Static text naming a status code (never NULL). */
const char *tessera_attn_status_string(int status);

/* Text of the last TESSERA_ERR_LAUNCH on the calling thread ("" if none). */
const char *tessera_attn_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int tessera_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TESSERA_ATTN_H */
