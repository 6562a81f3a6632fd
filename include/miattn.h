/*
 * miattn.h -- C ABI of libmiattn: grouped-query softmax attention forward on
 * AMD Instinct MI355X (gfx950).
 *
 *     O = softmax(alpha * Q K^T + M) V,   accumulated in FP32,
 *
 * with a float32 natural-log log-sum-exp per output row.
 *
 * Where the operation is defined (the pages):
 *   - TileOPs "Attention Operators", GQADenseFwdOp: the equation with FP32
 *     accumulation and the output in the input dtype; stage 1 (query row i sits
 *     at KV position p_i = i + S_kv - S_q); stage 4 (Z = alpha <Q, K>, alpha
 *     defaulting to 1/sqrt(D)); stage 5 (visibility: causal j <= p_i, and the
 *     sliding window p_i - w_L <= j <= p_i + w_R, -1 leaving a side
 *     unlimited); stage 6 (logit c tanh(Z / c) for a softcap c > 0); stage 7
 *     (softmax over keys, then the value sum); query head h reads KV head
 *     floor(h / (H_q / H_kv)); BSHD layout with D contiguous; a refusal names
 *     the limit it hit.  GQAPagedFwdOp takes the same window and softcap.
 *   - TileOPs "Attention Operators", MHADecodePagedWithKVCacheFwdOp: the paged
 *     layout (physical cache [rows, H_kv, D], real_seqlen_kv [B],
 *     block_table [B, num_pages]) and the per-request end-aligned causal rule;
 *     a query that sees no key outputs zeros.
 *   - TileOPs "Attention Operators", PagedKVCacheWriteFwdOp: a flattened cache
 *     row is page * page_size + offset.
 *   - RL-Kernel "Standard Softmax Attention", Tensor Contract: an explicit
 *     scale (0.0 included) is used verbatim; key_padding_mask [B, S_kv] with
 *     True = keep and False = that key column set to -inf.
 *   - MATE "QSA", Core Attention: the LSE is natural-log, an empty selection
 *     gives zero output and -inf LSE, split-KV partials are merged in FP32
 *     without recomputing QK or PV, and wrappers check shapes and layout
 *     without reading device contents.
 *   - TileOPs "Attention Operators", GQABwdOp: the gradients dq, dk, dv from
 *     q, k, v, o, do and lse, BSHD.
 *   - TileOPs "Attention Operators", PagedKVCacheWriteFwdOp: each token's key
 *     and value rows go to the pool row its slot names (page * page_size +
 *     offset, -1 skipping the token); an FP8 pool stores row / scale as
 *     E4M3FN, NaN preserved, finite overflow and infinities saturated to the
 *     largest finite magnitude; GQAPrefillPagedWithKVCacheFwdOp: a packed
 *     chunk's keys and values are appended after each request's cached ones
 *     and its queries attend to the cache.
 *   - TileOPs "Attention Operators", GQAVarlenFwdOp and GQAPagedFwdOp: packed
 *     THD tensors [total, heads, dim] with requests delimited by cumulative
 *     offsets, the causal mask bottom-right aligned per request, offsets not
 *     checked unless asked, and optional float32 sinks (one logit per query
 *     head in the softmax denominator only; not scaled or capped; -inf
 *     disables a sink, +inf zeroes the head's output; a row with no visible
 *     key returns zero whatever its sink).
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are HIP device pointers; the caller allocates and
 *     owns every tensor.  Work is enqueued on `stream` (a hipStream_t; NULL is
 *     the default stream) and the call returns without waiting for it, so the
 *     buffers must stay alive until that work completes.  Inputs are never
 *     written.
 *   - Tensors are dense row-major with the last axis contiguous.  q, k, v, o
 *     and the caches must be 16-byte aligned; lse 4-byte aligned.
 *   - Element offsets are computed in 64-bit; dimensions are int32.
 *   - A call returns MIATTN_OK or an error status and never throws.  On an error
 *     nothing is enqueued, and miattn_last_error() returns a message that names
 *     the violated limit (thread-local, valid until the next call on the thread).
 *   - Device-side contents (lengths, page-table entries) are not read by the
 *     host and not validated unless the environment variable MIATTN_VALIDATE=1
 *     is set, which copies them to the host (synchronising the stream).
 *     Out-of-range entries are otherwise the caller's error, with undefined
 *     results.
 *   - The library keeps one split-KV workspace per device (FP32 partial
 *     results of split key ranges, and the backward's per-row statistics),
 *     grown with hipMalloc on first need; a call that needs no larger
 *     workspace allocates nothing.  A grown workspace replaces the old one
 *     without freeing it (a HIP graph captured earlier may still use it):
 *     retired buffers are freed only by miattn_release_workspace().
 *   - Calls that use the workspace on different streams of one device are
 *     ordered: a call on a stream other than the workspace's previous user's
 *     first makes its stream wait for that use (an event).  Under stream
 *     capture the library records no such dependency and cannot grow the
 *     workspace (that call returns MIATTN_ERR_INVALID_ARG): run a call once
 *     before capturing it, and do not replay a captured graph concurrently
 *     with other calls of this library on the same device.
 *   - The only environment variables read are MIATTN_VALIDATE (above) and
 *     MIATTN_SPLIT_KEYS (keys per split-KV partition, as
 *     miattn_set_split_keys; for debugging).  Every other choice of schedule
 *     is fixed by the call's shapes.
 */
#ifndef MIATTN_H
#define MIATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MIATTN_OK = 0,
    MIATTN_ERR_INVALID_ARG = 1, /* arguments violate the contract          */
    MIATTN_ERR_UNSUPPORTED = 2, /* valid, but outside what the kernels serve */
    MIATTN_ERR_HIP = 3          /* a HIP runtime call failed                */
} miattn_status;

typedef enum { MIATTN_BF16 = 0, MIATTN_FP16 = 1 } miattn_dtype;

/* Element type of a KV-cache pool (the 16-bit ones equal the inputs' dtype). */
typedef enum {
    MIATTN_CACHE_BF16 = 0,
    MIATTN_CACHE_FP16 = 1,
    MIATTN_CACHE_FP8_E4M3 = 2 /* OCP E4M3FN bytes of value / scale */
} miattn_cache_dtype;

/*
 * Dense attention forward (TileOPs "Attention Operators", GQADenseFwdOp
 * stages 1, 4, 5 and 7; RL-Kernel "Standard Softmax Attention", Tensor
 * Contract: scale, key_padding_mask and the causal rule).
 *
 *   q    device, [B, Sq, Hq, D]  dtype
 *   k    device, [B, Skv, Hkv, D] dtype   (may be NULL when Skv == 0)
 *   v    device, [B, Skv, Hkv, D] dtype   (may be NULL when Skv == 0)
 *   B, Hq, Hkv, Sq, Skv, D   B, Sq, Skv >= 0; Hq, Hkv > 0; Hq % Hkv == 0;
 *                            D in {64, 128, 256}
 *   scale  alpha; NaN selects 1/sqrt(D) (rounded to float); any finite value,
 *          0.0 included, is used verbatim; +-inf is refused
 *   causal 0 or 1: key j is visible to query i iff j <= p_i = i + Skv - Sq.
 *          Sq > Skv is accepted; its first Sq - Skv rows see no key
 *   key_padding_mask  device, [B, Skv] bytes, nonzero = keep; NULL = no mask.
 *          Combined with the causal rule by AND
 *   o      device, [B, Sq, Hq, D] dtype, written in full
 *   lse    device, [B, Hq, Sq] float32, or NULL to skip it: the natural log of
 *          the softmax denominator, ln sum_j exp(alpha q.k_j) over the visible
 *          keys.  A row that sees no key gets o = 0 and lse = -inf
 *   dtype  MIATTN_BF16 or MIATTN_FP16, the type of q, k, v and o
 *   stream hipStream_t or NULL
 *
 * B == 0 or Sq == 0 returns MIATTN_OK without enqueuing anything.
 */
miattn_status attn_fwd_dense(const void *q, const void *k, const void *v, int B, int Hq,
                             int Hkv, int Sq, int Skv, int D, float scale, int causal,
                             const uint8_t *key_padding_mask, void *o, float *lse,
                             miattn_dtype dtype, void *stream);

/*
 * attn_fwd_dense with a sliding window and a logit softcap (TileOPs
 * "Attention Operators", GQADenseFwdOp stage 5: the window; stage 6: the
 * capped logit).  All other arguments as for attn_fwd_dense.
 *
 *   window_left, window_right  key j is visible to query i only if
 *          j >= p_i - window_left (when window_left != -1) and
 *          j <= p_i + window_right (when window_right != -1); -1 is
 *          unlimited, other negative values are refused (INVALID_ARG).
 *          Combined with the causal rule and the padding mask by AND
 *   softcap 0 for plain logits; c > 0 (finite) replaces each logit z by
 *          c * tanh(z / c); negative, infinite or NaN values are refused.
 *          lse is then the natural log of sum_j exp(capped logit_j)
 */
miattn_status attn_fwd_dense_ex(const void *q, const void *k, const void *v, int B, int Hq,
                                int Hkv, int Sq, int Skv, int D, float scale, int causal,
                                const uint8_t *key_padding_mask, void *o, float *lse,
                                int window_left, int window_right, float softcap,
                                miattn_dtype dtype, void *stream);

/*
 * Paged attention forward (decode, Sq = 1, and chunked prefill, Sq > 1;
 * TileOPs "Attention Operators", MHADecodePagedWithKVCacheFwdOp).
 *
 *   q        device, [B, Sq, Hq, D] dtype
 *   k_cache  device, [num_phys_pages * page_size, Hkv, D] dtype; the same bytes
 *            as [num_phys_pages, page_size, Hkv, D]
 *   v_cache  device, same layout as k_cache
 *   real_seqlen_kv device, int32 [B]: the number of cached keys of request b,
 *            its Sq query tokens included (they sit at the end); 0 <= len <=
 *            max_pages * page_size
 *   block_table device, int32 [B, max_pages]: physical page of logical page p
 *            of request b.  Key j of request b lives in cache row
 *            block_table[b, j / page_size] * page_size + j % page_size.  Entries
 *            at p >= ceil(len / page_size) are never read
 *   page_size a power of two >= 16 (others return MIATTN_ERR_UNSUPPORTED)
 *   causal   0 or 1: key j is visible to query i iff j <= p_i = i + len_b - Sq
 *   o, lse   as for attn_fwd_dense
 *   B, Sq, Hq, Hkv, D  as for attn_fwd_dense; max_pages > 0
 *   num_phys_pages  number of physical pages in each cache (only checked under
 *            MIATTN_VALIDATE=1)
 *   scale, dtype, stream  as for attn_fwd_dense
 *
 * Long key ranges are split across workgroups; the partial results (FP32
 * output rows and LSEs, in the library workspace) are merged by a second
 * kernel on the same stream (MATE "QSA", Core Attention: the split-KV merge).
 */
miattn_status attn_fwd_paged(const void *q, const void *k_cache, const void *v_cache,
                             const int32_t *real_seqlen_kv, const int32_t *block_table,
                             int page_size, int causal, void *o, float *lse, int B, int Sq,
                             int Hq, int Hkv, int D, int max_pages, int num_phys_pages,
                             float scale, miattn_dtype dtype, void *stream);

/*
 * attn_fwd_paged for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, and harnesses that forbid
 * hipMalloc.  Same arguments, kernels and results as attn_fwd_paged, but the
 * split-KV partials go to a fixed scratch array of 32 MiB that the library
 * holds on every GPU it runs on until the process ends (its address is looked
 * up once per device); the call allocates nothing, never uses the library
 * workspace, and ignores MIATTN_VALIDATE.
 *
 *   - A call whose partials would exceed 32 MiB returns
 *     MIATTN_ERR_UNSUPPORTED and enqueues nothing.  (Decode with Sq = 1 and
 *     Hq / Hkv = 4 at D = 128 needs about 8.3 KB per (request, KV head) plus
 *     about 2 MB; calls whose key ranges are not split need none.)
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's contents; no part of it needs to start at zero (each call writes
 *     every partial it merges).  Calls that overlap in time on one GPU --
 *     issued on different streams without ordering, or graph replays beside
 *     eager calls -- race on it and give undefined results.
 */
miattn_status attn_fwd_paged_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                     const int32_t *real_seqlen_kv, const int32_t *block_table,
                                     int page_size, int causal, void *o, float *lse, int B,
                                     int Sq, int Hq, int Hkv, int D, int max_pages,
                                     int num_phys_pages, float scale, miattn_dtype dtype,
                                     void *stream);

/*
 * attn_fwd_paged with a sliding window and a logit softcap (TileOPs
 * "Attention Operators", GQAPagedFwdOp takes the window and softcap of
 * GQADenseFwdOp stages 5 and 6).  window_left, window_right and softcap as
 * for attn_fwd_dense_ex, with p_i the position of query i in request b's own
 * key range; all other arguments as for attn_fwd_paged.
 */
miattn_status attn_fwd_paged_ex(const void *q, const void *k_cache, const void *v_cache,
                                const int32_t *real_seqlen_kv, const int32_t *block_table,
                                int page_size, int causal, void *o, float *lse, int B, int Sq,
                                int Hq, int Hkv, int D, int max_pages, int num_phys_pages,
                                float scale, int window_left, int window_right, float softcap,
                                miattn_dtype dtype, void *stream);

/*
 * Packed (THD) attention forward: requests of different lengths in one call.
 *
 *   q    device, [total_q, Hq, D] dtype; request b holds rows
 *        cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1
 *   k, v device, [total_kv, Hkv, D] dtype; request b holds rows
 *        cu_seqlens_kv[b] .. cu_seqlens_kv[b+1] - 1 (k, v may be NULL when
 *        total_kv == 0)
 *   cu_seqlens_q, cu_seqlens_kv  device, int32 [B + 1]: 0, nondecreasing,
 *        ending at total_q / total_kv.  Not read by the host (checked only
 *        under MIATTN_VALIDATE=1); the kernels clamp offsets into [0, total]
 *        and lengths into [0, max_seqlen], so malformed offsets give wrong
 *        results but no access outside the tensors
 *   max_seqlen_q, max_seqlen_kv  the most queries / keys one request holds
 *        (they size the launch)
 *   causal, window_left, window_right, softcap, scale  as for attn_fwd_dense_ex,
 *        with p_i = i + Skv_b - Sq_b inside request b
 *   sinks device, float32 [Hq] sink logits, or NULL: the head's sink enters
 *        the softmax denominator only, used as given; a +inf sink gives o = 0
 *        and lse = +inf; a row with no visible key gets o = 0 and lse = its
 *        sink (-inf without one)
 *   o    device, [total_q, Hq, D] dtype, written in full
 *   lse  device, [Hq, total_q] float32 (the log of the whole denominator,
 *        sink included), or NULL
 *   B, Hq, Hkv, D, dtype, stream  as for attn_fwd_dense
 *
 * B == 0, total_q == 0 or max_seqlen_q == 0 returns MIATTN_OK without
 * enqueuing anything.
 */
miattn_status attn_fwd_varlen(const void *q, const void *k, const void *v,
                              const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_kv, int B,
                              int total_q, int total_kv, int max_seqlen_q, int max_seqlen_kv,
                              int Hq, int Hkv, int D, float scale, int causal, int window_left,
                              int window_right, float softcap, const float *sinks, void *o,
                              float *lse, miattn_dtype dtype, void *stream);

/*
 * Paged attention forward over packed queries (requests with different query
 * counts, prefill and decode mixed).
 *
 *   q        device, [total_q, Hq, D] dtype, delimited by cu_seqlens_q as for
 *            attn_fwd_varlen
 *   k_cache, v_cache, block_table, page_size, max_pages, num_phys_pages  as
 *            for attn_fwd_paged
 *   cache_seqlens device, int32 [B]: keys of request b, its Sq_b query tokens
 *            included (they sit at the end); a request with no query is
 *            skipped
 *   max_seqlen_q  the most queries one request holds
 *   causal, window_left, window_right, softcap, sinks, scale  as for
 *            attn_fwd_varlen, with p_i = i + cache_seqlens[b] - Sq_b
 *   o, lse   [total_q, Hq, D] and [Hq, total_q], as for attn_fwd_varlen
 *   B, Hq, Hkv, D, dtype, stream  as for attn_fwd_paged
 *   cache_dtype  equal to dtype (16-bit pools), or MIATTN_CACHE_FP8_E4M3:
 *            the pools hold E4M3FN codes and a key (value) element is the
 *            code's value times *k_scale (*v_scale) (TileOPs "Attention
 *            Operators", GQAPrefillPagedWithKVCacheFwdOp: the dequantization
 *            scales of an FP8 pool; GQAVarlenFwdOp: each scale multiplies its
 *            tensor).  FP8 pools are served for D = 64 and 128 (D = 256:
 *            UNSUPPORTED); the pools must be 16-byte aligned
 *   k_scale, v_scale  device float32 [1], required with an FP8 pool (finite
 *            and positive, the caller's obligation: checked only under
 *            MIATTN_VALIDATE=1), else ignored
 */
miattn_status attn_fwd_paged_varlen(const void *q, const void *k_cache, const void *v_cache,
                                    const int32_t *cache_seqlens, const int32_t *block_table,
                                    const int32_t *cu_seqlens_q, int page_size, int causal,
                                    int window_left, int window_right, float softcap,
                                    const float *sinks, void *o, float *lse, int B,
                                    int total_q, int max_seqlen_q, int Hq, int Hkv, int D,
                                    int max_pages, int num_phys_pages, float scale,
                                    miattn_dtype dtype, miattn_cache_dtype cache_dtype,
                                    const float *k_scale, const float *v_scale, void *stream);

/*
 * Paged KV-cache write: scatter new key and value rows into the page pools.
 *
 *   k, v       device, [tokens, Hkv, D] dtype (16-byte aligned)
 *   k_pages, v_pages  device pools [num_slots, Hkv, D] of cache_dtype (the same
 *              bytes as [pages, page_size, Hkv, D], num_slots = pages *
 *              page_size); written in place, nothing outside the named rows
 *   slot_mapping device, int64 [tokens]: row of token n (page * page_size +
 *              offset), or -1 to skip it.  Distinct slots are the caller's
 *              obligation; slots outside [-1, num_slots) are skipped (refused
 *              with INVALID_ARG under MIATTN_VALIDATE=1)
 *   Hkv * D    a multiple of 8
 *   dtype      MIATTN_BF16 or MIATTN_FP16, the type of k and v
 *   cache_dtype  equal to dtype (rows copied), or MIATTN_CACHE_FP8_E4M3: each
 *              value is divided by *k_scale / *v_scale in float32 and stored
 *              as E4M3FN (nearest, ties to even; NaN kept; beyond +-448,
 *              infinities included, saturated to +-448)
 *   k_scale, v_scale  device float32 [1], required for an FP8 pool (finite and
 *              positive; checked only under MIATTN_VALIDATE=1), else ignored
 *   stream     hipStream_t or NULL
 */
miattn_status kv_cache_write(const void *k, const void *v, void *k_pages, void *v_pages,
                             const int64_t *slot_mapping, int tokens, int Hkv, int D,
                             int64_t num_slots, miattn_dtype dtype, miattn_cache_dtype cache_dtype,
                             const float *k_scale, const float *v_scale, void *stream);

/*
 * Paged prefill with append: request b's chunk -- queries,
 * keys and values at packed rows cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1 --
 * is written to logical positions cache_seqlens[b] + i of its cache (pool
 * row block_table[b, pos / page_size] * page_size + pos % page_size), then
 * its queries attend to the request's cache_seqlens[b] + Sq_b keys.
 *
 *   q, k_new, v_new  device, [total_q, Hq, D] / [total_q, Hkv, D] dtype
 *   k_cache, v_cache device pools as for attn_fwd_paged, written in place
 *   cache_seqlens    device, int32 [B]: keys cached before the chunk
 *   block_table      device, int32 [B, max_pages]; it must cover the appended
 *                    positions (tokens it does not cover are not written)
 *   cu_seqlens_q, max_seqlen_q  as for attn_fwd_paged_varlen
 *   causal, softcap, scale, o, lse, dtype, stream  as for attn_fwd_paged_varlen
 *                    (lse [Hq, total_q])
 *   B, Hq, Hkv, D, page_size, max_pages, num_phys_pages  as for attn_fwd_paged
 *   cache_dtype, k_scale, v_scale  as for attn_fwd_paged_varlen; with an FP8
 *                    pool the chunk is written as kv_cache_write writes it
 *                    (value / scale as E4M3FN) and read back dequantized
 */
miattn_status attn_fwd_paged_append(const void *q, const void *k_new, const void *v_new,
                                    void *k_cache, void *v_cache, const int32_t *cache_seqlens,
                                    const int32_t *block_table, const int32_t *cu_seqlens_q,
                                    int page_size, int causal, float softcap, void *o,
                                    float *lse, int B, int total_q, int max_seqlen_q, int Hq,
                                    int Hkv, int D, int max_pages, int num_phys_pages,
                                    float scale, miattn_dtype dtype,
                                    miattn_cache_dtype cache_dtype, const float *k_scale,
                                    const float *v_scale, void *stream);

/*
 * Attention backward (TileOPs "Attention Operators", GQABwdOp): the gradients
 * of the dense call's output with respect to q, k and v,
 *     P = exp(alpha q.k - lse) on visible keys,  dS = P (dO.v - <dO, o>),
 *     dq = alpha dS k,  dk = alpha dS^T q (summed over the g query heads of a
 *     KV head),  dv = P^T dO,
 * recomputing P from the forward's lse (no score matrix is stored).
 *
 *   q, o, dout device, [B, Sq, Hq, D] dtype (o: the forward's output, dout:
 *              the gradient of the loss with respect to it)
 *   k, v       device, [B, Skv, Hkv, D] dtype
 *   lse        device, [B, Hq, Sq] float32, natural log, as attn_fwd_dense
 *              writes it (-inf for a row that sees no key)
 *   B, Hq, Hkv, Sq, Skv, scale, causal, dtype, stream  as for attn_fwd_dense
 *              (no window, softcap or padding mask); D in {64, 128} (256
 *              returns MIATTN_ERR_UNSUPPORTED)
 *   dq         device, [B, Sq, Hq, D] dtype, written in full
 *   dk, dv     device, [B, Skv, Hkv, D] dtype, written in full
 *
 * Accumulation is FP32; every output element has one writer (no atomics), so
 * repeated calls give the same bits.  Uses the library workspace for
 * 2 * B * Hq * Sq floats.
 */
miattn_status attn_bwd(const void *q, const void *k, const void *v, const void *o,
                       const void *dout, const float *lse, int B, int Hq, int Hkv, int Sq, int Skv,
                       int D, float scale, int causal, void *dq, void *dk, void *dv,
                       miattn_dtype dtype, void *stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *miattn_last_error(void);

/*
 * Frees the workspace of the current device and every buffer it replaced
 * (waits for the device).  No graph captured before may be replayed after it.
 */
miattn_status miattn_release_workspace(void);

/*
 * Split-KV control: keys per split (rounded up to the kernel's key tile);
 * 0 restores the automatic choice.  Applies to both entry points; a value
 * that yields one split disables the merge.  Mainly for tests and tuning.
 */
void miattn_set_split_keys(int keys_per_split);

/*
 * Stream-K decode plan control, for tests: the plan weight, in key tiles, of
 * starting a piece of a (request, KV head) unit (0 .. 64; a negative value
 * restores the default, 6).  Any weight covers every key tile exactly once;
 * it only moves the boundaries between workgroups' shares.
 */
void miattn_set_streamk_piece(int tiles);

/*
 * Kernel timing.  Between miattn_profile_start() and miattn_profile_stop(),
 * every attention-kernel and merge-kernel launch is bracketed by HIP events
 * recorded on its own stream.  stop() waits for those events and returns the
 * summed durations (milliseconds) and launch counts of each kernel kind.
 */
void miattn_profile_start(void);
miattn_status miattn_profile_stop(double *attn_ms, int *attn_launches, double *merge_ms,
                                  int *merge_launches);

#ifdef __cplusplus
}
#endif

#endif /* MIATTN_H */
