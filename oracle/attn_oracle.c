/*
 * attn_oracle.c -- TEST INFRASTRUCTURE ONLY (not part of the product path).
 *
 * A plain, slow, fp64 CPU evaluation of grouped-query softmax attention
 * forward, written from its definition.  Only the tests, the smoke check and
 * the benchmark's CPU-baseline leg load this library; the HIP library never
 * links, includes or calls it, and this file includes nothing from it.
 *
 * What is computed, and where the pages define it:
 *   - TileOPs "Attention Operators", GQADenseFwdOp: stage 1 (query position
 *     p_i = i + S_kv - S_q), stage 4 (scores Z = alpha <Q, K_r(h)>), stage 5
 *     (visibility: not causal or j <= p_i, and inside the sliding window
 *     p_i - w_L <= j <= p_i + w_R, a bound of -1 being unlimited), stage 6
 *     (logits: c tanh(Z / c) with softcap c > 0, Z itself with c = 0),
 *     stage 7 (softmax over the KV axis, then the value reduction); the head
 *     map r(h) = floor(h / g) with g = H / H_kv; BSHD layout with D
 *     contiguous.  GQAPagedFwdOp and MHADecodePagedWithKVCacheFwdOp take the
 *     same window and softcap parameters.
 *   - TileOPs "Attention Operators", MHADecodePagedWithKVCacheFwdOp: physical
 *     cache [rows, H_kv, D], real_seqlen_kv[B] (the cache length, its query
 *     tokens included), block_table[B, num_pages]; query i sees keys up to
 *     i + real_seqlen_kv - S_q; a query that sees no key outputs zeros.
 *   - TileOPs "Attention Operators", PagedKVCacheWriteFwdOp: a flattened cache
 *     row is page * page_size + offset.
 *   - RL-Kernel "Standard Softmax Attention", Tensor Contract: scale None means
 *     1/sqrt(D), an explicit value (0.0 included) is used verbatim;
 *     key_padding_mask [B, S_kv], True = keep, False sets the column to -inf.
 *   - MATE "QSA", Core Attention: the log-sum-exp is natural-log and an empty
 *     selection returns zero output with -inf LSE.
 *   - TileOPs "Attention Operators", GQABwdOp: given q, k, v, o, do and lse,
 *     the gradients dq, dk, dv of O = softmax(alpha Q K^T + M) V (the
 *     standard softmax-attention backward, with P recomputed from the given
 *     lse and D_i = sum_d dO_id O_id from the given o); RL-Kernel "Standard
 *     Softmax Attention", Fixed Reduction Order: dK/dV of a KV head sum over
 *     its query heads in group order, then over query positions.
 *   - TileOPs "Attention Operators", PagedKVCacheWriteFwdOp: each token's K
 *     and V row goes to the pool row its slot names (page * page_size +
 *     offset; -1 skips the token); an FP8 pool stores row / scale as
 *     E4M3FN, NaN preserved, finite overflow and infinities saturated to the
 *     largest finite magnitude of the same sign.
 *   - TileOPs "Attention Operators", GQAPrefillPagedWithKVCacheFwdOp: the
 *     packed chunk's keys and values are appended after each request's
 *     cached ones (cache_seqlens counts them before the append), then the
 *     chunk's queries attend to the cache.
 *   - TileOPs "Attention Operators", GQAVarlenFwdOp and GQAPagedFwdOp: packed
 *     THD tensors [total, heads, dim] whose requests are delimited by
 *     cu_seqlens (request b holds rows cu[b] .. cu[b+1] - 1), the causal mask
 *     bottom-right aligned per request, and optional float32 sinks: one logit
 *     per query head added to the softmax denominator only (neither scaled
 *     nor capped); -inf disables a sink, +inf makes the head's output zero,
 *     and a row with no visible key returns zero whatever its sink.
 *
 * Readings where the pages leave a step open (each also listed in the design
 * notes): the scale multiplies the finished dot product; the LSE is
 * ln sum_j exp(L_j) over the visible keys, L_j being the logit of stage 6
 * (alpha <q, k_j>, capped when a softcap is given); a paged request's window
 * is placed at its own p_i; with a sink the LSE is the log of the whole
 * denominator, ln(sum_j exp(L_j) + exp(sink)), so a row with no visible key
 * has lse = sink; packed (THD) calls store lse as [H, total_q]; a causal call with
 * S_q > S_kv is accepted and its first S_q - S_kv rows are empty; a masked
 * key and a causally hidden key are combined with AND.
 *
 * Arithmetic: every element is decoded exactly to double; every sum runs in
 * double with its index ascending (d for dot products, j for the softmax and
 * the value reduction).  Build with -ffp-contract=off and no fast-math so the
 * compiler keeps that order.  Rows are independent, so the OpenMP schedule
 * does not change any bit of the result.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_BF16 0
#define ORACLE_FP16 1

/* bfloat16 is the top half of an IEEE binary32: widen by a 16-bit shift. */
static double decode_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Exponent 0 holds zero and subnormals (fraction * 2^-24); exponent 31 holds
 * infinities and NaN; otherwise the value is (1024 + fraction) * 2^(e - 25). */
static double decode_fp16(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int e = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double mag;
    if (e == 0)
        mag = ldexp((double)frac, -24);
    else if (e == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + frac), e - 25);
    return sign ? -mag : mag;
}

static double decode(const uint16_t *base, int64_t idx, int dtype)
{
    return dtype == ORACLE_BF16 ? decode_bf16(base[idx]) : decode_fp16(base[idx]);
}

/* Exposed so the tests can pin both decoders against library conversions. */
double oracle_decode(uint16_t bits, int dtype)
{
    return dtype == ORACLE_BF16 ? decode_bf16(bits) : decode_fp16(bits);
}

/* The score scale alpha: the sentinel NaN selects 1/sqrt(D), computed once in
 * double and rounded to float (the type the scale is passed in); any other
 * value is used as given. */
double oracle_resolve_scale(float scale, int D)
{
    if (isnan(scale))
        return (double)(float)(1.0 / sqrt((double)D));
    return (double)scale;
}

static double e4m3_value(int code);

/* Everything that locates a key or value row for one call. */
typedef struct {
    const uint16_t *q;
    const void *k, *v; /* 16-bit patterns, or E4M3FN codes when cache_fp8 */
    int dtype;
    /* an FP8 pool holds E4M3FN codes; element = decoded code * its scale */
    int cache_fp8;
    double k_scale, v_scale;
    int B, Sq, Hq, Hkv, D;
    int causal;
    double alpha;
    int window_left, window_right; /* -1: unlimited */
    double softcap;                /* 0: no cap */
    /* packed (THD) requests: row offsets [B + 1], or NULL for B equal blocks */
    const int32_t *cu_q, *cu_kv;
    int total_q;
    const float *sinks; /* [Hq] or NULL */
    /* dense */
    int Skv;
    const uint8_t *mask; /* [B, Skv] or NULL */
    /* paged */
    int paged;
    const int32_t *seqlen;      /* [B] */
    const int32_t *block_table; /* [B, max_pages] */
    int page_size, max_pages;
} call_t;

/* Number of keys request b holds. */
static int64_t kv_length(const call_t *c, int b)
{
    if (c->paged)
        return (int64_t)c->seqlen[b];
    if (c->cu_kv)
        return (int64_t)c->cu_kv[b + 1] - c->cu_kv[b];
    return (int64_t)c->Skv;
}

/* Number of queries request b holds, and the packed row of its query i. */
static int64_t q_length(const call_t *c, int b)
{
    return c->cu_q ? (int64_t)c->cu_q[b + 1] - c->cu_q[b] : (int64_t)c->Sq;
}

static int64_t q_row(const call_t *c, int b, int i)
{
    return c->cu_q ? (int64_t)c->cu_q[b] + i : (int64_t)b * c->Sq + i;
}

/* Element offset of key/value row (b, j, r): dense BSHD, or the page-table
 * translation row = block_table[b, j / page_size] * page_size + j % page_size. */
static int64_t kv_row_offset(const call_t *c, int b, int64_t j, int r)
{
    int64_t row;
    if (c->paged) {
        int64_t logical_page = j / c->page_size;
        int64_t in_page = j % c->page_size;
        int64_t phys_page = c->block_table[(int64_t)b * c->max_pages + logical_page];
        row = phys_page * c->page_size + in_page;
    } else if (c->cu_kv) {
        row = (int64_t)c->cu_kv[b] + j;
    } else {
        row = (int64_t)b * c->Skv + j;
    }
    return (row * c->Hkv + r) * c->D;
}

/* Element idx of the key (which = 0) or value (1) tensor: the 16-bit value,
 * or for an FP8 pool the code's value times the pool's dequantization scale
 * (TileOPs "Attention Operators", GQAPrefillPagedWithKVCacheFwdOp: k_scale and
 * v_scale of an FP8 pool; GQAVarlenFwdOp: each scale multiplies its tensor). */
static double kv_value(const call_t *c, int which, int64_t idx)
{
    const void *base = which ? c->v : c->k;
    if (c->cache_fp8)
        return e4m3_value(((const uint8_t *)base)[idx]) * (which ? c->v_scale : c->k_scale);
    return decode((const uint16_t *)base, idx, c->dtype);
}

/* Key j is visible to query i iff (not causal or j <= p_i), it lies inside
 * the window (p_i - w_L <= j when w_L != -1, j <= p_i + w_R when w_R != -1)
 * and the padding mask keeps column j. */
static int visible(const call_t *c, int b, int i, int64_t j)
{
    int64_t p = (int64_t)i + kv_length(c, b) - q_length(c, b);
    if (c->causal && j > p)
        return 0;
    if (c->window_left != -1 && j < p - c->window_left)
        return 0;
    if (c->window_right != -1 && j > p + c->window_right)
        return 0;
    if (c->mask && c->mask[(int64_t)b * c->Skv + j] == 0)
        return 0;
    return 1;
}

/* One output row (b, i, h): o_row[D] and *lse_out.  `s` and `w` are scratch
 * arrays of at least kv_length(b) doubles. */
static void attend_row(const call_t *c, int b, int i, int h, double *o_row,
                       double *lse_out, double *s, double *w)
{
    const int D = c->D;
    const int g = c->Hq / c->Hkv;
    const int r = h / g; /* query head h reads KV head floor(h / g) */
    const int64_t n = kv_length(c, b);
    const int64_t q_off = (q_row(c, b, i) * c->Hq + h) * D;
    /* the head's sink logit (-inf: none), used as given */
    const double sink = c->sinks ? (double)c->sinks[h] : -INFINITY;

    /* scores of the visible keys; s[j] is left unused for hidden keys */
    int64_t n_visible = 0;
    for (int64_t j = 0; j < n; ++j) {
        if (!visible(c, b, i, j))
            continue;
        int64_t k_off = kv_row_offset(c, b, j, r);
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += decode(c->q, q_off + d, c->dtype) * kv_value(c, 0, k_off + d);
        s[j] = c->alpha * dot;
        if (c->softcap > 0.0) /* stage 6: the logit is c tanh(Z / c) */
            s[j] = c->softcap * tanh(s[j] / c->softcap);
        ++n_visible;
    }

    if (n_visible == 0 || sink == INFINITY) {
        /* no visible key: zero output, and the LSE of what the denominator
         * holds (-inf without a sink); a +inf sink takes all the weight */
        for (int d = 0; d < D; ++d)
            o_row[d] = 0.0;
        *lse_out = n_visible == 0 ? sink : INFINITY;
        return;
    }

    /* softmax of the logits over the visible keys, shifted by their maximum
     * (and the sink's); the sink adds to the denominator only */
    double m = sink;
    for (int64_t j = 0; j < n; ++j)
        if (visible(c, b, i, j) && s[j] > m)
            m = s[j];
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        if (!visible(c, b, i, j))
            continue;
        w[j] = exp(s[j] - m);
        l += w[j];
    }
    l += exp(sink - m);

    for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            if (!visible(c, b, i, j))
                continue;
            acc += w[j] * kv_value(c, 1, kv_row_offset(c, b, j, r) + d);
        }
        o_row[d] = acc / l;
    }
    *lse_out = m + log(l);
}

static int check_common(int B, int Sq, int Hq, int Hkv, int D, int dtype)
{
    if (B < 0 || Sq < 0 || Hq <= 0 || Hkv <= 0 || D <= 0)
        return -1;
    if (Hq % Hkv != 0)
        return -1;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_FP16)
        return -1;
    return 0;
}

/* Window bounds are -1 (unlimited) or >= 0; the softcap is 0 (none) or a
 * positive finite value (a negative cap is an error on the pages). */
static int set_options(call_t *c, int window_left, int window_right, float softcap)
{
    if (window_left < -1 || window_right < -1)
        return -1;
    if (!(softcap >= 0.0f) || isinf(softcap))
        return -1;
    c->window_left = window_left;
    c->window_right = window_right;
    c->softcap = (double)softcap;
    return 0;
}

static int64_t max_kv_length(const call_t *c)
{
    int64_t mx = 0;
    for (int b = 0; b < c->B; ++b)
        if (kv_length(c, b) > mx)
            mx = kv_length(c, b);
    return mx;
}

/* Evaluate the rows listed in sel (triples b, i, h).  o: [nsel, D], lse: [nsel]. */
static int run_rows(const call_t *c, const int32_t *sel, int64_t nsel, double *o, double *lse)
{
    int64_t scratch = max_kv_length(c);
    if (scratch < 1)
        scratch = 1;
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)scratch);
        double *w = (double *)malloc(sizeof(double) * (size_t)scratch);
        if (!s || !w) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t t = 0; t < nsel; ++t) {
                int b = sel[3 * t], i = sel[3 * t + 1], h = sel[3 * t + 2];
                attend_row(c, b, i, h, o + t * c->D, lse + t, s, w);
            }
        }
        free(s);
        free(w);
    }
    return failed ? -2 : 0;
}

/* Evaluate every row: o [B, Sq, Hq, D], lse [B, Hq, Sq]. */
static int run_all(const call_t *c, double *o, double *lse)
{
    int64_t nrows = 0;
    for (int b = 0; b < c->B; ++b)
        nrows += q_length(c, b) * c->Hq;
    if (nrows == 0)
        return 0;
    int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * 3 * (size_t)nrows);
    double *lse_rows = (double *)malloc(sizeof(double) * (size_t)nrows);
    if (!sel || !lse_rows) {
        free(sel);
        free(lse_rows);
        return -2;
    }
    /* row order b, i, h matches the BSHD (or packed THD) output, so o can be
     * written in place */
    int64_t t = 0;
    for (int b = 0; b < c->B; ++b)
        for (int i = 0; i < q_length(c, b); ++i)
            for (int h = 0; h < c->Hq; ++h) {
                sel[3 * t] = b;
                sel[3 * t + 1] = i;
                sel[3 * t + 2] = h;
                ++t;
            }
    int rc = run_rows(c, sel, nrows, o, lse_rows);
    t = 0;
    for (int b = 0; b < c->B; ++b)
        for (int i = 0; i < q_length(c, b); ++i)
            for (int h = 0; h < c->Hq; ++h) {
                if (c->cu_q) /* packed: lse [Hq, total_q] */
                    lse[(int64_t)h * c->total_q + q_row(c, b, i)] = lse_rows[t++];
                else /* lse [B, Hq, Sq] */
                    lse[((int64_t)b * c->Hq + h) * c->Sq + i] = lse_rows[t++];
            }
    free(sel);
    free(lse_rows);
    return rc;
}

static int make_dense(call_t *c, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                      int dtype, int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale,
                      int causal, int window_left, int window_right, float softcap,
                      const uint8_t *mask)
{
    if (check_common(B, Sq, Hq, Hkv, D, dtype) || Skv < 0)
        return -1;
    memset(c, 0, sizeof *c);
    c->q = q; c->k = k; c->v = v; c->dtype = dtype;
    c->B = B; c->Sq = Sq; c->Hq = Hq; c->Hkv = Hkv; c->D = D; c->Skv = Skv;
    c->causal = causal != 0;
    c->alpha = oracle_resolve_scale(scale, D);
    c->mask = mask;
    return set_options(c, window_left, window_right, softcap);
}

static int make_paged(call_t *c, const uint16_t *q, const void *k_cache,
                      const void *v_cache, const int32_t *seqlen,
                      const int32_t *block_table, int page_size, int causal, int window_left,
                      int window_right, float softcap, int B, int Sq, int Hq, int Hkv, int D,
                      int max_pages, float scale, int dtype)
{
    if (check_common(B, Sq, Hq, Hkv, D, dtype) || page_size <= 0 || max_pages < 0)
        return -1;
    for (int b = 0; b < B; ++b)
        if (seqlen[b] < 0 || (int64_t)seqlen[b] > (int64_t)max_pages * page_size)
            return -1;
    memset(c, 0, sizeof *c);
    c->q = q; c->k = k_cache; c->v = v_cache; c->dtype = dtype;
    c->B = B; c->Sq = Sq; c->Hq = Hq; c->Hkv = Hkv; c->D = D;
    c->causal = causal != 0;
    c->alpha = oracle_resolve_scale(scale, D);
    c->paged = 1;
    c->seqlen = seqlen;
    c->block_table = block_table;
    c->page_size = page_size;
    c->max_pages = max_pages;
    return set_options(c, window_left, window_right, softcap);
}

/* Dense call: q [B,Sq,Hq,D], k/v [B,Skv,Hkv,D] (16-bit bit patterns), mask
 * [B,Skv] or NULL; window bounds -1 (unlimited) or >= 0; softcap 0 (none) or
 * > 0.  Writes o [B,Sq,Hq,D] and lse [B,Hq,Sq] in double.
 * Returns 0, -1 on invalid arguments, -2 on allocation failure. */
int oracle_attn_dense(const uint16_t *q, const uint16_t *k, const uint16_t *v, int dtype,
                      int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale, int causal,
                      int window_left, int window_right, float softcap,
                      const uint8_t *key_padding_mask, double *o, double *lse)
{
    call_t c;
    if (make_dense(&c, q, k, v, dtype, B, Hq, Hkv, Sq, Skv, D, scale, causal, window_left,
                   window_right, softcap, key_padding_mask))
        return -1;
    return run_all(&c, o, lse);
}

/* Dense call, selected rows only: sel holds nsel triples (b, i, h).
 * Writes o [nsel, D] and lse [nsel]. */
int oracle_attn_dense_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v, int dtype,
                           int B, int Hq, int Hkv, int Sq, int Skv, int D, float scale,
                           int causal, int window_left, int window_right, float softcap,
                           const uint8_t *key_padding_mask, const int32_t *sel, int64_t nsel,
                           double *o, double *lse)
{
    call_t c;
    if (make_dense(&c, q, k, v, dtype, B, Hq, Hkv, Sq, Skv, D, scale, causal, window_left,
                   window_right, softcap, key_padding_mask))
        return -1;
    for (int64_t t = 0; t < nsel; ++t)
        if (sel[3 * t] < 0 || sel[3 * t] >= B || sel[3 * t + 1] < 0 || sel[3 * t + 1] >= Sq ||
            sel[3 * t + 2] < 0 || sel[3 * t + 2] >= Hq)
            return -1;
    return run_rows(&c, sel, nsel, o, lse);
}

/* Paged call: q [B,Sq,Hq,D]; k_cache/v_cache [pages*page_size, Hkv, D];
 * real_seqlen_kv [B]; block_table [B, max_pages].  Writes o and lse as the
 * dense call does. */
int oracle_attn_paged(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                      const int32_t *real_seqlen_kv, const int32_t *block_table, int page_size,
                      int causal, int window_left, int window_right, float softcap, int B,
                      int Sq, int Hq, int Hkv, int D, int max_pages, float scale, int dtype,
                      double *o, double *lse)
{
    call_t c;
    if (make_paged(&c, q, k_cache, v_cache, real_seqlen_kv, block_table, page_size, causal,
                   window_left, window_right, softcap, B, Sq, Hq, Hkv, D, max_pages, scale,
                   dtype))
        return -1;
    return run_all(&c, o, lse);
}

/* Paged call, selected rows only (triples b, i, h). */
int oracle_attn_paged_rows(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                           const int32_t *real_seqlen_kv, const int32_t *block_table,
                           int page_size, int causal, int window_left, int window_right,
                           float softcap, int B, int Sq, int Hq, int Hkv, int D, int max_pages,
                           float scale, int dtype, const int32_t *sel, int64_t nsel, double *o,
                           double *lse)
{
    call_t c;
    if (make_paged(&c, q, k_cache, v_cache, real_seqlen_kv, block_table, page_size, causal,
                   window_left, window_right, softcap, B, Sq, Hq, Hkv, D, max_pages, scale,
                   dtype))
        return -1;
    for (int64_t t = 0; t < nsel; ++t)
        if (sel[3 * t] < 0 || sel[3 * t] >= B || sel[3 * t + 1] < 0 || sel[3 * t + 1] >= Sq ||
            sel[3 * t + 2] < 0 || sel[3 * t + 2] >= Hq)
            return -1;
    return run_rows(&c, sel, nsel, o, lse);
}

/* Packed offsets: cu[0] = 0, nondecreasing, cu[B] = total. */
static int check_offsets(const int32_t *cu, int B, int total)
{
    if (!cu || cu[0] != 0 || cu[B] != total)
        return -1;
    for (int b = 0; b < B; ++b)
        if (cu[b + 1] < cu[b])
            return -1;
    return 0;
}

/* Packed (THD) dense call: q [total_q, Hq, D], k/v [total_kv, Hkv, D]; request
 * b holds queries cu_q[b] .. cu_q[b+1]-1 and keys cu_kv[b] .. cu_kv[b+1]-1;
 * sinks [Hq] float32 or NULL.  Writes o [total_q, Hq, D] and lse [Hq, total_q]. */
int oracle_attn_varlen(const uint16_t *q, const uint16_t *k, const uint16_t *v, int dtype,
                       const int32_t *cu_q, const int32_t *cu_kv, int B, int total_q,
                       int total_kv, int Hq, int Hkv, int D, float scale, int causal,
                       int window_left, int window_right, float softcap, const float *sinks,
                       double *o, double *lse)
{
    call_t c;
    if (B < 0 || total_q < 0 || total_kv < 0)
        return -1;
    if (make_dense(&c, q, k, v, dtype, B, Hq, Hkv, 0, 0, D, scale, causal, window_left,
                   window_right, softcap, NULL))
        return -1;
    if (check_offsets(cu_q, B, total_q) || check_offsets(cu_kv, B, total_kv))
        return -1;
    c.cu_q = cu_q;
    c.cu_kv = cu_kv;
    c.total_q = total_q;
    c.sinks = sinks;
    return run_all(&c, o, lse);
}

/* Packed-query paged call: q [total_q, Hq, D] delimited by cu_q [B+1]; caches
 * and block_table as for oracle_attn_paged; cache_seqlens [B] counts each
 * request's keys, its queries included.  Writes o [total_q, Hq, D] and lse
 * [Hq, total_q]. */
int oracle_attn_paged_varlen(const uint16_t *q, const uint16_t *k_cache,
                             const uint16_t *v_cache, const int32_t *cache_seqlens,
                             const int32_t *block_table, int page_size, const int32_t *cu_q,
                             int causal, int window_left, int window_right, float softcap,
                             const float *sinks, int B, int total_q, int Hq, int Hkv, int D,
                             int max_pages, float scale, int dtype, double *o, double *lse)
{
    call_t c;
    if (total_q < 0)
        return -1;
    if (make_paged(&c, q, k_cache, v_cache, cache_seqlens, block_table, page_size, causal,
                   window_left, window_right, softcap, B, 0, Hq, Hkv, D, max_pages, scale,
                   dtype))
        return -1;
    if (check_offsets(cu_q, B, total_q))
        return -1;
    c.cu_q = cu_q;
    c.total_q = total_q;
    c.sinks = sinks;
    return run_all(&c, o, lse);
}

/* As oracle_attn_paged_varlen over FP8 pools: k_cache / v_cache hold E4M3FN
 * codes, dequantized by k_scale / v_scale (finite and positive, else -1). */
int oracle_attn_paged_varlen_fp8(const uint16_t *q, const uint8_t *k_cache,
                                 const uint8_t *v_cache, float k_scale, float v_scale,
                                 const int32_t *cache_seqlens, const int32_t *block_table,
                                 int page_size, const int32_t *cu_q, int causal,
                                 int window_left, int window_right, float softcap,
                                 const float *sinks, int B, int total_q, int Hq, int Hkv, int D,
                                 int max_pages, float scale, int dtype, double *o, double *lse)
{
    call_t c;
    if (total_q < 0)
        return -1;
    if (!(k_scale > 0.0f) || !(v_scale > 0.0f) || isinf(k_scale) || isinf(v_scale))
        return -1;
    if (make_paged(&c, q, k_cache, v_cache, cache_seqlens, block_table, page_size, causal,
                   window_left, window_right, softcap, B, 0, Hq, Hkv, D, max_pages, scale,
                   dtype))
        return -1;
    if (check_offsets(cu_q, B, total_q))
        return -1;
    c.cu_q = cu_q;
    c.total_q = total_q;
    c.sinks = sinks;
    c.cache_fp8 = 1;
    c.k_scale = (double)k_scale;
    c.v_scale = (double)v_scale;
    return run_all(&c, o, lse);
}

/* ---------------------------------------------------------------- backward
 *
 * Dense call, inputs as for oracle_attn_dense plus o [B,Sq,Hq,D] and lse
 * [B,Hq,Sq] as doubles (exact copies of whatever the caller holds) and do
 * [B,Sq,Hq,D] 16-bit patterns.  With s_ij = alpha <q_i, k_j> over visible keys,
 *     P_ij = exp(s_ij - lse_i),  dP_ij = <dO_i, v_j>,  D_i = <dO_i, o_i>,
 *     dS_ij = P_ij (dP_ij - D_i),
 *     dq_i = alpha sum_j dS_ij k_j,  dk_j = alpha sum_i dS_ij q_i,
 *     dv_j = sum_i P_ij dO_i,
 * the sums over i running over the query heads of the KV head in group order,
 * then over query positions.  A row with lse = -inf (no visible key)
 * contributes nothing.  Writes dq [B,Sq,Hq,D], dk and dv [B,Skv,Hkv,D]. */
int oracle_attn_bwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, const double *o,
                    const uint16_t *dout, const double *lse, int dtype, int B, int Hq, int Hkv,
                    int Sq, int Skv, int D, float scale, int causal, double *dq, double *dk,
                    double *dv)
{
    call_t c;
    if (make_dense(&c, q, k, v, dtype, B, Hq, Hkv, Sq, Skv, D, scale, causal, -1, -1, 0.0f,
                   NULL))
        return -1;
    const int g = Hq / Hkv;
    const double alpha = c.alpha;
    memset(dq, 0, sizeof(double) * (size_t)B * Sq * Hq * D);
    memset(dk, 0, sizeof(double) * (size_t)B * Skv * Hkv * D);
    memset(dv, 0, sizeof(double) * (size_t)B * Skv * Hkv * D);
    /* one KV head at a time: its dk/dv rows are only touched here, and each
     * query row's dq only by its own head */
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < B; ++b)
        for (int r = 0; r < Hkv; ++r)
            for (int local = 0; local < g; ++local) {
                const int h = r * g + local;
                for (int i = 0; i < Sq; ++i) {
                    const double l_i = lse[((int64_t)b * Hq + h) * Sq + i];
                    if (l_i == -INFINITY)
                        continue;
                    const int64_t qo = (((int64_t)b * Sq + i) * Hq + h) * D;
                    double Di = 0.0;
                    for (int d = 0; d < D; ++d)
                        Di += decode(dout, qo + d, dtype) * o[qo + d];
                    for (int64_t j = 0; j < Skv; ++j) {
                        if (!visible(&c, b, i, j))
                            continue;
                        const int64_t ko = kv_row_offset(&c, b, j, r);
                        double s = 0.0, dp = 0.0;
                        for (int d = 0; d < D; ++d) {
                            s += decode(q, qo + d, dtype) * decode(k, ko + d, dtype);
                            dp += decode(dout, qo + d, dtype) * decode(v, ko + d, dtype);
                        }
                        const double p = exp(alpha * s - l_i);
                        const double ds = p * (dp - Di);
                        for (int d = 0; d < D; ++d) {
                            dq[qo + d] += alpha * ds * decode(k, ko + d, dtype);
                            dk[ko + d] += alpha * ds * decode(q, qo + d, dtype);
                            dv[ko + d] += p * decode(dout, qo + d, dtype);
                        }
                    }
                }
            }
    return 0;
}

/* ---------------------------------------------------------------- FP8 E4M3FN
 *
 * OCP 8-bit E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits; no
 * infinities; S.1111.111 is NaN, so the largest finite magnitude is
 * 1.110b * 2^8 = 448; exponent 0 holds zero and subnormals (fraction * 2^-9).
 */
static double e4m3_value(int code)
{
    int e = (code >> 3) & 15, f = code & 7;
    double mag;
    if (e == 15 && f == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)f, -9);
    else
        mag = ldexp((double)(8 + f), e - 10);
    return (code & 0x80) ? -mag : mag;
}

double oracle_e4m3_decode(int code) { return e4m3_value(code & 0xff); }

/* The E4M3FN code of x: the nearest finite value, ties to the even code (the
 * one with fraction bit 0), found by checking every non-negative code; NaN
 * stays NaN; magnitudes above 448, infinities included, saturate to 448. */
int oracle_e4m3_encode(double x)
{
    if (isnan(x))
        return signbit(x) ? 0xff : 0x7f;
    int sign = signbit(x) ? 0x80 : 0;
    double a = fabs(x);
    if (a >= 448.0)
        return sign | 0x7e;
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c <= 0x7e; ++c) {
        double err = fabs(e4m3_value(c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return sign | best;
}

/* ---------------------------------------------------------------- KV write
 *
 * Write token n's rows k[n], v[n] ([Hkv, D] 16-bit patterns) into pool row
 * slot[n] of k_pool / v_pool ([num_slots, Hkv, D]); slot -1 skips the token.
 * cache_fp8 = 0: the pool holds the same 16-bit patterns; 1: E4M3FN codes of
 * the value divided by k_scale / v_scale, the division done in float32 (the
 * precision of the scale and of the device computation).  Returns -1 for a
 * slot outside [-1, num_slots) or a non-positive scale. */
int oracle_kv_write(const uint16_t *k, const uint16_t *v, int dtype, const int64_t *slot,
                    int tokens, int Hkv, int D, int64_t num_slots, int cache_fp8,
                    float k_scale, float v_scale, void *k_pool, void *v_pool)
{
    if (tokens < 0 || Hkv <= 0 || D <= 0 || num_slots < 0)
        return -1;
    if (cache_fp8 && (!(k_scale > 0.0f) || !(v_scale > 0.0f) || isinf(k_scale) || isinf(v_scale)))
        return -1;
    for (int n = 0; n < tokens; ++n)
        if (slot[n] < -1 || slot[n] >= num_slots)
            return -1;
    const int64_t row = (int64_t)Hkv * D;
    for (int n = 0; n < tokens; ++n) {
        if (slot[n] < 0)
            continue;
        for (int64_t e = 0; e < row; ++e) {
            const int64_t src = (int64_t)n * row + e, dst = slot[n] * row + e;
            if (!cache_fp8) {
                ((uint16_t *)k_pool)[dst] = k[src];
                ((uint16_t *)v_pool)[dst] = v[src];
            } else {
                float kq = (float)decode(k, src, dtype) / k_scale;
                float vq = (float)decode(v, src, dtype) / v_scale;
                ((uint8_t *)k_pool)[dst] = (uint8_t)oracle_e4m3_encode((double)kq);
                ((uint8_t *)v_pool)[dst] = (uint8_t)oracle_e4m3_encode((double)vq);
            }
        }
    }
    return 0;
}

/* Paged prefill with append: request b's chunk (queries and
 * new keys/values at packed rows cu_q[b] .. cu_q[b+1]-1) is written to its
 * logical positions cache_seqlens[b] + i, i.e. pool row
 * block_table[b, pos / page_size] * page_size + pos % page_size; then the
 * chunk's queries attend to the request's cache_seqlens[b] + Sq_b keys.  The
 * pools (16-bit, or FP8 with cache_fp8 and its two scales: the chunk is
 * written quantized and read back dequantized) are updated in place;
 * o [total_q, Hq, D], lse [Hq, total_q]. */
int oracle_attn_paged_append(const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                             void *k_cache, void *v_cache, int cache_fp8, float k_scale,
                             float v_scale, const int32_t *cache_seqlens,
                             const int32_t *block_table, int page_size, const int32_t *cu_q,
                             int causal, float softcap, int B, int total_q, int Hq, int Hkv,
                             int D, int max_pages, int num_pages, float scale, int dtype,
                             double *o, double *lse)
{
    if (B < 0 || total_q < 0 || page_size <= 0 || max_pages <= 0 || num_pages < 0)
        return -1;
    if (check_offsets(cu_q, B, total_q))
        return -1;
    int64_t *slot = (int64_t *)malloc(sizeof(int64_t) * (size_t)(total_q > 0 ? total_q : 1));
    int32_t *lens = (int32_t *)malloc(sizeof(int32_t) * (size_t)(B > 0 ? B : 1));
    if (!slot || !lens) {
        free(slot);
        free(lens);
        return -2;
    }
    int rc = 0;
    for (int b = 0; b < B && rc == 0; ++b) {
        lens[b] = cache_seqlens[b] + (cu_q[b + 1] - cu_q[b]);
        if (cache_seqlens[b] < 0 || (int64_t)lens[b] > (int64_t)max_pages * page_size)
            rc = -1;
        for (int i = cu_q[b]; i < cu_q[b + 1] && rc == 0; ++i) {
            int64_t pos = (int64_t)cache_seqlens[b] + (i - cu_q[b]);
            int32_t page = block_table[(int64_t)b * max_pages + pos / page_size];
            if (page < 0 || page >= num_pages)
                rc = -1;
            slot[i] = (int64_t)page * page_size + pos % page_size;
        }
    }
    if (rc == 0)
        rc = oracle_kv_write(k_new, v_new, dtype, slot, total_q, Hkv, D,
                             (int64_t)num_pages * page_size, cache_fp8, k_scale, v_scale,
                             k_cache, v_cache);
    if (rc == 0 && cache_fp8)
        rc = oracle_attn_paged_varlen_fp8(q, (const uint8_t *)k_cache, (const uint8_t *)v_cache,
                                          k_scale, v_scale, lens, block_table, page_size, cu_q,
                                          causal, -1, -1, softcap, NULL, B, total_q, Hq, Hkv, D,
                                          max_pages, scale, dtype, o, lse);
    else if (rc == 0)
        rc = oracle_attn_paged_varlen(q, (const uint16_t *)k_cache, (const uint16_t *)v_cache,
                                      lens, block_table, page_size, cu_q, causal, -1, -1,
                                      softcap, NULL, B, total_q, Hq, Hkv, D, max_pages, scale,
                                      dtype, o, lse);
    free(slot);
    free(lens);
    return rc;
}

/* Number of threads an OpenMP parallel region uses here. */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
