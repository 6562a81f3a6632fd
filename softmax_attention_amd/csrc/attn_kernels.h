// attn_kernels.h -- launch parameters shared by the host library and the
// attention kernels of libmiattn (internal; not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace miattn {

// Packed-row tiling shared by the host planner and the kernels.
//
// The query rows of one (batch, KV head) pair are packed so that the g query
// heads that read this KV head sit next to each other: packed row r holds
// query i = r / g of head kvh * g + r % g.  Every packed row reads the same
// keys, so one K/V tile staged in LDS serves the whole group.
constexpr int kRowsPerWave = 32;  // one 32x32 MFMA column block

// Two schedules share one kernel template:
//   8 waves (512 threads, two per SIMD): the waves form two groups that
//     alternate, phase by phase, between an MFMA phase (QK^T of one tile and
//     P.V of the previous one) and a softmax phase, so each SIMD always has
//     one wave feeding the matrix core while the other runs VALU work
//     ("ping-pong"); used for D <= 128 prefill (paged only at D = 64).
//   streaming (3 waves for decode-shaped calls with D <= 128 -- wave 0
//     computes, waves 1 and 2 issue all loads -- and 4 waves for D = 256 and
//     for dense prefill at D = 64): each step computes one tile while later
//     tiles load.
//   paired decode (WAVES = 5 in the kernel template; four waves run, seven
//     over FP8 pools): the decode schedule for two adjacent KV heads at once
//     -- waves 0 and 1 compute one head each, waves 2 and 3 load both heads'
//     rows of every key (one contiguous 4 D-byte segment instead of two
//     2 D-byte ones); over FP8 pools wave 2 loads the 2 D-byte FP8 segments
//     and waves 3-6 convert them.
constexpr int kPairWaves = 5;
constexpr int rows_per_workgroup(int waves) {
    return (waves == 3 || waves == kPairWaves) ? kRowsPerWave : kRowsPerWave * waves;
}

// Keys per KV tile.  8 waves: 8192 / D keys, 16 KB per K or V tile (128 keys
// at D = 64, 64 at D = 128): the same registers and LDS either way, and at
// D = 64 twice the keys per softmax phase, which measured 6 % faster on the
// key-padding MHA than 64-key tiles.
// Decode-shaped (3 waves): 64 keys (16 KB at D = 128); the three-stage
// K and V rings then take 96 KB and one workgroup runs per CU, which streamed
// the paged decode 4-5 % faster than 32-key tiles with two workgroups per CU.
// Over FP8 pools: tiles of 8 KB of 16-bit values (4096 / D keys, at least
// one 32-key score block), so that the FP8 ring and the converted stages fit
// two workgroups per CU.  D = 256 (4 waves): 32 keys (16 KB).  Paired decode:
// 4096 / D keys (16 KB holding both heads' rows), over FP8 pools too.
constexpr int keys_per_tile(int D, int waves, bool fp8 = false) {
    return waves == 8 ? 8192 / D
           : waves == 4 ? 32
           : waves == kPairWaves ? 4096 / D
           : fp8 ? (4096 / D > 32 ? 4096 / D : 32) : 64;
}

// Per-request extents of a call, as the attention kernel, its stream-K plan
// and the merge kernel all read them (device helpers in attn_device.h clamp
// them identically).
struct SeqDesc {
    const int32_t *seqlen;  // paged: keys of request b, its queries included; else nullptr
    const int32_t *cu_q;    // packed queries: request b holds rows cu_q[b] .. cu_q[b+1]-1
    const int32_t *cu_kv;   // packed dense keys, likewise; nullptr: B blocks of skv keys
    int B;
    int sq;                 // queries per request (packed: the most one may hold)
    int skv;                // dense keys per request (packed: the most one may hold)
    int total_q, total_kv;  // packed row counts
    int cap;                // paged: max_pages * page_size (0 for an empty cache)
    int append;             // paged: seqlen counts the keys before a chunk of Sq_b queries
                            // whose keys were appended (the request holds seqlen + Sq_b)
};

struct FwdParams {
    const uint16_t *q;   // [B, Sq, Hq, D]
    const uint16_t *k;   // dense [B, Skv, Hkv, D] or paged cache [rows, Hkv, D]
    const uint16_t *v;
    uint16_t *o;         // [B, Sq, Hq, D]
    float *lse;          // [B, Hq, Sq] or nullptr
    float *o_part;       // [B*Hkv, n_splits, rows, D] when n_splits > 1
    float *lse_part;     // [B*Hkv, n_splits, rows]
    const uint8_t *mask; // dense key padding [B, Skv] or nullptr
    const int32_t *seqlen;      // paged: [B]
    const int32_t *block_table; // paged: [B, max_pages]
    const int32_t *cu_q;        // packed (THD) queries: offsets [B + 1], or nullptr
    const int32_t *cu_kv;       // packed dense keys: offsets [B + 1], or nullptr
    const float *sinks;         // [Hq] sink logits, or nullptr
    // FP8 E4M3FN pools (paged, 3-wave schedule): k/v point at codes, and the
    // element is code * *k_scale (or *v_scale); nullptr for 16-bit K/V
    const float *k_scale, *v_scale;
    int kv_append;              // paged: seqlen excludes the appended chunk (see SeqDesc)
    int total_q, total_kv;      // packed row counts (lse of a packed call is [Hq, total_q])
    int B, Sq, Hq, Hkv, G, Skv; // packed calls: Sq and Skv are the per-request maxima
    int page_shift, max_pages, num_pages;  // paged: log2(page size), table width, cache pages
    int rows;        // Sq * G packed rows per (batch, KV head)
    int n_mblocks;   // ceil(rows / rows_per_workgroup(waves))
    int n_splits;    // key-range splits per (batch, KV head)
    int split_len;   // keys per split, a multiple of the key tile
    int causal;
    // sliding window: query i sees keys [p_i - win_left, p_i + win_right]
    // (p_i = i + len - Sq), -1 = unlimited on that side; the host turns a
    // bound that cannot exclude any key into -1
    int win_left, win_right;
    float scale_log2;  // |alpha| * log2(e)
    // logit softcap C (capped kernels only): L log2(e) = cap_k2 * tanh(z alpha / C)
    // with cap_k2 = C log2(e) and tanh(x) = 1 - 2 / (2^(cap_x s) + 1),
    // cap_x = 2 log2(e) |alpha| / C, s being the raw score q.k
    float cap_x, cap_k2;
    int q_mode;        // 0: q as given; 1: q negated (alpha < 0); 2: q zeroed (alpha == 0)
    int xcd_units;     // (batch*KV head, split) units per XCD, or 0 for linear order
    int heads_inner;   // units ordered (batch, split, KV head) instead of (batch, KV head, split)
    // stream-K decode (split-role schedules): grid size G (a multiple of U =
    // Hkv / KV heads per workgroup), or 0.  Workgroup g serves the head unit
    // g % U (KV head g % U, or heads 2 (g % U) and 2 (g % U) + 1 when
    // paired), and the G / U workgroups of one unit split its key tiles, so
    // the U workgroups g, g + 1, ... read the same cache rows together
    int sk_grid;
    // stream-K: plan weight, in key tiles, of starting a piece of a unit
    int sk_piece;
};

struct MergeParams {
    const float *o_part;
    const float *lse_part;
    uint16_t *o;
    float *lse;
    const int32_t *seqlen;  // paged lengths, or nullptr for dense
    const int32_t *cu_q, *cu_kv;
    const float *sinks;
    int total_q, total_kv;
    int kv_append;
    int Skv;
    int B, Sq, Hq, Hkv, G, rows, n_splits, split_len;
    // stream-K decode: grid size (0 otherwise), keys per tile and the length
    // clamp the attention kernel applies (max_pages * page_size, 0 for an
    // empty cache), the left window bound (-1: none), the plan weight of a
    // piece and the KV heads one workgroup served (1, or 2 when paired) --
    // all as the attention kernel had them
    int sk_grid, sk_bn, sk_cap, sk_win_left, sk_piece, sk_hpw;
};

// Launchers: return the hipGetLastError() status of the launch.  The
// attention kernels of one head dimension and logit kind (plain or capped)
// are compiled in a translation unit of their own (attn_fwd.hip built once
// per pair), which defines these two templates for its pair.
template <int D, bool CAP>
hipError_t launch_attn_fwd_dc(const FwdParams &p, bool bf16, bool paged, int waves, int grid,
                              hipStream_t stream);
// Workgroups of the decode-shaped (3-wave) attention kernel one CU runs
// at once (0 if unknown).
template <int D, bool CAP>
int decode_blocks_per_cu_dc(const FwdParams &p, bool bf16, bool paged, int waves);

// Dispatch over the (D, CAP) pairs (miattn.hip; kept out of this header so
// that a kernel unit does not instantiate the other units' kernels).
hipError_t launch_attn_fwd(const FwdParams &p, int D, bool bf16, bool paged, int waves,
                           bool cap, int grid, hipStream_t stream);
int attn_fwd_decode_blocks_per_cu(const FwdParams &p, int D, bool bf16, bool paged, int waves,
                                  bool cap);

hipError_t launch_lse_merge(const MergeParams &p, int D, bool bf16, hipStream_t stream);

// Attention backward (attn_bwd.hip): dq [B,Sq,Hq,D], dk and dv [B,Skv,Hkv,D]
// from q, k, v, o, do (16-bit, BSHD) and lse [B,Hq,Sq]; d_rows and lse2_rows
// ([B,Hq,Sq] fp32, library workspace) carry <dO_i, o_i> and lse_i log2(e).
struct BwdParams {
    const uint16_t *q, *k, *v, *o, *dout;
    const float *lse;
    uint16_t *dq, *dk, *dv;
    float *d_rows, *lse2_rows;
    int B, Sq, Skv, Hq, Hkv, G;
    int rows;       // Sq * G packed rows per (batch, KV head)
    int n_mblocks;  // ceil(rows / 128)
    int causal;
    float scale;       // alpha
    float scale_log2;  // alpha log2(e)
    int down_wgs;      // bwd_dkdv workgroups 0 .. down_wgs - 1 walk their row tiles downwards
};
hipError_t launch_attn_bwd(const BwdParams &p, int D, bool bf16, hipStream_t stream);
// Zero `bytes` (a multiple of 16) at a 16-byte aligned device address with a
// kernel (no memset node, so the call can sit inside a captured graph).
hipError_t launch_zero_fill(void *ptr, size_t bytes, hipStream_t stream);

// Paged KV-cache write (kv_write.hip): token n's K and V rows ([row_elems]
// 16-bit values) go to pool row slot(n) -- slot_mapping[n], or in append mode
// the position cache_seqlens[b] + i of the packed chunk's token i of request
// b through the block table; slots outside [0, num_slots) are skipped.
struct KvWriteParams {
    const uint16_t *k, *v;             // [tokens, row_elems]
    uint16_t *k_pool16, *v_pool16;     // 16-bit pools [num_slots, row_elems]
    uint8_t *k_pool8, *v_pool8;        // FP8 E4M3FN pools [num_slots, row_elems]
    const float *k_scale, *v_scale;    // FP8: device divisors [1]
    const int64_t *slot_mapping;       // [tokens]
    const int32_t *cu_q, *cache_seqlens, *block_table;  // append mode
    int tokens, row_elems, B, page_size, max_pages;
    int64_t num_slots;
};
hipError_t launch_kv_write(const KvWriteParams &p, bool bf16, bool fp8, bool append,
                           hipStream_t stream);

}  // namespace miattn
