// attn_fwd.hip -- grouped-query softmax attention forward for gfx950 (CDNA4).
//
// Computes, for each packed query row of one (batch, KV head) pair, the
// online-softmax form of
//     O = softmax(alpha * Q K^T + M) V,  lse = ln sum_j exp(alpha <q, k_j>)
// over a range of keys (all keys, or one split of them).  Definitions: TileOPs
// "Attention Operators", GQADenseFwdOp stages 1, 4, 5 and 7 (end-aligned
// causal visibility j <= i + S_kv - S_q, FP32 accumulation, output in the
// input dtype) and MHADecodePagedWithKVCacheFwdOp (paged layout); RL-Kernel
// "Standard Softmax Attention", Tensor Contract (key padding mask, verbatim
// scale).  The streaming form -- a running maximum m, a running denominator l
// and the output rescaled by exp(m_old - m_new) whenever m grows -- is the
// published online softmax (Milakov & Gimelshein 2018, as used by Dao et al.
// 2022); it equals the plain definition in exact arithmetic.
//
// Work decomposition:
//   * rows: the query rows of the G = Hq/Hkv heads that share a KV head are
//     packed (row r = query r / G, head kvh*G + r % G), so one K/V tile
//     serves the whole group; a computing wave owns 32 packed rows.  In
//     decode (Sq = 1) the whole GQA group lands in one wave's MFMA tile.
//   * keys: a workgroup walks its key range in tiles; K and V go from HBM
//     straight into LDS ring stages with buffer_load ... lds (no registers),
//     ordered by counted vmcnt waits and an LDS-only barrier.  Schedules
//     (WAVES): 8 waves in two groups alternating MFMA and softmax phases over
//     16 KB tiles (prefill, D <= 128); 3 waves where wave 0 computes
//     and the others only load (decode, D <= 128; over FP8 pools one wave
//     loads and two convert), optionally as a persistent stream-K grid that
//     gives every workgroup an equal share of all key tiles; 4 waves that all
//     load and compute over 32-key tiles (D = 256, and dense prefill at
//     D = 64, several workgroups per CU).
//   * scores: S^T = K Q^T with v_mfma_f32_32x32x16_{bf16,f16}: K (from LDS) is
//     the A operand, Q (held in registers for the whole kernel) the B operand.
//     Each lane then holds 16 scores per 32-key block for ONE query row (its
//     column), so the row max needs one cross-lane step (lane ^ 32) and the row
//     sum none until the end.
//   * P.V: O^T = V^T P^T.  The exponentiated scores are already laid out as the
//     B operand (row = lane's column, 8 keys per lane), so P goes from the
//     score registers to the MFMA without any data movement; V^T is read from
//     the row-major V tile with the transposing LDS read; O^T accumulates in
//     registers with each lane owning one row, which makes the per-row
//     rescaling lane-local.
//   * masking: a tile that is fully visible to every row of a wave takes no
//     per-element test; a tile beyond a wave's last visible key is skipped by
//     that wave; tiles beyond the workgroup's last visible key are never
//     loaded; with a key padding mask, tiles whose keys are all masked are
//     skipped before their K/V is loaded.
#include "attn_kernels.h"

#include <type_traits>

#include "attn_device.h"

namespace miattn {
namespace {

using namespace dev;


// Waves per SIMD the register budget is sized for: the 8-wave schedule needs
// its two waves per SIMD, and so do two decode workgroups over FP8 pools (four
// waves each) on one CU; a 16-bit decode workgroup (96 KB of LDS at D = 128)
// and the 4-wave D = 256 schedule run one workgroup per CU.  The 4-wave
// schedule at D = 64 (24 KB of LDS) is held to four waves' registers per SIMD
// (128), so that four workgroups share a CU and the hardware interleaves their
// softmax and MFMA work: on the key-padding MHA (D = 64, fp16) this ran
// 85 -> 80 us against the 8-wave ping-pong, whose softmax phase there is about
// 2.7 times its MFMA phase.
template <int D, int WAVES, bool FP8>
constexpr int waves_per_eu() {
    return WAVES == kPairWaves ? 1
           : (WAVES == 4 && D == 64) ? 4
           : (WAVES == 8 || (WAVES == 3 && (FP8 || D < 128))) ? 2 : 1;
}

#ifndef MIATTN_READ_AHEAD
#define MIATTN_READ_AHEAD 6
#endif
constexpr int kReadAhead = MIATTN_READ_AHEAD;

// Scheduling hint for a block of LDS operand reads feeding MFMAs: issue
// kReadAhead reads first, then keep about that many in flight ahead of the
// MFMAs that consume them, so the matrix core does not wait out each read.
template <int N_READS, int N_MFMA>
__device__ __forceinline__ void sched_read_ahead() {
    constexpr int per = (N_READS - kReadAhead + N_MFMA - 1) / N_MFMA;
    __builtin_amdgcn_sched_group_barrier(0x100, kReadAhead, 0);  // DS read
#pragma unroll
    for (int i = 0; i < N_MFMA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, per, 0);  // DS read
    }
}

// (The kernel's helper lambdas are marked always_inline: an outlined one
// would take the parameter block by address and push it to scratch.)
//
// K/V source: dense tensors, a paged cache whose pages hold whole key tiles,
// or a paged cache with pages smaller than a tile (each 1 KB piece then
// looks up its own page); the last two again over FP8 E4M3FN pools.
enum KvMode { kDense = 0, kPagedTile = 1, kPagedPiece = 2, kPagedTile8 = 3, kPagedPiece8 = 4 };

// Waves of a workgroup: the schedule's WAVES (the paired decode: two
// computing and two loading waves); over FP8 pools one computing, one
// loading and two converting waves, or paired two computing, one loading and
// four converting waves
template <int WAVES, int KV>
constexpr int group_waves() {
    return (KV == kPagedTile8 || KV == kPagedPiece8) ? (WAVES == kPairWaves ? 7 : WAVES + 1)
                                                     : (WAVES == kPairWaves ? 4 : WAVES);
}

// CAP: logits are capped (c tanh(z / c), TileOPs "Attention Operators",
// GQADenseFwdOp stage 6); otherwise the logit is the scaled score itself.
template <int D, bool BF16, int KV, int WAVES, bool CAP>
__global__ __launch_bounds__((64 * group_waves<WAVES, KV>()))
__attribute__((amdgpu_waves_per_eu(waves_per_eu<D, WAVES, (KV == kPagedTile8 || KV == kPagedPiece8)>(),
                                   waves_per_eu<D, WAVES, (KV == kPagedTile8 || KV == kPagedPiece8)>())))
void attn_fwd_kernel(const FwdParams p) {
    constexpr bool PAGED = KV != kDense;
    // FP8 pools: K and V hold E4M3FN codes (paging mode KV - 2), dequantized
    // by one scale each (TileOPs "Attention Operators",
    // GQAPrefillPagedWithKVCacheFwdOp: the k_scale and v_scale of an FP8 pool)
    constexpr bool FP8 = KV == kPagedTile8 || KV == kPagedPiece8;
    constexpr int KVP = FP8 ? KV - 2 : KV;
    using H = Half<BF16>;
    using vec8 = typename H::vec8;
    // Paired decode: two adjacent KV heads, waves 0 and 1 computing one each;
    // an LDS row (and the segment loaded per key) holds both heads' DL = 2 D
    // values.
    constexpr bool PAIR = WAVES == kPairWaves;
    constexpr int DL = PAIR ? 2 * D : D;           // values per LDS key row
    constexpr int BM = rows_per_workgroup(WAVES);  // packed rows per workgroup
    constexpr int BN = keys_per_tile(D, WAVES, FP8);  // keys per tile
    constexpr int TILE_BYTES = BN * DL * 2;        // one K (or V) tile
    constexpr int PIECES = TILE_BYTES / 1024;      // 1 KB direct loads per tile
    // The decode schedule (3 waves) splits the roles: wave 0 computes,
    // the other waves issue every load (one loading wave streams only about
    // half of what a CU's memory path takes).  Otherwise each wave issues an
    // equal share.
    constexpr bool SPLIT_ROLES = WAVES == 3 || PAIR;
    constexpr int NCOMP = PAIR ? 2 : 1;            // computing waves of the split roles
    constexpr int LOADERS = PAIR ? 2 : SPLIT_ROLES ? WAVES - 1 : WAVES;
    constexpr int PPW = PIECES / LOADERS;          // 1 KB pieces per loading wave
    constexpr int NT = BN / 32;                    // 32-key score blocks per tile
    constexpr int KSTEPS = D / 16;                 // MFMA k-steps over D
    constexpr int DT = D / 32;                     // 32-wide d blocks of O^T
    constexpr int PSTEPS = BN / 16;                // MFMA k-steps over the tile's keys
    static_assert(PIECES % LOADERS == 0, "whole 1 KB pieces per loading wave");
    // The decode schedules stream K/V that no other workgroup reads again:
    // their loads carry the non-temporal hint (paged decode: kernel 184 ->
    // 163 us, call 195 -> 173 us; FP8 pools 107 -> 104 us).  The prefill
    // schedules share each tile between workgroups through L2 and keep the
    // default policy (the hint there: causal GQA prefill 276-282 -> 291-293 us).
    constexpr int LOAD_POLICY = SPLIT_ROLES ? kLoadNonTemporal : 0;
    static_assert(!FP8 || SPLIT_ROLES, "FP8 pools are read by the split-role schedules");

    // K and V rings of up to four stages each (the schedules use three or
    // four); separate arrays so that the compiler can tell a load into one
    // stage from reads of another
    __shared__ __attribute__((aligned(1024))) uint8_t sK0[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sV0[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sK1[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sV1[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sK2[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sV2[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sK3[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sV3[TILE_BYTES];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hl = lane >> 5;

    // request extents: uniform blocks, packed (THD) offsets or paged lengths,
    // clamped so that malformed ones stay inside the tensors
    const SeqDesc sd = {PAGED ? p.seqlen : nullptr, p.cu_q, PAGED ? nullptr : p.cu_kv, p.B,
                        p.Sq, p.Skv, p.total_q, p.total_kv,
                        (PAGED && p.num_pages > 0) ? (p.max_pages << p.page_shift) : 0,
                        PAGED ? p.kv_append : 0};

    // ---- the computing wave's state for its current unit: the key limits of
    // its row, Q, the output accumulator, the running max and denominator
    const bool has_mask = !PAGED && p.mask != nullptr;
    int my_last = -1, my_first = 0;
    int64_t slot_head_stride = 0;  // paired stream-K: partial slots between the two heads
    vec8 qf[KSTEPS];
    f32x16 acc[DT];
    float m_run = -INFINITY;  // running (possibly stale) max, scaled log2 units
    float l_run = 0.f;        // this lane's part of the running denominator

    // Q of this lane's row (at qrow) as the B operand -- 8 d-values per
    // k-step -- and a fresh accumulator.  The host folds the sign of the
    // scale into Q (an exact sign flip) and turns a zero scale into a zero Q,
    // so the kernel always scales by c > 0 and the row max stays a max.
    auto begin_rows = [&](const uint16_t *qrow, const bool row_ok) __attribute__((always_inline)) {
        const uint32_t flip = p.q_mode == 1 ? 0x80008000u : 0u;
        const bool load_q = row_ok && p.q_mode != 2;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (load_q) raw = *(const u32x4 *)(qrow + 16 * ks + 8 * hl) ^ flip;
            qf[ks] = __builtin_bit_cast(vec8, raw);
        }
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
        m_run = -INFINITY;
        l_run = 0.f;
    };

    // (an FP8 pool's key scale multiplies every raw score, so it joins the
    // factors applied to the raw score)
    const float k_deq = FP8 ? *p.k_scale : 1.f;
    const float c = p.scale_log2 * k_deq;  // > 0
    const float cap_x = p.cap_x * k_deq, cap_k2 = p.cap_k2;

    // ---- LDS read addresses, fixed per lane for the whole kernel.  With the
    // swizzle depending on row & 15 only, the 32-key block t and the 16-key
    // step kk move a read by whole rows (an immediate offset); only the chunk
    // index varies with the swizzle, so one byte offset per chunk position is
    // kept in a register.
    //   K (QK^T A operand): lane reads row 32t + l32, chunk 2ks + hl.
    //   V (transposing read): in each 16-lane group g, lane 4r+q reads row
    //   4*(g/2) + r (+8 for k-slots 4..7) of the 16-key step, d-columns
    //   32t + 16*(g%2) + 4q .. +3.
    // (paired: computing wave w reads the half of each row that holds head
    // kvh + w, chunks [w D / 8, (w + 1) D / 8); the swizzle only permutes a
    // row's chunks within aligned groups of 16, so each head keeps its half)
    const int hc = PAIR ? (wave & 1) * (D / 8) : 0;
    int k_addr[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) k_addr[ks] = tile_off<DL>(l32, hc + 2 * ks + hl);
    const int tr_g = lane >> 4;
    const int tr_row = 4 * (tr_g >> 1) + ((lane & 15) >> 2);
    const int tr_col = 16 * (tr_g & 1) + 4 * (lane & 3);
    int v_addr[DT][2];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int col = 8 * hc + 32 * t + tr_col;
            v_addr[t][h] = tile_off<DL>(tr_row + 8 * h, col >> 3) + (col & 7) * 2;
        }

    // ---- S^T = K Q^T for one tile (K from an LDS stage)
    auto qk = [&](const uint8_t *sk, f32x16 (&sc)[NT]) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[t][r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const vec8 a = __builtin_bit_cast(
                    vec8, *(const u32x4 *)(sk + k_addr[ks] + 32 * t * (2 * DL)));
                sc[t] = H::mfma(a, qf[ks], sc[t]);
            }
        }
    };

    // ---- online softmax of one tile's scores: masks (MASKED tiles only), the
    // lazy max update (unmasked tiles: only when their exponentials against
    // the running max would leave the range kFastSum allows), P rounded to 16
    // bits as the B operand of P.V, and the running denominator.  Branch-free, so that the scheduler can interleave
    // it with the next tile's QK^T MFMAs.  Returns the factor the output
    // accumulator must be multiplied by (1 when the max did not move).
    auto softmax = [&](auto masked_tag, int j0, uint64_t mlo, uint64_t mhi, f32x16 (&sc)[NT],
                       vec8 (&pb)[PSTEPS]) __attribute__((always_inline)) -> float {
        constexpr bool MASKED = decltype(masked_tag)::value;
        if constexpr (MASKED) {
            // S^T layout: register r of lane half hl holds key
            // 32t + 8*(r/4) + 4*hl + r%4 of the tile
            // this lane's keys of block t are 32t + 4hl + bit, bit = 8*(r/4) + r%4;
            // one word per block holds the visible ones: the padding mask's
            // bits and-ed with the row's key range [lim_lo, lim]
            const int lim = my_last - j0 - 4 * hl;
            const int lim_lo = my_first - j0 - 4 * hl;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                uint32_t w = ~0u;
                if (has_mask) w = (uint32_t)((t < 2 ? mlo : mhi) >> (32 * (t & 1) + 4 * hl));
                const int hi_c = min(max(lim - 32 * t, -1), 31);
                const int lo_c = min(max(lim_lo - 32 * t, 0), 32);
                w &= (uint32_t)((1ull << (hi_c + 1)) - 1) & (uint32_t)(~0ull << lo_c);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const bool vis = (w >> (8 * (r >> 2) + (r & 3))) & 1u;
                    sc[t][r] = vis ? sc[t][r] : -INFINITY;
                }
            }
        }
        // The tile's exponentials against offset m_off (the running max, or
        // 0 while it is -inf), rounded to 16 bits into pb; returns this
        // lane's part of their sum.
        auto exps = [&](const float m_off) __attribute__((always_inline)) -> float {
            // exp2 argument of raw score s: the logit minus the running max
            const float cap_off = cap_k2 - m_off;
            auto arg = [&](float s) __attribute__((always_inline)) -> float {
                if constexpr (CAP) {
                    // capped logit in log2 units: cap_k2 tanh(x) with
                    // tanh(x) = 1 - 2 / (e^{2x} + 1), which needs no sign
                    // split (e^{2x} -> 0 gives -1, -> inf gives 1)
                    const float r = __builtin_amdgcn_rcpf(fast_exp2(s * cap_x) + 1.f);
                    const float a = __builtin_fmaf(r, -2.f * cap_k2, cap_off);
                    // a hidden key (s = -inf) would get r = 1, a finite logit
                    return (MASKED && s == -INFINITY) ? -INFINITY : a;
                } else {
                    return __builtin_fmaf(s, c, -m_off);
                }
            };
            float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
            for (int kk = 0; kk < PSTEPS; ++kk) {
                const int t = kk >> 1, u = kk & 1;
                u32x4 packed;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float e0 = fast_exp2(arg(sc[t][8 * u + 2 * e]));
                    const float e1 = fast_exp2(arg(sc[t][8 * u + 2 * e + 1]));
                    packed[e] = pack_half2<BF16>(e0, e1);
                    // For bf16 the denominator sums P in FP32 before rounding:
                    // in a row dominated by one key, that key's P rounded to
                    // bf16 (8 significant bits) would carry up to 2^-8 of
                    // relative error into l and the lse.  fp16 (11 bits,
                    // error <= 2^-11) sums the rounded pair with one dot product.
                    if constexpr (BF16) {
                        if (e & 1)
                            rs1 += e0 + e1;
                        else
                            rs0 += e0 + e1;
                    } else {
                        if (e & 1)
                            rs1 = add_pair<BF16>(packed[e], rs1);
                        else
                            rs0 = add_pair<BF16>(packed[e], rs0);
                    }
                }
                pb[kk] = __builtin_bit_cast(vec8, packed);
            }
            return rs0 + rs1;
        };

        // (Not for capped logits at D = 64: there the two passes' capped
        // logits overflowed the registers of the 8-wave schedule into
        // scratch inside the loop.)
        if constexpr (!MASKED && !(CAP && D == 64)) {
            // An unmasked tile first takes its exponentials against the
            // running max as it stands, without forming the tile's max: the
            // max only guards the exponentials' range, so as long as every
            // lane's sum stays at most kFastSum (each P at most 2^24) the
            // result is the same in exact arithmetic and O needs no
            // rescaling.  A row that has not seen a key (running max -inf)
            // gets infinite exponentials, which send the tile through the
            // max below like a sum over the limit.  (A NaN score gives a NaN
            // sum, which passes the test and goes on into l, as below.)
            const float rs = exps(m_run);
            if (!__any(rs > kFastSum)) {
                l_run += rs;
                return 1.f;
            }
        }
        // row max of the raw scores (the logit is increasing in the raw
        // score, capped or not, so the max logit is the logit of the max)
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[t][r]);
        mx = max_halves(mx);
        float tile_max;
        if constexpr (CAP)
            tile_max = (mx == -INFINITY)
                           ? -INFINITY
                           : cap_k2 - 2.f * cap_k2 *
                                          __builtin_amdgcn_rcpf(fast_exp2(mx * cap_x) + 1.f);
        else
            tile_max = (mx == -INFINITY) ? -INFINITY : mx * c;
        const bool raise = __any(tile_max > m_run + kLazy);
        const float m_new = raise ? fmaxf(m_run, tile_max) : m_run;
        const float corr = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
        m_run = m_new;
        const float rs = exps((m_new == -INFINITY) ? 0.f : m_new);
        l_run = __builtin_fmaf(l_run, corr, rs);
        return corr;
    };

    // ---- O^T += V^T P^T; the V^T operand comes from two transposing reads of
    // 4 keys each (k-slots 0..3 and 4..7 of this lane half)
    auto pv = [&](const uint8_t *sv, const vec8 (&pb)[PSTEPS]) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int kk = 0; kk < PSTEPS; ++kk) {
                const int step = 16 * kk * (2 * DL);
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)(sv + v_addr[t][0] + step));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)(sv + v_addr[t][1] + step));
                const vec8 a = __builtin_bit_cast(
                    vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                acc[t] = H::mfma(a, pb[kk], acc[t]);
            }
    };

    // ---- the same two products with every operand read of a batch (up to
    // 8 MFMAs) issued before its MFMAs: for the streaming schedules, where the
    // scheduler otherwise waits out one LDS read before each MFMA
    auto qk_batched = [&](const uint8_t *sk, f32x16 (&sc)[NT]) __attribute__((always_inline)) {
        constexpr int CH = KSTEPS < 8 ? KSTEPS : 8;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[t][r] = 0.f;
#pragma unroll
            for (int k0 = 0; k0 < KSTEPS; k0 += CH) {
                vec8 a[CH];
#pragma unroll
                for (int c = 0; c < CH; ++c)
                    a[c] = __builtin_bit_cast(
                        vec8, *(const u32x4 *)(sk + k_addr[k0 + c] + 32 * t * (2 * DL)));
                __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
#pragma unroll
                for (int c = 0; c < CH; ++c) sc[t] = H::mfma(a[c], qf[k0 + c], sc[t]);
            }
        }
    };
    auto pv_batched = [&](const uint8_t *sv, const vec8 (&pb)[PSTEPS]) __attribute__((always_inline)) {
        constexpr int TB = (8 / PSTEPS) < DT ? (8 / PSTEPS) : DT;  // d blocks per batch
#pragma unroll
        for (int t0 = 0; t0 < DT; t0 += TB) {
            vec8 a[TB][PSTEPS];
#pragma unroll
            for (int t = 0; t < TB; ++t)
#pragma unroll
                for (int kk = 0; kk < PSTEPS; ++kk) {
                    const int step = 16 * kk * (2 * DL);
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4 *)(sv + v_addr[t0 + t][0] + step));
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4 *)(sv + v_addr[t0 + t][1] + step));
                    a[t][kk] = __builtin_bit_cast(
                        vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < TB; ++t)
#pragma unroll
                for (int kk = 0; kk < PSTEPS; ++kk) acc[t0 + t] = H::mfma(a[t][kk], pb[kk], acc[t0 + t]);
        }
    };


    // ---- HBM -> LDS, no registers: each 1 KB piece of a tile is one
    // buffer_load_dwordx4 ... lds (lane l fills bytes [16l, 16l+16) of the
    // piece); piece e*WAVES + wave is this wave's e-th and covers RPP
    // consecutive keys.  The load's base address is scalar (block-table
    // entries are read through the scalar cache) and each lane adds a small
    // offset: its key, and the chunk that the swizzle puts at its position.
    // Keys past the end load the last key (finite data, masked later).
    //
    // The buffer form, unlike global_load_lds, is not a FLAT instruction: the
    // compiler then counts the LDS reads that follow (lgkmcnt(n)) instead of
    // waiting for all of them whenever a direct load is in flight.
    constexpr int RPP = 512 / DL;                               // keys per piece
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);    // wave-uniform
    const int loader = SPLIT_ROLES ? wave_u - NCOMP : wave_u;  // this wave's index among the loaders
    const bool loads = !SPLIT_ROLES || wave_u >= NCOMP;
    const int l_dr = lane / (DL / 8);   // this lane's key within a piece
    const int l_pos = lane % (DL / 8);  // this lane's 16-byte position in the row
    const int64_t hstride = (int64_t)p.Hkv * D;  // elements between consecutive keys
    const int row_bytes = p.Hkv * D * 2;
    int l_chunk[PPW];  // byte offset, within its key row, of the chunk this lane fetches
#pragma unroll
    for (int e = 0; e < PPW; ++e)
        l_chunk[e] = 16 * (l_pos ^ swz<DL>((e * LOADERS + loader) * RPP + l_dr));
    // Where a tile lies in one page (always, for dense K/V) a single buffer
    // descriptor based at the tile's first key serves all pieces and each
    // lane clamps its own key; with smaller pages each piece gets its own
    // base.  (The scalar unit is shared by the CU's waves, so the per-step
    // scalar address arithmetic is kept small.)
    constexpr bool tile_in_page = KVP != kPagedPiece;
    typedef __attribute__((address_space(4))) const int32_t const_i32;
    int l_key[PPW];  // this lane's key row within the tile, per piece
#pragma unroll
    for (int e = 0; e < PPW; ++e) l_key[e] = (e * LOADERS + loader) * RPP + l_dr;
    auto cache_row = [&](int32_t phys, int j) __attribute__((always_inline)) -> int64_t {
        // (page ids clamped into the cache, so that a malformed table cannot
        // address memory outside it)
        return ((int64_t)min(max(phys, 0), p.num_pages - 1) << p.page_shift) +
               (j & ((1 << p.page_shift) - 1));
    };

    // a split result: the normalised FP32 output row and its natural-log LSE
    // at partial row `part`
    auto store_partial = [&](const int64_t part, const float inv, const float lse_v) __attribute__((always_inline)) {
        float *op = p.o_part + part * D;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int d0 = 32 * t + 8 * w + 4 * hl;
                const f32x4 v4 = {acc[t][4 * w] * inv, acc[t][4 * w + 1] * inv,
                                  acc[t][4 * w + 2] * inv, acc[t][4 * w + 3] * inv};
                *(f32x4 *)(op + d0) = v4;
            }
        if (hl == 0) p.lse_part[part] = lse_v;
    };

    // Keys query i of a request with kv_len keys may see before the padding
    // mask (TileOPs "Attention Operators", GQADenseFwdOp stage 5): [key_lo,
    // key_hi], both nondecreasing in i; the query sits at key position i +
    // delta.  (The host keeps i + delta + win_right in range.)
    auto key_hi_of = [&](int i, int kv_len, int delta) __attribute__((always_inline)) -> int {
        int h = kv_len - 1;
        if (p.causal) h = min(h, i + delta);
        if (p.win_right >= 0) h = min(h, i + delta + p.win_right);
        return h;
    };
    auto key_lo_of = [&](int i, int delta) __attribute__((always_inline)) -> int {
        return p.win_left >= 0 ? max(0, i + delta - p.win_left) : 0;
    };

    // ---- one unit of work: the key range [kbeg, kend) of row block `mblock`
    // of (batch b, KV head kvh), whose length is kv_len; a split result goes
    // to partial slot `slot`, a whole result straight to o and lse.
    auto run = [&](const int mblock, const int b, const int kvh, const int kv_len,
                   const int kbeg, const int kend, const int64_t slot,
                   const bool partial) __attribute__((always_inline)) {
    // this request's queries: packed rows q_row0 .. q_row0 + sq_b - 1
    int64_t q_row0;
    int sq_b;
    q_span(sd, b, q_row0, sq_b);
    const int rows_b = sq_b * p.G;  // its packed rows
    if (mblock * BM >= rows_b) return;  // a shorter request: no rows in this block
    const int delta = kv_len - sq_b;  // query i sits at key position p_i = i + delta

    auto key_hi = [&](int i) __attribute__((always_inline)) -> int {
        return key_hi_of(i, kv_len, delta);
    };
    auto key_lo = [&](int i) __attribute__((always_inline)) -> int { return key_lo_of(i, delta); };

    const int row0 = mblock * BM;
    const int row_last = min(rows_b, row0 + BM) - 1;
    const int wg_end = min(kend, key_hi(row_last / p.G) + 1);
    // the first tile (on the kbeg + n BN grid) that holds a key this
    // workgroup's rows may see
    const int wg_begin = max(kbeg, key_lo(row0 / p.G));
    const int tile_begin = wg_begin >= wg_end ? wg_end : kbeg + (wg_begin - kbeg) / BN * BN;

    const int wrow0 = row0 + (SPLIT_ROLES ? 0 : wave * kRowsPerWave);
    const bool wave_active = (!SPLIT_ROLES || wave < NCOMP) && wrow0 < rows_b;
    // the KV head this wave's rows read (paired: kvh + the computing wave's
    // index; loading waves keep kvh, whose Q they load but never use)
    const int hw = kvh + ((PAIR && wave_u < NCOMP) ? wave_u : 0);
    const int wrow_last = min(rows_b, wrow0 + kRowsPerWave) - 1;
    // keys in [wave_full_begin, wave_full_end) are visible to every row of
    // this wave (mask aside); keys outside [wave_begin, wave_end) to none
    const int wave_end = !wave_active ? kbeg : min(kend, key_hi(wrow_last / p.G) + 1);
    const int wave_full_end = !wave_active ? kbeg : min(kend, key_hi(wrow0 / p.G) + 1);
    const int wave_begin = key_lo(wrow0 / p.G);
    const int wave_full_begin = key_lo(wrow_last / p.G);
    // does this wave compute on the tile starting at key t?
    auto sees = [&](int t) __attribute__((always_inline)) -> bool {
        return wave_active && t < wave_end && t + BN > wave_begin;
    };
    auto full_tile = [&](int t) __attribute__((always_inline)) -> bool {
        return t + BN <= wave_full_end && t >= wave_full_begin;
    };

    // ---- this lane's query row (the column it holds in every MFMA tile)
    const int my_row = wrow0 + l32;
    const bool row_ok = my_row < rows_b;
    const int my_i = my_row / p.G;
    const int my_gh = my_row - my_i * p.G;
    my_last = !row_ok ? -1 : key_hi(my_i);
    my_first = key_lo(my_i);
    begin_rows(p.q + ((q_row0 + my_i) * p.Hq + (int64_t)hw * p.G + my_gh) * D, row_ok);

    // ---- key padding mask: one bit per key of a tile, wave-uniform
    const uint8_t *mrow = has_mask ? p.mask + (int64_t)b * p.Skv : nullptr;
    constexpr uint64_t kLoMask = BN >= 64 ? ~0ull : ((1ull << (BN & 63)) - 1);
    auto tile_bits = [&](int j0, uint64_t &lo, uint64_t &hi) __attribute__((always_inline)) {
        const int j = j0 + lane;
        const bool keep0 = (lane < BN) && j < kv_len && mrow[j] != 0;
        lo = __ballot(keep0) & kLoMask;
        hi = 0;
        if (BN > 64) {
            const bool keep1 = j + 64 < kv_len && mrow[j + 64] != 0;
            hi = __ballot(keep1);
        }
    };
    // Tile summary of the mask, taken once: bit n of mask_any (mask_all) is set
    // when tile tile_begin + n BN holds a kept key (only kept keys), for the
    // first 64 tiles of this workgroup's range -- lane n reads tile n's bytes.
    // Inside that window the steps then need no mask load for tiles that are
    // fully kept or fully masked; past it (or for a partly kept tile) they
    // read the tile's bytes.
    uint64_t mask_any = 0, mask_all = 0;
    if (has_mask) {
        // one pass covers 1 KB of keys (16 per lane) = 1024 / BN tiles of
        // BN / 16 lanes each; bytes past the keys or past wg_end count as
        // masked.  Rows that are not 16-byte aligned are read bytewise.
        constexpr int TPP = 1024 / BN;
        constexpr int LPT = BN / 16;
        constexpr uint64_t kLaneGroup = LPT >= 64 ? ~0ull : ((1ull << LPT) - 1);
        const bool vec = (((uintptr_t)mrow) & 15) == 0;
        const int lim = min(kv_len, wg_end);
#pragma unroll 1
        for (int pass = 0; pass < 64 / TPP; ++pass) {
            const int j = tile_begin + pass * 1024 + 16 * lane;
            bool any = false, all = false;
            if (j < lim) {
                uint32_t w[4] = {0u, 0u, 0u, 0u};
                if (vec && j + 16 <= lim) {
                    const u32x4 x = *(const u32x4 *)(mrow + j);
                    w[0] = x[0]; w[1] = x[1]; w[2] = x[2]; w[3] = x[3];
                } else {
                    for (int i = 0; i < 16; ++i)
                        if (j + i < lim && mrow[j + i] != 0) w[i >> 2] |= 0xffu << (8 * (i & 3));
                }
                // a byte is kept when nonzero: fold each byte to its top bit
                uint32_t nz_any = 0u, nz_all = 0x80808080u;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t t = ((w[q] & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w[q];
                    nz_any |= t & 0x80808080u;
                    nz_all &= t;
                }
                any = nz_any != 0u;
                all = (nz_all & 0x80808080u) == 0x80808080u && j + 16 <= lim;
            }
            const uint64_t ba = __ballot(any), bb = __ballot(all);
#pragma unroll
            for (int t = 0; t < TPP; ++t) {
                const uint64_t ga = (ba >> (t * LPT)) & kLaneGroup;
                const uint64_t gb = (bb >> (t * LPT)) & kLaneGroup;
                mask_any |= (uint64_t)(ga != 0) << (pass * TPP + t);
                mask_all |= (uint64_t)(gb == kLaneGroup) << (pass * TPP + t);
            }
        }
    }
    const int mask_window_end = tile_begin + 64 * BN;  // first tile the summary does not cover
    // first tile start >= j that holds a kept key (or wg_end), with its mask bits
    auto find_tile = [&](int j, uint64_t &lo, uint64_t &hi) __attribute__((always_inline)) -> int {
        if (!has_mask) return j;
        if (j < mask_window_end) {
            const uint64_t rest = mask_any >> ((j - tile_begin) / BN);
            if (rest == 0) {
                j = mask_window_end;
            } else {
                j += __builtin_ctzll(rest) * BN;
                if (j >= wg_end) return wg_end;
                if ((mask_all >> ((j - tile_begin) / BN)) & 1) {
                    lo = kLoMask;
                    hi = ~0ull;
                } else {
                    tile_bits(j, lo, hi);
                }
                return j;
            }
        }
        for (; j < wg_end; j += BN) {
            tile_bits(j, lo, hi);
            if (lo | hi) return j;
        }
        return wg_end;
    };

    const int64_t head_off = (int64_t)kvh * D + (PAGED ? 0 : seq_kv_row0(sd, b) * hstride);
    const_i32 *bt_row =
        PAGED ? (const_i32 *)(p.block_table + (int64_t)b * p.max_pages) : nullptr;
    // first tile holding a visible key (wg_end if none), with its mask bits
    uint64_t first_lo = ~0ull, first_hi = ~0ull;
    const int first_tile = find_tile(tile_begin, first_lo, first_hi);
    // Block-table entry of the page holding tile j (of the first tile for a
    // tile past the range).  With whole-tile pages the schedules read it a
    // step before the tile's loads are issued, so that the scalar load's
    // latency stays off the issue path.
    auto tile_page = [&](int j) __attribute__((always_inline)) -> int32_t {
        if constexpr (KVP == kPagedTile)
            return bt_row[(j < wg_end ? j : first_tile) >> p.page_shift];
        else
            return 0;
    };
    // Loads of tile j0 into stage dst; `phys` is tile_page(j0).
    auto issue = [&](int j0, int32_t phys, const uint16_t *src, uint8_t *dst) __attribute__((always_inline)) {
        // A tile past the range keeps the ring's load count but fetches almost
        // nothing: every lane reads the same 16 bytes of the first tile.
        const bool pad = j0 >= wg_end;
        const int keep = pad ? 0 : -1;  // lane offsets are and-ed with this (no branch)
        if (pad) j0 = first_tile;
        if constexpr (tile_in_page) {
            int64_t row = j0;
            if constexpr (PAGED) row = cache_row(phys, j0);
            const uint16_t *base = src + head_off + row * hstride;
            const int last = kv_len - 1 - j0;  // last valid key row of the tile
#pragma unroll
            for (int e = 0; e < PPW; ++e)
                buffer_load_lds16<LOAD_POLICY>(base, BN * row_bytes,
                                               (lds_void *)(dst + (e * LOADERS + loader) * 1024),
                                               (min(l_key[e], last) * row_bytes + l_chunk[e]) & keep);
        } else {
            // pages smaller than a tile: each of the tile's pages (at most
            // BN / 16) is looked up once -- all reads issued before any is
            // waited for -- and each piece picks its own
            constexpr int kTilePages = BN / 16;
            const int pg0 = j0 >> p.page_shift;
            const int pg_last = (kv_len - 1) >> p.page_shift;
            int32_t phys[kTilePages];
#pragma unroll
            for (int q = 0; q < kTilePages; ++q) phys[q] = bt_row[min(pg0 + q, pg_last)];
#pragma unroll
            for (int e = 0; e < PPW; ++e) {
                const int jr = min(j0 + (e * LOADERS + loader) * RPP, kv_len - 1);
                const int qi = (jr >> p.page_shift) - pg0;
                int32_t pe = phys[0];
#pragma unroll
                for (int q = 1; q < kTilePages; ++q) pe = qi == q ? phys[q] : pe;
                buffer_load_lds16<LOAD_POLICY>(
                    src + head_off + cache_row(pe, jr) * hstride, RPP * row_bytes,
                    (lds_void *)(dst + (e * LOADERS + loader) * 1024),
                    (min(l_dr, kv_len - 1 - jr) * row_bytes + l_chunk[e]) & keep);
            }
        }
    };
    // K of tile kt and V of tile vt (page entries pk and pv_)
    auto issue_kv = [&](int kt, int32_t pk, uint8_t *dk, int vt, int32_t pv_, uint8_t *dv) __attribute__((always_inline)) {
        if (!loads) return;
        issue(kt, pk, p.k, dk);
        issue(vt, pv_, p.v, dv);
    };

    if constexpr (WAVES == 8) {
        // ---- ping-pong main loop.  Waves 0-3 (group 0) and 4-7 (group 1)
        // sit on the four SIMDs in pairs.  Each tile k takes one step of two
        // phases, each ending in a workgroup barrier:
        //   phase A: group 0 runs its MFMA phase (QK^T of tile k, P.V of
        //            tile k-1); group 1 its softmax of tile k-1;
        //   phase B: group 0 runs the softmax of tile k; group 1 its MFMA
        //            phase (QK^T of tile k, P.V of tile k-1).
        // A wave's scores go from its MFMA phase to its next softmax phase,
        // its probabilities from there to its next MFMA phase.
        //
        // K and V have rings of three stages (96 KB of LDS at D = 128, one
        // workgroup per CU).  Step k reads K(k) and V(k-1) and issues the
        // loads of K(k+2) and V(k+1) into the stages step k-1 freed, so a load
        // has two steps to land.  (Four stages, loads three steps ahead,
        // measured 3.5 % slower, the same bits.)  Every step issues the same
        // number of loads (pad loads for tiles past the range), so one counted
        // wait -- all but the youngest step's loads -- orders the ring.
        static_assert(PPW == 1 || PPW == 2, "counted waits below assume 1 or 2 loads per tile");

        const int group = wave >> 2;
        f32x16 sc[NT];
        vec8 pb[PSTEPS];
        float corr_pending = 1.f;
        // The wave in its MFMA phase issues at raised priority, so that the
        // matrix core is fed first and the other wave's softmax fills the
        // remaining issue cycles (measured 293 -> 289 us on the causal GQA
        // prefill).
        auto mma_phase = [&](int cur, int prev, const uint8_t *sk, const uint8_t *sv) __attribute__((always_inline)) {
            __builtin_amdgcn_s_setprio(1);
            const bool do_qk = sees(cur);
            const bool do_pv = prev >= 0 && sees(prev);
            if (do_pv && corr_pending != 1.f) {
#pragma unroll
                for (int t = 0; t < DT; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[t][r] *= corr_pending;
            }
            if (do_qk && do_pv) {
                qk(sk, sc);
                pv(sv, pb);
                sched_read_ahead<NT * KSTEPS + 2 * DT * PSTEPS, NT * KSTEPS + DT * PSTEPS>();
            } else if (do_qk) {
                qk(sk, sc);
                sched_read_ahead<NT * KSTEPS, NT * KSTEPS>();
            } else if (do_pv) {
                pv(sv, pb);
                sched_read_ahead<2 * DT * PSTEPS, DT * PSTEPS>();
            }
            __builtin_amdgcn_s_setprio(0);
        };
        auto softmax_phase = [&](int tile, uint64_t lo, uint64_t hi) __attribute__((always_inline)) {
            if (!(tile >= 0 && sees(tile))) return;
            bool full = full_tile(tile);
            if (has_mask) full = full && (lo == kLoMask) && (BN <= 64 || hi == ~0ull);
            if (full)
                corr_pending = softmax(std::false_type{}, tile, lo, hi, sc, pb);
            else
                corr_pending = softmax(std::true_type{}, tile, lo, hi, sc, pb);
        };

        // upcoming tiles t0 (current), t1, t2 with their mask bits; tiles
        // past the workgroup's range read as wg_end
        uint64_t lo0 = ~0ull, hi0 = ~0ull, lo1 = ~0ull, hi1 = ~0ull, lo2 = ~0ull, hi2 = ~0ull,
                 plo = ~0ull, phi = ~0ull;
        int t0 = first_tile;
        lo0 = first_lo;
        hi0 = first_hi;
        int t1 = t0 < wg_end ? find_tile(t0 + BN, lo1, hi1) : wg_end;
        int t2 = wg_end;
        int prev = -1;
        const bool any_tile = t0 < wg_end;
        int32_t pg_next = 0, pg_t1 = 0;  // page entries of the next K tile and of t1
        // one step: K(t0) in K_CUR, V(prev) in V_PREV; K(t2) -> K_NEW, V(t1) -> V_NEW.
        // The step with t0 == wg_end only finishes P.V of the last tile; steps
        // after it find no visible tile and issue pad loads.  (A macro, expanded
        // in the loop below: the step holds the workgroup barriers, which the
        // compiler mishandled inside a lambda -- it deleted the computation.)
#define MIATTN_PP_STEP(K_CUR, V_PREV, K_NEW, V_NEW)                                     \
        {                                                                               \
            t2 = t1 < wg_end ? find_tile(t1 + BN, lo2, hi2) : wg_end;                   \
            issue_kv(t2, pg_next, K_NEW, t1, pg_t1, V_NEW);                             \
            pg_t1 = pg_next;                                                            \
            if (group == 0) /* phase A */                                               \
                mma_phase(t0, prev, K_CUR, V_PREV);                                     \
            else                                                                        \
                softmax_phase(prev, plo, phi);                                          \
            ring_barrier();                                                             \
            if (group == 0) /* phase B */                                               \
                softmax_phase(t0 < wg_end ? t0 : -1, lo0, hi0);                         \
            else                                                                        \
                mma_phase(t0, prev, K_CUR, V_PREV);                                     \
            /* (the next page entry is read here: a scalar load in flight during */    \
            /* the phases would force every LDS wait there to lgkmcnt(0)) */            \
            pg_next = tile_page(t2 + BN);                                               \
            /* the loads issued a step ago hold K(t1) and V(t0) */                      \
            wait_vmcnt<2 * PPW>();                                                      \
            ring_barrier();                                                             \
            prev = t0; plo = lo0; phi = hi0;                                            \
            t0 = t1; lo0 = lo1; hi0 = hi1;                                              \
            t1 = t2; lo1 = lo2; hi1 = hi2;                                              \
        }

        // A workgroup without a visible tile skips the ring altogether.  Inside
        // it every step issues its loads unconditionally: the compiler tracks
        // which LDS array each direct load writes, and a load that might not
        // have been issued would make it wait for all of them before each read.
        if (any_tile) {
            // prologue: steps -2, -1 of loads (K(t0) with a pad V; K(t1),
            // V(t0)), then wait for the first
            {
                const int32_t g0 = tile_page(t0), g1 = tile_page(t1);
                issue_kv(t0, g0, sK0, wg_end, g0, sV2);
                issue_kv(t1, g1, sK1, t0, g0, sV0);
                pg_t1 = g1;
                pg_next = tile_page(t1 + BN);
            }
            wait_vmcnt<2 * PPW>();
            ring_barrier();
            // The shared arrays are named only here, in the kernel body, and
            // handed to the helpers as pointers.  The loop leaves only after a
            // whole round of three steps: an exit between steps makes the
            // compiler merge the ring states of all three into the loop header
            // and wait for every load there.
            do {
                MIATTN_PP_STEP(sK0, sV2, sK2, sV1)  // k % 3 == 0
                MIATTN_PP_STEP(sK1, sV0, sK0, sV2)  // k % 3 == 1
                MIATTN_PP_STEP(sK2, sV1, sK1, sV0)  // k % 3 == 2
            } while (prev < wg_end);
            // no load may still be writing this workgroup's LDS when it exits
            wait_vmcnt<0>();
        }
#undef MIATTN_PP_STEP
    } else {
        // ---- streaming loop (decode-shaped calls and D = 256).  Each step
        // computes one tile (QK^T, softmax, P.V) from LDS while the loads of
        // the tile three steps ahead land in the stage the previous step
        // freed; the same counted wait as above (all but the two youngest
        // steps' loads) and one barrier per step order the ring.
        // ring depth: three stages for the decode workgroups and the D = 64
        // prefill (24 KB of LDS: 77 -> 70 us on the key-padding MHA against
        // four stages), four otherwise
        constexpr int kStages = (SPLIT_ROLES || (WAVES == 4 && D == 64)) ? 3 : 4;
        f32x16 sc[NT];
        vec8 pb[PSTEPS];
        uint64_t lo0 = first_lo, hi0 = first_hi, lo1 = ~0ull, hi1 = ~0ull, lo2 = ~0ull,
                 hi2 = ~0ull, lo3 = ~0ull, hi3 = ~0ull;
        int t0 = first_tile;
        int t1 = t0 < wg_end ? find_tile(t0 + BN, lo1, hi1) : wg_end;
        int t2 = (kStages == 4 && t1 < wg_end) ? find_tile(t1 + BN, lo2, hi2) : wg_end;
        int t3 = wg_end;
        int32_t pg_next = 0;  // page entry of the next tile to load
        auto compute = [&](const uint8_t *sk, const uint8_t *sv) __attribute__((always_inline)) {
            if (!sees(t0)) return;
            bool full = full_tile(t0);
            if (has_mask) full = full && (lo0 == kLoMask) && (BN <= 64 || hi0 == ~0ull);
            qk_batched(sk, sc);
            const float corr = full ? softmax(std::false_type{}, t0, lo0, hi0, sc, pb)
                                    : softmax(std::true_type{}, t0, lo0, hi0, sc, pb);
            if (corr != 1.f) {
#pragma unroll
                for (int t = 0; t < DT; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[t][r] *= corr;
            }
            pv_batched(sv, pb);
        };
        if constexpr (FP8) {
        // ---- FP8 pools.  Wave 1 moves E4M3FN key and value tiles HBM -> LDS
        // with direct loads into an S8-stage FP8 ring; waves 2 and 3 convert
        // each landed tile, half of its pieces each, into the 16-bit MFMA type,
        // written to one of two 16-bit stages in the swizzled layout of the
        // 16-bit tiles, so wave 0 runs the 16-bit path unchanged.  (With one
        // converting wave the conversion set the pace: 130 us per decode
        // launch against 114 with two, the same bits.)  The roles stay apart: no wave reads LDS
        // while direct loads of its own are in flight (the compiler would
        // make it wait for all of them), so the stages need not be separate
        // arrays.  Step n: wave 0 computes tile n from 16-bit stage n & 1;
        // waves 2, 3 convert tile n + 1 (landed during step n - 1); wave 1 issues
        // tile n + S8 into the FP8 stage tile n left, then waits for tile
        // n + 2 -- S8 - 2 tiles stay in flight.  (Tiles of a paged call
        // follow one another: there is no padding mask.)  Paired (two
        // adjacent KV heads, 2 D-byte FP8 segments per key): waves 0 and 1
        // compute, wave 2 loads and waves 3-6 convert, a quarter each (FP8
        // decode kernel 104.5 -> 102 us; with two converting waves 117 us).
        //
        // A piece (1 KB) holds, at lane l's 16 bytes, the 16-byte chunk f_chunk
        // (16 d-values) of key row piece_row(e) + f_row -- an order chosen for
        // the conversion's 16-bit writes: a 16-byte LDS write is served eight
        // lanes at a time, and those eight must fall in one 128-byte half of
        // the 256-byte bank line, on distinct banks, or the write takes twice
        // as long (measured: every lane order that spreads eight lanes over
        // both halves doubles the write's LDS cycles, as SQ_LDS_BANK_CONFLICT
        // cycles).  Lanes 8k..8k+7 therefore hold rows r and r + 8 -- whose
        // swizzles put their chunks in the same half and apart in bank -- and
        // four chunks of each.  A piece's rows lie in one aligned 16-row block.
        constexpr int S8 = 4;                // FP8 ring stages
        constexpr int U16 = DL / 16;         // 16-byte chunks per FP8 key row
        constexpr int CG = U16 / 4;          // groups of four chunks per row
        constexpr int STAGE8 = BN * DL;      // bytes of one FP8 K (or V) tile
        constexpr int PC8 = STAGE8 / 1024;   // pieces per tensor and tile
        constexpr int NCONV = PAIR ? 4 : 2;  // converting waves
        static_assert(PC8 % NCONV == 0, "whole pieces per converting wave");
        static_assert(CG == 1 || CG == 2 || CG == 4, "FP8 pools: 64, 128 or 256 values per key row");
        static_assert((S8 - 2) * 2 * PC8 <= 63, "the counted wait fits vmcnt");
        __shared__ __attribute__((aligned(1024))) uint8_t fK[S8][STAGE8];
        __shared__ __attribute__((aligned(1024))) uint8_t fV[S8][STAGE8];
        const uint8_t *k8 = (const uint8_t *)p.k, *v8 = (const uint8_t *)p.v;
        const int row8 = p.Hkv * D;  // bytes between consecutive keys
        const int f_g = lane >> 3, f_i = lane & 7;
        const int f_row = f_g / CG + 8 * (f_i >> 2);     // row within the piece's rows
        const int f_chunk = 4 * (f_g % CG) + (f_i & 3);  // 16-byte chunk within the row
        // first row of piece e's rows (within the tile), and of its 16-row block
        auto piece_row = [](int e) { return 16 * (e / CG) + (8 / CG) * (e % CG); };
        auto piece_block = [](int e) { return 16 * (e / CG); };
        // (roles: the NCOMP computing waves, then the loading wave, then
        // the two converting waves)
        const bool dma = wave_u == NCOMP, conv = wave_u > NCOMP;
        auto issue8 = [&](int j0, int stage) __attribute__((always_inline)) {
            if (!dma) return;
            uint8_t *dk = fK[stage], *dv = fV[stage];
            // a tile past the range keeps the load count, every lane reading
            // the first tile's first 16 bytes
            const bool pad = j0 >= wg_end;
            const int keep = pad ? 0 : -1;
            if (pad) j0 = first_tile;
            const int last = kv_len - 1 - j0;  // last valid key row of the tile
            if constexpr (KVP == kPagedTile) {
                const int64_t off =
                    cache_row(bt_row[j0 >> p.page_shift], j0) * row8 + (int64_t)kvh * D;
#pragma unroll
                for (int e = 0; e < PC8; ++e) {
                    const int vo = (min(piece_row(e) + f_row, last) * row8 + 16 * f_chunk) & keep;
                    buffer_load_lds16<LOAD_POLICY>(k8 + off, BN * row8, (lds_void *)(dk + e * 1024), vo);
                    buffer_load_lds16<LOAD_POLICY>(v8 + off, BN * row8, (lds_void *)(dv + e * 1024), vo);
                }
            } else {
                // pages smaller than a tile (16 keys or more): a piece's 16-row
                // block lies in one page
#pragma unroll
                for (int e = 0; e < PC8; ++e) {
                    const int jr = min(j0 + piece_block(e), kv_len - 1);
                    const int64_t off =
                        cache_row(bt_row[jr >> p.page_shift], jr) * row8 + (int64_t)kvh * D;
                    const int in_block = piece_row(e) - piece_block(e) + f_row;
                    const int vo = (min(in_block, kv_len - 1 - jr) * row8 + 16 * f_chunk) & keep;
                    buffer_load_lds16<LOAD_POLICY>(k8 + off, 16 * row8, (lds_void *)(dk + e * 1024), vo);
                    buffer_load_lds16<LOAD_POLICY>(v8 + off, 16 * row8, (lds_void *)(dv + e * 1024), vo);
                }
            }
        };
        // FP8 stage -> 16-bit stage: lane l's 16 bytes of piece e become the
        // 16-bit chunks 2 f_chunk and 2 f_chunk + 1 of key row piece_row(e) +
        // f_row, written to their swizzled positions.
        auto convert8 = [&](int stage, uint8_t *dk, uint8_t *dv) __attribute__((always_inline)) {
            if (!conv) return;
            const uint8_t *fk = fK[stage], *fv = fV[stage];
            const int cw = wave_u - NCOMP - 1;  // this converting wave's share of the pieces
#pragma unroll
            for (int e2 = 0; e2 < PC8 / NCONV; ++e2) {
                const int e = cw * (PC8 / NCONV) + e2;
                const u32x4 kw = *(const u32x4 *)(fk + e * 1024 + 16 * lane);
                const u32x4 vw = *(const u32x4 *)(fv + e * 1024 + 16 * lane);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const u32x2 k01 = fp8x4_to_half4<BF16>(h ? kw[2] : kw[0]);
                    const u32x2 k23 = fp8x4_to_half4<BF16>(h ? kw[3] : kw[1]);
                    const u32x2 v01 = fp8x4_to_half4<BF16>(h ? vw[2] : vw[0]);
                    const u32x2 v23 = fp8x4_to_half4<BF16>(h ? vw[3] : vw[1]);
                    const int at = tile_off<DL>(piece_row(e) + f_row, 2 * f_chunk + h);
                    *(u32x4 *)(dk + at) = u32x4{k01[0], k01[1], k23[0], k23[1]};
                    *(u32x4 *)(dv + at) = u32x4{v01[0], v01[1], v23[0], v23[1]};
                }
            }
        };
        if (first_tile < wg_end) {
#pragma unroll
            for (int st = 0; st < S8; ++st) issue8(first_tile + st * BN, st);
            wait_vmcnt<(S8 - 2) * 2 * PC8>();  // tiles 0 and 1
            ring_barrier();
            convert8(0, sK0, sV0);
            ring_barrier();
            int st_new = 0, st_nxt = 1;  // FP8 stages of tiles n (refilled) and n + 1
            for (int n = 0; first_tile + n * BN < wg_end; ++n) {
                t0 = first_tile + n * BN;
                issue8(t0 + S8 * BN, st_new);
                const bool odd = n & 1;
                compute(odd ? sK1 : sK0, odd ? sV1 : sV0);
                convert8(st_nxt, odd ? sK0 : sK1, odd ? sV0 : sV1);
                // tile n + 2 has landed when only the S8 - 2 younger tiles' loads remain
                wait_vmcnt<(S8 - 2) * 2 * PC8>();
                ring_barrier();
                st_new = st_nxt;
                st_nxt = st_nxt + 1 == S8 ? 0 : st_nxt + 1;
            }
            wait_vmcnt<0>();
        }
        } else {
#define MIATTN_ST_STEP(K_CUR, V_CUR, K_NEW, V_NEW)                                      \
        {                                                                               \
            t3 = t2 < wg_end ? find_tile(t2 + BN, lo3, hi3) : wg_end;                   \
            issue_kv(t3, pg_next, K_NEW, t3, pg_next, V_NEW);                           \
            compute(K_CUR, V_CUR);                                                      \
            pg_next = tile_page(t3 + BN);                                               \
            /* the loads issued two steps ago hold tile t1 */                          \
            wait_vmcnt<4 * PPW>();                                                      \
            ring_barrier();                                                             \
            t0 = t1; lo0 = lo1; hi0 = hi1;                                              \
            t1 = t2; lo1 = lo2; hi1 = hi2;                                              \
            t2 = t3; lo2 = lo3; hi2 = hi3;                                              \
        }
        if (t0 < wg_end && kStages == 4) {
            {
                const int32_t g0 = tile_page(t0), g1 = tile_page(t1), g2 = tile_page(t2);
                issue_kv(t0, g0, sK0, t0, g0, sV0);
                issue_kv(t1, g1, sK1, t1, g1, sV1);
                issue_kv(t2, g2, sK2, t2, g2, sV2);
                pg_next = tile_page(t2 + BN);
            }
            wait_vmcnt<4 * PPW>();
            ring_barrier();
            do {
                MIATTN_ST_STEP(sK0, sV0, sK3, sV3)
                MIATTN_ST_STEP(sK1, sV1, sK0, sV0)
                MIATTN_ST_STEP(sK2, sV2, sK1, sV1)
                MIATTN_ST_STEP(sK3, sV3, sK2, sV2)
            } while (t0 < wg_end);
            wait_vmcnt<0>();
        }
#undef MIATTN_ST_STEP
        // three stages (decode: 96 KB of LDS at D = 128, one workgroup per
        // CU): step k computes t0 while t2 loads; at its end the loads of the
        // previous step (tile t1) must have landed -- all but this step's.
#define MIATTN_ST3_STEP(K_CUR, V_CUR, K_NEW, V_NEW)                                     \
        {                                                                               \
            t2 = t1 < wg_end ? find_tile(t1 + BN, lo2, hi2) : wg_end;                   \
            issue_kv(t2, pg_next, K_NEW, t2, pg_next, V_NEW);                           \
            compute(K_CUR, V_CUR);                                                      \
            pg_next = tile_page(t2 + BN);                                               \
            wait_vmcnt<2 * PPW>();                                                      \
            ring_barrier();                                                             \
            t0 = t1; lo0 = lo1; hi0 = hi1;                                              \
            t1 = t2; lo1 = lo2; hi1 = hi2;                                              \
        }
        if (t0 < wg_end && kStages == 3) {
            {
                const int32_t g0 = tile_page(t0), g1 = tile_page(t1);
                issue_kv(t0, g0, sK0, t0, g0, sV0);
                issue_kv(t1, g1, sK1, t1, g1, sV1);
                pg_next = tile_page(t1 + BN);
            }
            wait_vmcnt<2 * PPW>();
            ring_barrier();
            do {
                MIATTN_ST3_STEP(sK0, sV0, sK2, sV2)
                MIATTN_ST3_STEP(sK1, sV1, sK0, sV0)
                MIATTN_ST3_STEP(sK2, sV2, sK1, sV1)
            } while (t0 < wg_end);
            wait_vmcnt<0>();
        }
#undef MIATTN_ST3_STEP
        }
    }

    // ---- epilogue: normalise and store (no barrier below this point)
    if (!wave_active) return;
    const float l_tot = sum_halves(l_run);
    if (!row_ok) return;
    // (only a row without a visible key has l = 0; a NaN score -- a NaN in q
    // or k -- makes l NaN, and the NaN goes on into o and lse)
    float inv = l_tot != 0.f ? 1.f / l_tot : 0.f;
    float lse_v = l_tot != 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    const int my_h = hw * p.G + my_gh;
    if (!partial && p.sinks != nullptr) {
        // The head's sink logit joins the denominator only, used as given
        // (TileOPs "Attention Operators", GQAVarlenFwdOp / GQAPagedFwdOp): a
        // row without visible keys stays zero with lse = sink, and a +inf
        // sink takes all the weight.  (A split result gets its sink in the
        // merge.)
        const float sk = p.sinks[my_h];
        if (l_tot == 0.f || sk == INFINITY) {
            inv = 0.f;
            lse_v = l_tot == 0.f ? sk : INFINITY;
        } else {
            const float s2 = sk * kLog2e;
            const float mx = fmaxf(m_run, s2);
            const float a = fast_exp2(m_run - mx);
            const float den = __builtin_fmaf(l_tot, a, fast_exp2(s2 - mx));
            inv = a / den;
            lse_v = (mx + __builtin_amdgcn_logf(den)) * kLn2;
        }
    }

    if constexpr (FP8) inv *= *p.v_scale;  // the value pool's scale multiplies the output

    if (!partial) {
        uint16_t *orow = p.o + ((q_row0 + my_i) * p.Hq + my_h) * D;
        // Registers 4w..4w+3 of block t hold d = 32t + 8w + 4 hl + 0..3.  The
        // two lanes of a row (hl = 0, 1) trade halves with v_permlane32_swap
        // so that each holds 8 consecutive values: lane hl stores d = 32t +
        // 8(w + hl) + 0..7 for w = 0, 2, a row's two lanes 32 contiguous
        // bytes -- half the store instructions, each writing 16 bytes per lane
        // (causal GQA prefill 274 -> 268 us; both lanes of a row are active or
        // neither).
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int w = 0; w < 4; w += 2) {
                auto pk = [&](int r) __attribute__((always_inline)) {
                    return pack_half2<BF16>(acc[t][r] * inv, acc[t][r + 1] * inv);
                };
                // (the swap trades lanes 32..63 of its first operand with lanes
                // 0..31 of its second)
                const auto lo = __builtin_amdgcn_permlane32_swap(pk(4 * w), pk(4 * w + 4), false, false);
                const auto hi =
                    __builtin_amdgcn_permlane32_swap(pk(4 * w + 2), pk(4 * w + 6), false, false);
                const u32x4 packed = {(uint32_t)lo[0], (uint32_t)hi[0], (uint32_t)lo[1],
                                      (uint32_t)hi[1]};
                // (streaming stores in the D = 64 four-wave schedule, four
                // workgroups per CU: key-padding MHA 70.5 -> 68.5 us; the
                // prefill schedules measured no change)
                u32x4 *const dst = (u32x4 *)(orow + 32 * t + 8 * (w + hl));
                if constexpr (WAVES == 4 && D == 64)
                    __builtin_nontemporal_store(packed, dst);
                else
                    *dst = packed;
            }
        if (p.lse != nullptr && hl == 0) {
            if (p.cu_q)  // packed: [Hq, total_q]
                p.lse[(int64_t)my_h * p.total_q + q_row0 + my_i] = lse_v;
            else         // [B, Hq, Sq]
                p.lse[((int64_t)b * p.Hq + my_h) * p.Sq + my_i] = lse_v;
        }
    } else {
        // (paired: head kvh + 1's slots follow head kvh's at a fixed stride)
        store_partial((slot + (hw - kvh) * slot_head_stride) * p.rows + my_row, inv, lse_v);
    }

    };

    // ---- which work this workgroup owns
    const int units = p.B * p.Hkv * p.n_splits;
    if constexpr (SPLIT_ROLES) {
        if (p.sk_grid > 0) {
            // Stream-K decode, by head: workgroup g serves head unit g % U (KV
            // head g % Hkv, or the pair 2 (g % U), 2 (g % U) + 1 when paired),
            // and the S = G / U workgroups of one unit cut its sequence of
            // (request) units -- plan weight T1, each unit its key tiles plus
            // the cost of starting a piece of it (sk_weight) -- into equal
            // shares: share c = g / U takes the weight [c T1 / S, (c+1) T1 / S)
            // whatever the lengths, and writes one partial per unit (and head)
            // whose tiles it touches, to slot h (B + S) + b + c for head h
            // (the merge kernel finds the slots the same way).  The U
            // workgroups g, g + 1, ... run side by side and read the same cache
            // rows.  A unit of weight w = piece + tiles holds its tiles at
            // weight offsets [piece, w).
            const int g = blockIdx.x;
            const SkBatch sb = {sd, BN, p.win_left, p.sk_piece};
            int unused;
            // head units: one KV head, or a pair of adjacent heads
            const int U = PAIR ? p.Hkv / 2 : p.Hkv;
            const int kvh = (g % U) * (PAIR ? 2 : 1), c = g / U, shares = p.sk_grid / U;
            slot_head_stride = p.B + shares;
            const int64_t T1 = sk_sums(sb, 0, unused);
            const int64_t s0 = (int64_t)c * T1 / shares;
            const int64_t s1 = (int64_t)(c + 1) * T1 / shares;
            if (s0 >= s1) return;
            int b, pre, wb;
            sk_find(sb, 1, s0, b, pre, wb);
            int off = (int)(s0 - pre);  // weight offset into request b
            for (int64_t at = s0; at < s1; ++b, off = 0) {
                const int len = seq_kv_len(sd, b);
                int64_t unused_row0;
                int sq_u;
                q_span(sd, b, unused_row0, sq_u);
                // (the unit's tiles start at the first one its window reaches)
                const int t_first = sk_first_tile(sb, len, sq_u);
                const int tiles = sk_tiles(sb, b);
                const int w = sk_weight(sb, tiles);
                // the share's part of the unit's tiles, as weight offsets
                const int lo = max(off, sb.piece);
                const int hi = (int)min((int64_t)w, off + (s1 - at));
                at += w - off;
                if (hi <= lo) continue;
                run(0, b, kvh, len, (t_first + lo - sb.piece) * BN,
                    min(len, (t_first + hi - sb.piece) * BN),
                    (int64_t)kvh * (p.B + shares) + b + c, true);
            }
            return;
        }
    }
    // (paired kernels are launched for stream-K plans only)
    if constexpr (PAIR) return;
    // Workgroups are dispatched round-robin over the 8 XCDs; when the unit
    // count allows, consecutive workgroups of one XCD share a (batch, KV head)
    // so its K/V stays in that XCD's L2.  Causal row blocks run heaviest first.
    int rank, unit;
    if (p.xcd_units > 0 && !p.causal) {
        // every row block weighs the same: each XCD runs its units one after
        // another (units u = xcd, xcd + 8, ... interleaved over the XCDs, so
        // that units of different lengths spread over all of them)
        const int s = blockIdx.x >> 3;
        unit = (blockIdx.x & 7) + 8 * (s / p.n_mblocks);
        rank = s % p.n_mblocks;
    } else if (p.xcd_units > 0) {
        // causal: heaviest row blocks first, the units of each XCD interleaved
        const int s = blockIdx.x >> 3;
        unit = (blockIdx.x & 7) * p.xcd_units + s % p.xcd_units;
        rank = s / p.xcd_units;
    } else {
        rank = blockIdx.x / units;
        unit = blockIdx.x - rank * units;
    }
    const int mblock = p.causal ? (p.n_mblocks - 1 - rank) : rank;
    // Units are (batch, KV head, split) with the split fastest, or -- with
    // heads_inner -- (batch, split, KV head) with the head fastest: the KV
    // heads of one position share the cache rows, so workgroups that run
    // together then read whole rows of the same pages.
    int b, kvh, split;
    if (p.heads_inner) {
        const int bs = unit / p.Hkv;
        kvh = unit - bs * p.Hkv;
        b = bs / p.n_splits;
        split = bs - b * p.n_splits;
    } else {
        const int bh_ = unit / p.n_splits;
        split = unit - bh_ * p.n_splits;
        b = bh_ / p.Hkv;
        kvh = bh_ - b * p.Hkv;
    }
    // (a paged length is clamped to the table's capacity, and an empty cache
    // holds no keys, so that malformed lengths cannot address memory
    // outside the table or the cache)
    const int kv_len = seq_kv_len(sd, b);
    const int kbeg = split * p.split_len;
    // Splits past the end are never read by the merge, which counts the
    // splits that hold keys from the same length.
    if (p.n_splits > 1 && kbeg >= kv_len) return;
    const int kend = min(kv_len, kbeg + p.split_len);
    run(mblock, b, kvh, kv_len, kbeg, kend, (int64_t)(b * p.Hkv + kvh) * p.n_splits + split,
        p.n_splits > 1);
}

template <int D, bool BF16, int KV, int WAVES, bool CAP>
hipError_t launch_one(const FwdParams &p, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((attn_fwd_kernel<D, BF16, KV, WAVES, CAP>), dim3(grid), dim3(64 * group_waves<WAVES, KV>()),
                       0, stream, p);
    return hipGetLastError();
}

template <int D, bool BF16, int KV, int WAVES, bool CAP>
int blocks_per_cu() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, attn_fwd_kernel<D, BF16, KV, WAVES, CAP>, 64 * group_waves<WAVES, KV>(), 0) != hipSuccess)
        return 0;
    return n;
}

template <int D, int W, bool CAP>
int decode_blocks(const FwdParams &p, bool bf16, bool paged) {
    const bool tile =
        p.page_shift >= __builtin_ctz(keys_per_tile(D, W, paged && p.k_scale != nullptr));
    if constexpr (W == 3 || W == kPairWaves) {
        if (paged && p.k_scale != nullptr) {
            if (tile)
                return bf16 ? blocks_per_cu<D, true, kPagedTile8, W, CAP>()
                            : blocks_per_cu<D, false, kPagedTile8, W, CAP>();
            return bf16 ? blocks_per_cu<D, true, kPagedPiece8, W, CAP>()
                        : blocks_per_cu<D, false, kPagedPiece8, W, CAP>();
        }
    }
    if (p.k_scale != nullptr) return 0;  // FP8 pools: the decode schedules only
    if (!paged)
        return bf16 ? blocks_per_cu<D, true, kDense, W, CAP>()
                    : blocks_per_cu<D, false, kDense, W, CAP>();
    if (tile)
        return bf16 ? blocks_per_cu<D, true, kPagedTile, W, CAP>()
                    : blocks_per_cu<D, false, kPagedTile, W, CAP>();
    return bf16 ? blocks_per_cu<D, true, kPagedPiece, W, CAP>()
                : blocks_per_cu<D, false, kPagedPiece, W, CAP>();
}

template <int D, int WAVES, int KV, bool CAP>
hipError_t launch_kv(const FwdParams &p, bool bf16, int grid, hipStream_t stream) {
    return bf16 ? launch_one<D, true, KV, WAVES, CAP>(p, grid, stream)
                : launch_one<D, false, KV, WAVES, CAP>(p, grid, stream);
}

template <int D, int WAVES, bool CAP>
hipError_t launch_w(const FwdParams &p, bool bf16, bool paged, int grid, hipStream_t stream) {
    const bool tile =
        p.page_shift >= __builtin_ctz(keys_per_tile(D, WAVES, paged && p.k_scale != nullptr));
    if constexpr (WAVES == 3 || WAVES == kPairWaves) {
        if (paged && p.k_scale != nullptr)
            return tile ? launch_kv<D, WAVES, kPagedTile8, CAP>(p, bf16, grid, stream)
                        : launch_kv<D, WAVES, kPagedPiece8, CAP>(p, bf16, grid, stream);
    }
    if (p.k_scale != nullptr) return hipErrorInvalidValue;  // FP8 pools: the decode schedules only
    if (!paged) return launch_kv<D, WAVES, kDense, CAP>(p, bf16, grid, stream);
    if (tile)
        return launch_kv<D, WAVES, kPagedTile, CAP>(p, bf16, grid, stream);
    return launch_kv<D, WAVES, kPagedPiece, CAP>(p, bf16, grid, stream);
}

}  // namespace

// Schedules per head dimension: D <= 128 has the 8-wave prefill schedule, the
// 3-wave decode schedule and the paired decode schedule, D = 64 also the
// 4-wave streaming schedule for dense prefill; D = 256 the 4-wave streaming
// schedule.
template <int D, bool CAP>
hipError_t launch_attn_fwd_dc(const FwdParams &p, bool bf16, bool paged, int waves, int grid,
                              hipStream_t stream) {
    if constexpr (D == 256) {
        if (waves == 4) return launch_w<256, 4, CAP>(p, bf16, paged, grid, stream);
    } else {
        if constexpr (D == 64)
            if (waves == 4 && !paged) return launch_kv<D, 4, kDense, CAP>(p, bf16, grid, stream);
        if (waves == 8) return launch_w<D, 8, CAP>(p, bf16, paged, grid, stream);
        if (waves == 3) return launch_w<D, 3, CAP>(p, bf16, paged, grid, stream);
        if (waves == kPairWaves) return launch_w<D, kPairWaves, CAP>(p, bf16, paged, grid, stream);
    }
    return hipErrorInvalidValue;
}

template <int D, bool CAP>
int decode_blocks_per_cu_dc(const FwdParams &p, bool bf16, bool paged, int waves) {
    if constexpr (D <= 128) {
        if (waves == 3) return decode_blocks<D, 3, CAP>(p, bf16, paged);
        if (waves == kPairWaves) return decode_blocks<D, kPairWaves, CAP>(p, bf16, paged);
    }
    return 0;
}

// This translation unit holds the kernels of one (D, CAP) pair, chosen by the
// build (-DMIATTN_KD=64|128|256 -DMIATTN_KCAP=0|1).
#if !defined(MIATTN_KD) || !defined(MIATTN_KCAP)
#error "build attn_fwd.hip with -DMIATTN_KD=<head dim> -DMIATTN_KCAP=<0|1>"
#endif
template hipError_t launch_attn_fwd_dc<MIATTN_KD, (MIATTN_KCAP != 0)>(const FwdParams &, bool,
                                                                       bool, int, int,
                                                                       hipStream_t);
template int decode_blocks_per_cu_dc<MIATTN_KD, (MIATTN_KCAP != 0)>(const FwdParams &, bool,
                                                                     bool, int);

}  // namespace miattn
