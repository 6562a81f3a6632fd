// lse_merge.hip -- combine split-KV partial results by their log-sum-exps.
//
// Each split s of a row's key range produced a normalised partial output o_s
// (FP32) and its natural-log LSE lse_s (-inf when the split holds no visible
// key for that row).  The whole-range result is
//     lse = M + ln sum_s exp(lse_s - M),  M = max_s lse_s,
//     o   = sum_s exp(lse_s - lse) o_s,
// computed in FP32 without recomputing QK or PV (the split-KV merge of MATE
// "QSA", Core Attention).  A row whose every split is empty gets o = 0 and
// lse = -inf (TileOPs "Attention Operators", MHADecodePagedWithKVCacheFwdOp:
// a query that sees no key outputs zeros; MATE "QSA": empty -> -inf LSE).
// A head's sink logit, when given, joins the merged denominator once
// (GQAVarlenFwdOp / GQAPagedFwdOp: denominator only, used as given).
//
// One wave per packed row, reading partial rows with 16-byte loads.
#include "attn_kernels.h"

#include "attn_device.h"

namespace miattn {
namespace {

using namespace dev;

template <bool BF16>
__device__ __forceinline__ uint16_t to_half_bits(float x) {
    if constexpr (BF16)
        return __builtin_bit_cast(uint16_t, (__bf16)x);
    else
        return __builtin_bit_cast(uint16_t, (_Float16)x);
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void lse_merge_kernel(const MergeParams p) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t gr = (int64_t)blockIdx.x * 4 + wave;
    const int64_t total = (int64_t)p.B * p.Hkv * p.rows;
    if (gr >= total) return;
    const int bh = (int)(gr / p.rows);
    const int r = (int)(gr - (int64_t)bh * p.rows);
    const int b = bh / p.Hkv;
    const int kvh = bh - b * p.Hkv;
    const int i = r / p.G;
    const int gh = r - i * p.G;
    // the same request extents as the attention kernel
    const SeqDesc sd = {p.seqlen, p.cu_q, p.cu_kv, p.B, p.Sq, p.Skv, p.total_q, p.total_kv,
                        p.sk_cap, p.seqlen ? p.kv_append : 0};
    int64_t q_row0;
    int sq_b;
    q_span(sd, b, q_row0, sq_b);
    if (r >= sq_b * p.G) return;  // a shorter request: no such row

    // The partial results of this (batch, KV head): n_valid slots, `stride`
    // rows apart, from row `base` on.
    int n_valid;
    int64_t base, stride = p.rows;
    int64_t g_first = 0;  // stream-K: the first share holding this unit's tiles
    int64_t T = 0;        // stream-K: plan weight of this head's sequence
    int64_t sk_g = 0;     // stream-K: shares that cut it
    if (p.sk_grid > 0) {
        // Stream-K (by head): the shares of KV head kvh's plan weight T held
        // this unit's tiles, at [P + piece, P + piece + tiles) of that
        // sequence (the unit starts at P); share c held [c T / S, (c+1) T / S)
        // and wrote slot kvh (B + S) + b + c.
        const SkBatch sb = {sd, p.sk_bn, p.sk_win_left, p.sk_piece};
        int before;
        T = sk_sums(sb, b, before);
        const int tiles = sk_tiles(sb, b);
        const int64_t P = before;
        const int G = p.sk_grid * p.sk_hpw / p.Hkv;  // shares per KV head
        sk_g = G;
        if (tiles == 0 || T == 0) {
            n_valid = 0;
            g_first = 0;
        } else {
            // the share holding position s is the largest c with c T / S <= s
            const int64_t first = P + p.sk_piece, last = P + p.sk_piece + tiles - 1;
            g_first = ((first + 1) * G - 1) / T;
            const int64_t g_last = ((last + 1) * G - 1) / T;
            n_valid = (int)(g_last - g_first + 1);
        }
        const int64_t slot0 = (int64_t)kvh * (p.B + G) + b + g_first;
        base = slot0 * p.rows + r;
    } else {
        const int kv_len = seq_kv_len(sd, b);
        // the splits that hold keys of this request (the attention kernel
        // writes every row of each of them and nothing for the others)
        n_valid = min(p.n_splits, (kv_len + p.split_len - 1) / p.split_len);
        base = (int64_t)bh * p.n_splits * p.rows + r;
    }
    // stream-K: a share that is empty (T < shares) wrote nothing
    auto skip = [&](int s) -> bool {
        if (p.sk_grid == 0) return false;
        const int64_t g = g_first + s;
        return g * T / sk_g == (g + 1) * T / sk_g;
    };

    // the largest partial LSE; a NaN one (a NaN score in its share) wins, so
    // that the NaN reaches o and lse
    auto max_nan = [](float a, float b) -> float {
        return a != a ? a : (b != b ? b : fmaxf(a, b));
    };
    // lane s % 64 reads the LSE of split s (-inf for a skipped one); the
    // first 64 stay in their lanes for the weights below
    auto split_lse = [&](int s) -> float {
        return s < n_valid && !skip(s) ? p.lse_part[base + (int64_t)s * stride] : -INFINITY;
    };
    const float ls0 = split_lse(lane);
    float M = ls0;
    for (int s = lane + 64; s < n_valid; s += 64) M = max_nan(M, split_lse(s));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = max_nan(M, __shfl_xor(M, off));

    // o = sum_s exp(lse_s - M) o_s / sum_s exp(lse_s - M), in FP32.  A partial
    // row is D floats: D / 4 lanes hold it with 16-byte loads, so the wave
    // reads SPI = 256 / D splits per load instruction -- lane group g = lane /
    // (D / 4) takes splits g, g + SPI, ... in ascending order -- and up to
    // four such loads per lane are issued before any is used.  The groups'
    // sums are added at the end (a fixed order: the result does not depend
    // on timing).
    constexpr int LPR = D / 4;       // lanes per partial row
    constexpr int SPI = 64 / LPR;    // splits per load instruction
    const int grp = lane / LPR, pos = lane % LPR;
    f32x4 accv = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    if (M != -INFINITY) {
        for (int c = 0; c < n_valid; c += 64) {
            const float ls = c == 0 ? ls0 : split_lse(c + lane);
            const int cnt = min(64, n_valid - c);
            for (int q0 = 0; q0 < cnt; q0 += 4 * SPI) {
                float lq[4];
                f32x4 ov[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int s = q0 + k * SPI + grp;  // this group's split (within chunk c)
                    // lanes past the last split hold -inf
                    lq[k] = __shfl(ls, min(s, 63));
                    ov[k] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (s < cnt && lq[k] != -INFINITY)
                        ov[k] = *(const f32x4 *)(p.o_part +
                                                 (base + (int64_t)(c + s) * stride) * D + 4 * pos);
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int s = q0 + k * SPI + grp;
                    if (s >= cnt || lq[k] == -INFINITY) continue;
                    const float w = __expf(lq[k] - M);
                    den += w;
                    accv += w * ov[k];
                }
            }
        }
    }
    // add the lane groups' partial sums (groups differ in lane bits >= log2 LPR)
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
        den += __shfl_xor(den, off);
#pragma unroll
        for (int e = 0; e < 4; ++e) accv[e] += __shfl_xor(accv[e], off);
    }
    const int h = kvh * p.G + gh;
    float inv = den != 0.f ? 1.f / den : 0.f;
    float lse_out = den != 0.f ? M + __logf(den) : -INFINITY;
    if (p.sinks != nullptr) {
        const float sk = p.sinks[h];
        if (den == 0.f || sk == INFINITY) {
            inv = 0.f;
            lse_out = den == 0.f ? sk : INFINITY;
        } else {
            const float mx = fmaxf(M, sk);
            const float a = __expf(M - mx);
            const float den2 = __builtin_fmaf(den, a, __expf(sk - mx));
            inv = a / den2;
            lse_out = mx + __logf(den2);
        }
    }
    if (grp == 0) {
        uint16_t *dst = p.o + ((q_row0 + i) * p.Hq + h) * D + 4 * pos;
        const u32x2 packed = {(uint32_t)to_half_bits<BF16>(accv[0] * inv) |
                                  ((uint32_t)to_half_bits<BF16>(accv[1] * inv) << 16),
                              (uint32_t)to_half_bits<BF16>(accv[2] * inv) |
                                  ((uint32_t)to_half_bits<BF16>(accv[3] * inv) << 16)};
        *(u32x2 *)dst = packed;
    }
    if (p.lse != nullptr && lane == 0) {
        if (p.cu_q)  // packed: [Hq, total_q]
            p.lse[(int64_t)h * p.total_q + q_row0 + i] = lse_out;
        else
            p.lse[((int64_t)b * p.Hq + h) * p.Sq + i] = lse_out;
    }
}

template <int D, bool BF16>
hipError_t launch_one(const MergeParams &p, hipStream_t stream) {
    const int64_t rows = (int64_t)p.B * p.Hkv * p.rows;
    const int grid = (int)((rows + 3) / 4);
    hipLaunchKernelGGL((lse_merge_kernel<D, BF16>), dim3(grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(const MergeParams &p, int D, bool bf16, hipStream_t stream) {
    switch (D) {
        case 64: return bf16 ? launch_one<64, true>(p, stream) : launch_one<64, false>(p, stream);
        case 128: return bf16 ? launch_one<128, true>(p, stream) : launch_one<128, false>(p, stream);
        case 256: return bf16 ? launch_one<256, true>(p, stream) : launch_one<256, false>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace miattn
