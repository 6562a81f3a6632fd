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
// Work decomposition (one workgroup = 4 waves = 256 threads):
//   * rows: the query rows of the G = Hq/Hkv heads that share a KV head are
//     packed (row r = query r / G, head kvh*G + r % G); a workgroup owns 128
//     packed rows, each wave 32 of them.  In decode (Sq = 1) the whole GQA
//     group lands in one wave's MFMA tile.
//   * keys: a workgroup walks its key range in tiles of 8192 / D keys.  All 256
//     threads load the next K and V tile from HBM with 16-byte loads into
//     registers while the waves compute on the current tile from LDS.  K is
//     stored row-major; V is stored transposed (d-major) so that the P.V MFMA
//     reads its key-contiguous operand with one 16-byte LDS read per lane.
//   * scores: S^T = K Q^T with v_mfma_f32_32x32x16_{bf16,f16}: K (from LDS) is
//     the A operand, Q (held in registers for the whole kernel) the B operand.
//     Each lane then holds 16 scores per 32-key block for ONE query row (its
//     column), so the row max needs one cross-lane step (lane ^ 32) and the row
//     sum none until the end.
//   * P.V: O^T = V^T P^T.  The exponentiated scores are already laid out as the
//     B operand (row = lane's column, 8 keys per lane), so P goes from the
//     score registers to the MFMA without any data movement; O^T accumulates in
//     registers with each lane owning one row, which makes the per-row
//     rescaling lane-local.
//   * masking: a tile that is fully visible to every row of a wave takes no
//     per-element test; a tile beyond a wave's last visible key is skipped by
//     that wave; tiles beyond the workgroup's last visible key are never
//     loaded; with a key padding mask, tiles whose keys are all masked are
//     skipped before their K/V is loaded.
#include "attn_kernels.h"

namespace miattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.6931471805599453f;

template <bool BF16>
struct Half;

template <>
struct Half<true> {
    using vec8 = bf16x8;
    using scalar = __bf16;
    static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Half<false> {
    using vec8 = f16x8;
    using scalar = _Float16;
    static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// Round-to-nearest-even conversion of two floats into one packed dword.
template <bool BF16>
__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
    using S = typename Half<BF16>::scalar;
    const S a = (S)lo, b = (S)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Within each 16-key group of the transposed V tile, the four 4-key units are
// stored in the order the 32x32 score layout hands them to a lane half: lane
// half h holds keys {4h..4h+3, 8+4h..8+4h+3} of the group, so units 0 and 2
// go first (half 0), then units 1 and 3 (half 1).
__device__ __forceinline__ int unit_slot(int unit) {
    const int u = unit & 3;
    return (unit >> 2) * 16 + ((u == 1) ? 2 : (u == 2) ? 1 : u) * 4;
}

template <int D, bool BF16, bool PAGED>
__global__ __launch_bounds__(kThreadsPerBlock) void attn_fwd_kernel(const FwdParams p) {
    using H = Half<BF16>;
    using vec8 = typename H::vec8;
    constexpr int BN = keys_per_tile(D);   // keys per tile
    constexpr int KSTR = D + 8;            // K tile row stride (elements); +16 B pad
    constexpr int VSTR = BN + 8;           // V^T tile row stride (elements); +16 B pad
    constexpr int NT = BN / 32;            // 32-key score blocks per tile
    constexpr int KSTEPS = D / 16;         // MFMA k-steps over D
    constexpr int DT = D / 32;             // 32-wide d blocks of O^T
    constexpr int PSTEPS = BN / 16;        // MFMA k-steps over the tile's keys
    constexpr int DCH = D / 8;             // 16-byte chunks per row
    constexpr int VUNITS = BN / 4;         // 4-key units per tile
    static_assert(BN * DCH == 4 * kThreadsPerBlock, "K tile: 4 chunks per thread");
    static_assert(VUNITS * DCH == kThreadsPerBlock, "V tile: one 4x8 block per thread");

    __shared__ __attribute__((aligned(16))) uint16_t sK[BN * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t sV[D * VSTR];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hl = lane >> 5;

    // ---- which (row block, batch, KV head, split) this workgroup owns.
    // Workgroups are dispatched round-robin over the 8 XCDs; when the unit
    // count allows, consecutive workgroups of one XCD share a (batch, KV head)
    // so its K/V stays in that XCD's L2.  Causal row blocks run heaviest first.
    const int units = p.B * p.Hkv * p.n_splits;
    int rank, unit;
    if (p.xcd_units > 0) {
        const int s = blockIdx.x >> 3;
        unit = (blockIdx.x & 7) * p.xcd_units + s % p.xcd_units;
        rank = s / p.xcd_units;
    } else {
        rank = blockIdx.x / units;
        unit = blockIdx.x - rank * units;
    }
    const int mblock = p.causal ? (p.n_mblocks - 1 - rank) : rank;
    const int bh = unit / p.n_splits;
    const int split = unit - bh * p.n_splits;
    const int b = bh / p.Hkv;
    const int kvh = bh - b * p.Hkv;

    const int kv_len = PAGED ? p.seqlen[b] : p.Skv;
    const int kbeg = split * p.split_len;
    // Splits past the end are never read by the merge, which counts the
    // splits that hold keys from the same length.
    if (p.n_splits > 1 && kbeg >= kv_len) return;
    const int kend = min(kv_len, kbeg + p.split_len);
    const int delta = kv_len - p.Sq;  // query i sits at key position i + delta

    const int row0 = mblock * kRowsPerBlock;
    const int row_last = min(p.rows, row0 + kRowsPerBlock) - 1;
    const int wg_end = p.causal ? min(kend, row_last / p.G + delta + 1) : kend;

    const int wrow0 = row0 + wave * kRowsPerWave;
    const bool wave_active = wrow0 < p.rows;
    const int wrow_last = min(p.rows, wrow0 + kRowsPerWave) - 1;
    // keys < wave_full_end are visible to every row of this wave; keys >=
    // wave_end to none of them
    const int wave_end =
        !wave_active ? kbeg : (p.causal ? min(kend, wrow_last / p.G + delta + 1) : kend);
    const int wave_full_end =
        !wave_active ? kbeg : (p.causal ? min(kend, wrow0 / p.G + delta + 1) : kend);

    // ---- this lane's query row (the column it holds in every MFMA tile)
    const int my_row = wrow0 + l32;
    const bool row_ok = my_row < p.rows;
    const int my_i = my_row / p.G;
    const int my_gh = my_row - my_i * p.G;
    const int my_last = !row_ok ? -1 : (p.causal ? min(kv_len - 1, my_i + delta) : kv_len - 1);

    // ---- Q for the whole kernel: B operand, lane = row, 8 d-values per k-step
    vec8 qf[KSTEPS];
    {
        const uint16_t *qrow =
            p.q + (((int64_t)b * p.Sq + my_i) * p.Hq + (int64_t)kvh * p.G + my_gh) * D;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (row_ok) raw = *(const u32x4 *)(qrow + 16 * ks + 8 * hl);
            qf[ks] = __builtin_bit_cast(vec8, raw);
        }
    }

    f32x16 acc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
    float m_run = -INFINITY;  // running max of the scaled log2-domain scores
    float l_run = 0.f;        // this lane's part of the running denominator

    // ---- key padding mask: one bit per key of a tile, wave-uniform
    const bool has_mask = !PAGED && p.mask != nullptr;
    const uint8_t *mrow = has_mask ? p.mask + (int64_t)b * p.Skv : nullptr;
    constexpr uint64_t kLoMask = BN >= 64 ? ~0ull : ((1ull << BN) - 1);
    auto tile_bits = [&](int j0, uint64_t &lo, uint64_t &hi) {
        const int j = j0 + lane;
        const bool keep0 = (lane < BN) && j < kv_len && mrow[j] != 0;
        lo = __ballot(keep0) & kLoMask;
        hi = 0;
        if (BN > 64) {
            const bool keep1 = j + 64 < kv_len && mrow[j + 64] != 0;
            hi = __ballot(keep1);
        }
    };
    // first tile start >= j that holds a kept key (or wg_end)
    auto find_tile = [&](int j, uint64_t &lo, uint64_t &hi) -> int {
        if (!has_mask) return j;
        for (; j < wg_end; j += BN) {
            tile_bits(j, lo, hi);
            if (lo | hi) return j;
        }
        return wg_end;
    };

    // ---- element offset of key j's row for this KV head
    const int64_t hstride = (int64_t)p.Hkv * D;
    auto key_row = [&](int j) -> int64_t {
        int64_t row;
        if (PAGED) {
            const int page = p.block_table[(int64_t)b * p.max_pages + (j >> p.page_shift)];
            row = ((int64_t)page << p.page_shift) + (j & ((1 << p.page_shift) - 1));
        } else {
            row = (int64_t)b * p.Skv + j;
        }
        return row * hstride + (int64_t)kvh * D;
    };

    // ---- HBM -> registers for one tile (keys >= kv_len read as zero)
    u32x4 kr[4], vr[4];
    const int v_unit = tid % VUNITS;
    const int v_chunk = tid / VUNITS;
    auto gload = [&](int j0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = tid + kThreadsPerBlock * e;
            const int kk = c / DCH, dc = c % DCH;
            const int j = j0 + kk;
            kr[e] = u32x4{0u, 0u, 0u, 0u};
            if (j < kv_len) kr[e] = *(const u32x4 *)(p.k + key_row(j) + dc * 8);
        }
        const int jv = j0 + 4 * v_unit;  // 4 consecutive keys, one page (page >= 16)
#pragma unroll
        for (int e = 0; e < 4; ++e) vr[e] = u32x4{0u, 0u, 0u, 0u};
        if (jv < kv_len) {
            const uint16_t *src = p.v + key_row(jv) + v_chunk * 8;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (jv + e < kv_len) vr[e] = *(const u32x4 *)(src + e * hstride);
        }
    };

    // ---- registers -> LDS (K row-major; V transposed to [d][key])
    auto lstore = [&]() {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = tid + kThreadsPerBlock * e;
            const int kk = c / DCH, dc = c % DCH;
            *(u32x4 *)&sK[kk * KSTR + dc * 8] = kr[e];
        }
        const int slot = unit_slot(v_unit);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            // dword w of each key row holds d = 2w (low half) and 2w + 1 (high)
            const u32x2 even = {(vr[0][w] & 0xffffu) | (vr[1][w] << 16),
                                (vr[2][w] & 0xffffu) | (vr[3][w] << 16)};
            const u32x2 odd = {(vr[0][w] >> 16) | (vr[1][w] & 0xffff0000u),
                               (vr[2][w] >> 16) | (vr[3][w] & 0xffff0000u)};
            *(u32x2 *)&sV[(v_chunk * 8 + 2 * w) * VSTR + slot] = even;
            *(u32x2 *)&sV[(v_chunk * 8 + 2 * w + 1) * VSTR + slot] = odd;
        }
    };

    // ---- one tile of scores, online softmax and P.V for this wave's rows
    auto compute = [&](int j0, uint64_t mlo, uint64_t mhi) {
        f32x16 s[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[t][r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const vec8 a = __builtin_bit_cast(
                    vec8, *(const u32x4 *)&sK[(32 * t + l32) * KSTR + 16 * ks + 8 * hl]);
                s[t] = H::mfma(a, qf[ks], s[t]);
            }
        }
        // scale into the log2 domain, then mask (so a negative or zero scale
        // never meets an infinite score)
        const float c = p.scale_log2;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[t][r] *= c;

        bool full = j0 + BN <= wave_full_end;
        if (has_mask) full = full && (mlo == kLoMask) && (BN <= 64 || mhi == ~0ull);
        if (!full) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    // S^T layout: register r of lane half hl holds key
                    // 8*(r/4) + 4*hl + r%4 of the 32-key block
                    const int kk = 32 * t + 8 * (r >> 2) + 4 * hl + (r & 3);
                    bool vis = j0 + kk <= my_last;
                    if (has_mask) vis = vis && (((kk < 64 ? mlo >> kk : mhi >> (kk - 64)) & 1ull) != 0);
                    if (!vis) s[t][r] = -INFINITY;
                }
        }

        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float corr = fast_exp2(m_run - m_use);
        float rs = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = fast_exp2(s[t][r] - m_use);
                s[t][r] = e;
                rs += e;
            }
        l_run = l_run * corr + rs;
        m_run = m_new;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[t][r] *= corr;

        // P^T as the B operand: k-step kk takes registers 8u..8u+7 of block kk/2
        vec8 pb[PSTEPS];
#pragma unroll
        for (int kk = 0; kk < PSTEPS; ++kk) {
            const int t = kk >> 1, u = kk & 1;
            u32x4 packed;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                packed[e] = pack_half2<BF16>(s[t][8 * u + 2 * e], s[t][8 * u + 2 * e + 1]);
            pb[kk] = __builtin_bit_cast(vec8, packed);
        }
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int kk = 0; kk < PSTEPS; ++kk) {
                const vec8 a = __builtin_bit_cast(
                    vec8, *(const u32x4 *)&sV[(32 * t + l32) * VSTR + 16 * kk + 8 * hl]);
                acc[t] = H::mfma(a, pb[kk], acc[t]);
            }
    };

    // ---- main loop: one tile in LDS, the next one in flight to registers
    uint64_t cur_lo = ~0ull, cur_hi = ~0ull, nxt_lo = ~0ull, nxt_hi = ~0ull;
    int cur = find_tile(kbeg, cur_lo, cur_hi);
    if (cur < wg_end) gload(cur);
    while (cur < wg_end) {
        __syncthreads();  // every wave is done reading the previous tile
        lstore();
        __syncthreads();
        const int nxt = find_tile(cur + BN, nxt_lo, nxt_hi);
        if (nxt < wg_end) gload(nxt);
        if (wave_active && cur < wave_end) compute(cur, cur_lo, cur_hi);
        cur = nxt;
        cur_lo = nxt_lo;
        cur_hi = nxt_hi;
    }

    // ---- epilogue: normalise and store (no barrier below this point)
    if (!wave_active) return;
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (!row_ok) return;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse_v = l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;

    if (p.n_splits == 1) {
        uint16_t *orow =
            p.o + (((int64_t)b * p.Sq + my_i) * p.Hq + (int64_t)kvh * p.G + my_gh) * D;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // registers 4w..4w+3 hold d = 32t + 8w + 4*hl + 0..3
                const int d0 = 32 * t + 8 * w + 4 * hl;
                const u32x2 packed = {pack_half2<BF16>(acc[t][4 * w] * inv, acc[t][4 * w + 1] * inv),
                                      pack_half2<BF16>(acc[t][4 * w + 2] * inv,
                                                       acc[t][4 * w + 3] * inv)};
                *(u32x2 *)(orow + d0) = packed;
            }
        if (p.lse != nullptr && hl == 0)
            p.lse[((int64_t)b * p.Hq + (int64_t)kvh * p.G + my_gh) * p.Sq + my_i] = lse_v;
    } else {
        const int64_t part = ((int64_t)bh * p.n_splits + split) * p.rows + my_row;
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
    }
}

template <int D, bool BF16, bool PAGED>
hipError_t launch_one(const FwdParams &p, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((attn_fwd_kernel<D, BF16, PAGED>), dim3(grid), dim3(kThreadsPerBlock), 0,
                       stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdParams &p, bool bf16, bool paged, int grid, hipStream_t stream) {
    if (bf16)
        return paged ? launch_one<D, true, true>(p, grid, stream)
                     : launch_one<D, true, false>(p, grid, stream);
    return paged ? launch_one<D, false, true>(p, grid, stream)
                 : launch_one<D, false, false>(p, grid, stream);
}

}  // namespace

hipError_t launch_attn_fwd(const FwdParams &p, int D, bool bf16, bool paged, int grid,
                           hipStream_t stream) {
    switch (D) {
        case 64: return launch_d<64>(p, bf16, paged, grid, stream);
        case 128: return launch_d<128>(p, bf16, paged, grid, stream);
        case 256: return launch_d<256>(p, bf16, paged, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace miattn
