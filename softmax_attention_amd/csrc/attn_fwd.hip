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

#include <type_traits>

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

// Round-to-nearest-even conversion of two floats into one packed dword (a
// single v_cvt_pk_{bf16,f16}_f32).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <bool BF16>
__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    if constexpr (BF16)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- LDS tiles.  A K or V tile is stored row-major (one key per row, D
// contiguous) without padding; the 16-byte chunks of row r are XOR-swizzled
// (chunk c sits at position c ^ swz(r)) so that both read patterns below hit
// distinct LDS banks: the QK^T operand (16 rows, one chunk each) and the
// transposing V read (4 consecutive rows, two adjacent chunks each).
//
// For D >= 128 the swizzle is a bit permutation of row & 15 (bits 0,1,2,3 of
// the row go to bits 2,3,1,0 of the chunk mask): any 16 consecutive rows get
// 16 distinct masks (conflict-free K reads), and the four rows a transposing
// read gathers differ in the mask's upper bits, so the two chunk pairs that
// neighbouring 16-lane groups fetch never share a bank.  Measured on gfx950:
// ~190 B/clk/CU for the K reads and ~124 B/clk/CU for the transposing reads.
template <int D>
__device__ __forceinline__ int swz(int row) {
    if constexpr (D == 64)
        return ((row >> 1) & 3) * 2 + ((row >> 3) & 1);
    else
        return ((row & 3) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1);
}

template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk) {  // bytes
    return row * (2 * D) + 16 * (chunk ^ swz<D>(row));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Sum of the two 16-bit values packed in `pk`, accumulated into acc in FP32.
template <bool BF16>
__device__ __forceinline__ float add_pair(uint32_t pk, float acc) {
    if constexpr (BF16)
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk),
                                               __builtin_bit_cast(bf16x2, 0x3f803f80u), acc,
                                               false);
    else
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk),
                                      __builtin_bit_cast(f16x2, 0x3c003c00u), acc, false);
}

// The running max is only raised when a tile's max exceeds it by more than
// this many powers of two; until then exponentials are taken against the
// stale max (bounded by 2^kLazy), which leaves the result unchanged in exact
// arithmetic and saves rescaling O for almost every tile.
constexpr float kLazy = 8.0f;

template <int D>
constexpr int waves_per_eu() { return D <= 128 ? 2 : 1; }

#ifndef MIATTN_VALU_PER_MFMA
#define MIATTN_VALU_PER_MFMA 6
#endif
constexpr int kValuPerMfma = MIATTN_VALU_PER_MFMA;

template <int D, bool BF16, bool PAGED>
__global__ __launch_bounds__(kThreadsPerBlock)
__attribute__((amdgpu_waves_per_eu(waves_per_eu<D>(), waves_per_eu<D>())))
void attn_fwd_kernel(const FwdParams p) {
    using H = Half<BF16>;
    using vec8 = typename H::vec8;
    constexpr int BN = keys_per_tile(D);   // keys per tile
    constexpr int TILE_BYTES = BN * D * 2; // 16 KB for K, the same for V
    constexpr int NT = BN / 32;            // 32-key score blocks per tile
    constexpr int KSTEPS = D / 16;         // MFMA k-steps over D
    constexpr int DT = D / 32;             // 32-wide d blocks of O^T
    constexpr int PSTEPS = BN / 16;        // MFMA k-steps over the tile's keys
    static_assert(TILE_BYTES == 16 * 1024, "one tile = 16 direct 1 KB loads");

    // two stages of (K tile, V tile); separate arrays so the compiler can
    // tell a load into one stage from reads of the other
    __shared__ __attribute__((aligned(1024))) uint8_t sK0[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sV0[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sK1[TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sV1[TILE_BYTES];

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

    // ---- Q for the whole kernel: B operand, lane = row, 8 d-values per k-step.
    // The host folds the sign of the scale into Q (an exact sign flip) and
    // turns a zero scale into a zero Q, so the kernel always scales by c > 0
    // and the row max stays a max.
    vec8 qf[KSTEPS];
    {
        const uint32_t flip = p.q_mode == 1 ? 0x80008000u : 0u;
        const bool load_q = row_ok && p.q_mode != 2;
        const uint16_t *qrow =
            p.q + (((int64_t)b * p.Sq + my_i) * p.Hq + (int64_t)kvh * p.G + my_gh) * D;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (load_q) raw = *(const u32x4 *)(qrow + 16 * ks + 8 * hl) ^ flip;
            qf[ks] = __builtin_bit_cast(vec8, raw);
        }
    }

    f32x16 acc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
    float m_run = -INFINITY;  // running (possibly stale) max, scaled log2 units
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

    // ---- HBM -> LDS, no registers: each of the tile's 16 1-KB pieces is one
    // global_load_lds_dwordx4 (lane l fills bytes [16l, 16l+16) of its piece);
    // piece e*4 + wave is this wave's e-th.  Lane l therefore always fills the
    // same (row, chunk) of every tile: fetch the chunk the swizzle puts there.
    const int64_t hstride = (int64_t)p.Hkv * D;  // elements between consecutive keys
    int ld_row[4];
    int64_t ld_base[4];  // element offset of this lane's chunk, key row 0
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int byte = (e * 4 + wave) * 1024 + 16 * lane;
        const int row = byte / (2 * D);
        const int pos = (byte % (2 * D)) / 16;
        ld_row[e] = row;
        ld_base[e] = (int64_t)kvh * D + 8 * (pos ^ swz<D>(row)) +
                     (PAGED ? 0 : (int64_t)b * p.Skv * hstride);
    }
    // a page holds whole tiles when page_size >= BN: one page per tile
    const bool page_per_tile = PAGED && p.page_shift >= __builtin_ctz(BN);
    const int32_t *bt_row = PAGED ? p.block_table + (int64_t)b * p.max_pages : nullptr;
    auto issue = [&](int j0, const uint16_t *src, uint8_t *dst) {
        int64_t tile_page_row = 0;
        if (page_per_tile) tile_page_row = (int64_t)bt_row[j0 >> p.page_shift] << p.page_shift;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // keys past the end load the last key (finite data, masked later)
            const int j = min(j0 + ld_row[e], kv_len - 1);
            int64_t row;
            if (!PAGED)
                row = j;
            else if (page_per_tile)
                row = tile_page_row + (j & ((1 << p.page_shift) - 1));
            else
                row = ((int64_t)bt_row[j >> p.page_shift] << p.page_shift) +
                      (j & ((1 << p.page_shift) - 1));
            const int64_t off = ld_base[e] + row * hstride;
            __builtin_amdgcn_global_load_lds((const void *)(src + off),
                                             (lds_void *)(dst + (e * 4 + wave) * 1024), 16, 0, 0);
        }
    };
    auto issue_k = [&](int j0, uint8_t *dst) { issue(j0, p.k, dst); };
    auto issue_v = [&](int j0, uint8_t *dst) { issue(j0, p.v, dst); };

    const float c = p.scale_log2;  // > 0

    // ---- LDS read addresses, fixed per lane for the whole kernel.  With the
    // swizzle depending on row & 15 only, the 32-key block t and the 16-key
    // step kk move a read by whole rows (an immediate offset); only the chunk
    // index varies with the swizzle, so one byte offset per chunk position is
    // kept in a register.
    //   K (QK^T A operand): lane reads row 32t + l32, chunk 2ks + hl.
    //   V (transposing read): in each 16-lane group g, lane 4r+q reads row
    //   4*(g/2) + r (+8 for k-slots 4..7) of the 16-key step, d-columns
    //   32t + 16*(g%2) + 4q .. +3.
    int k_addr[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) k_addr[ks] = tile_off<D>(l32, 2 * ks + hl);
    const int tr_g = lane >> 4;
    const int tr_row = 4 * (tr_g >> 1) + ((lane & 15) >> 2);
    const int tr_col = 16 * (tr_g & 1) + 4 * (lane & 3);
    int v_addr[DT][2];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int col = 32 * t + tr_col;
            v_addr[t][h] = tile_off<D>(tr_row + 8 * h, col >> 3) + (col & 7) * 2;
        }

    // ---- S^T = K Q^T for one tile (K from an LDS stage)
    auto qk = [&](const uint8_t *sk, f32x16 (&sc)[NT]) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[t][r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const vec8 a = __builtin_bit_cast(
                    vec8, *(const u32x4 *)(sk + k_addr[ks] + 32 * t * (2 * D)));
                sc[t] = H::mfma(a, qf[ks], sc[t]);
            }
        }
    };

    // ---- online softmax of one tile's scores: masks (MASKED tiles only), the
    // lazy max update, P rounded to 16 bits as the B operand of P.V, and the
    // running denominator.  Branch-free, so that the scheduler can interleave
    // it with the next tile's QK^T MFMAs.  Returns the factor the output
    // accumulator must be multiplied by (1 when the max did not move).
    auto softmax = [&](auto masked_tag, int j0, uint64_t mlo, uint64_t mhi, f32x16 (&sc)[NT],
                       vec8 (&pb)[PSTEPS]) -> float {
        constexpr bool MASKED = decltype(masked_tag)::value;
        if constexpr (MASKED) {
            // S^T layout: register r of lane half hl holds key
            // 32t + 8*(r/4) + 4*hl + r%4 of the tile
            const int lim = my_last - j0 - 4 * hl;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                uint32_t w = ~0u;
                if (has_mask) w = (uint32_t)((t < 2 ? mlo : mhi) >> (32 * (t & 1) + 4 * hl));
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kc = 32 * t + 8 * (r >> 2) + (r & 3);
                    const bool vis = (kc <= lim) && ((w >> (8 * (r >> 2) + (r & 3))) & 1u);
                    sc[t][r] = vis ? sc[t][r] : -INFINITY;
                }
            }
        }
        // row max of the raw scores (scaling by c > 0 keeps the order)
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[t][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float tile_max = (mx == -INFINITY) ? -INFINITY : mx * c;
        const bool raise = __any(tile_max > m_run + kLazy);
        const float m_new = raise ? fmaxf(m_run, tile_max) : m_run;
        const float corr = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
        m_run = m_new;
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;

        float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
        for (int kk = 0; kk < PSTEPS; ++kk) {
            const int t = kk >> 1, u = kk & 1;
            u32x4 packed;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float e0 = fast_exp2(__builtin_fmaf(sc[t][8 * u + 2 * e], c, -m_use));
                const float e1 = fast_exp2(__builtin_fmaf(sc[t][8 * u + 2 * e + 1], c, -m_use));
                packed[e] = pack_half2<BF16>(e0, e1);
                if (e & 1)
                    rs1 = add_pair<BF16>(packed[e], rs1);
                else
                    rs0 = add_pair<BF16>(packed[e], rs0);
            }
            pb[kk] = __builtin_bit_cast(vec8, packed);
        }
        l_run = __builtin_fmaf(l_run, corr, rs0 + rs1);
        return corr;
    };

    // ---- O^T += V^T P^T; the V^T operand comes from two transposing reads of
    // 4 keys each (k-slots 0..3 and 4..7 of this lane half)
    auto pv = [&](const uint8_t *sv, const vec8 (&pb)[PSTEPS]) {
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int kk = 0; kk < PSTEPS; ++kk) {
                const int step = 16 * kk * (2 * D);
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)(sv + v_addr[t][0] + step));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)(sv + v_addr[t][1] + step));
                const vec8 a = __builtin_bit_cast(
                    vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                acc[t] = H::mfma(a, pb[kk], acc[t]);
            }
    };

    // ---- scheduling hint for a block holding the next tile's QK^T and this
    // tile's softmax: alternate one K read, one MFMA and a few VALU
    // (transcendental included) instructions, so the MFMA pipe is fed while
    // the softmax runs
    auto interleave = [&]() {
#pragma unroll
        for (int i = 0; i < NT * KSTEPS; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x402, kValuPerMfma, 0);  // VALU + TRANS
        }
    };

    // ---- one pipeline step for this wave: softmax and P.V of tile `cur`
    // (scores already in sc_cur, V in stage sv), overlapped with QK^T of tile
    // `nxt` (K in stage sk) into sc_nxt
    auto step = [&](int cur, uint64_t mlo, uint64_t mhi, int nxt, f32x16 (&sc_cur)[NT],
                    f32x16 (&sc_nxt)[NT], const uint8_t *sk, const uint8_t *sv) {
        if (!(wave_active && cur < wave_end)) return;  // nothing for this wave any more
        bool full = cur + BN <= wave_full_end;
        if (has_mask) full = full && (mlo == kLoMask) && (BN <= 64 || mhi == ~0ull);
        vec8 pb[PSTEPS];
        float corr;
        if (nxt < wave_end) {
            if (full) {
                qk(sk, sc_nxt);
                corr = softmax(std::false_type{}, cur, mlo, mhi, sc_cur, pb);
                interleave();
            } else {
                qk(sk, sc_nxt);
                corr = softmax(std::true_type{}, cur, mlo, mhi, sc_cur, pb);
                interleave();
            }
        } else {
            if (full)
                corr = softmax(std::false_type{}, cur, mlo, mhi, sc_cur, pb);
            else
                corr = softmax(std::true_type{}, cur, mlo, mhi, sc_cur, pb);
        }
        if (corr != 1.f) {
#pragma unroll
            for (int t = 0; t < DT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[t][r] *= corr;
        }
        pv(sv, pb);
    };

    // ---- main loop.  K and V have rings of two stages each.  At the start of
    // the step for tile `cur`: its scores are in registers, its V is in one V
    // stage and the next tile's K in one K stage; the step streams the K of
    // the tile after next and the V of the next tile into the free stages
    // (straight from HBM, no registers) while the waves compute.
    uint64_t mc_lo = ~0ull, mc_hi = ~0ull, mn_lo = ~0ull, mn_hi = ~0ull, m2_lo = ~0ull,
             m2_hi = ~0ull;
    f32x16 scA[NT], scB[NT];
    int cur = find_tile(kbeg, mc_lo, mc_hi);
    int nxt = cur < wg_end ? find_tile(cur + BN, mn_lo, mn_hi) : wg_end;
    if (cur < wg_end) {
        issue_k(cur, sK0);
        issue_v(cur, sV0);
    }
    if (nxt < wg_end) issue_k(nxt, sK1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (wave_active && cur < wave_end) qk(sK0, scA);
    while (cur < wg_end) {
        // tile cur: scores in scA, V in sV0; tile nxt: K in sK1
        int nxt2 = nxt < wg_end ? find_tile(nxt + BN, m2_lo, m2_hi) : wg_end;
        if (nxt2 < wg_end) issue_k(nxt2, sK0);
        if (nxt < wg_end) issue_v(nxt, sV1);
        step(cur, mc_lo, mc_hi, nxt, scA, scB, sK1, sV0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        cur = nxt; mc_lo = mn_lo; mc_hi = mn_hi;
        nxt = nxt2; mn_lo = m2_lo; mn_hi = m2_hi;
        if (cur >= wg_end) break;
        // tile cur: scores in scB, V in sV1; tile nxt: K in sK0
        nxt2 = nxt < wg_end ? find_tile(nxt + BN, m2_lo, m2_hi) : wg_end;
        if (nxt2 < wg_end) issue_k(nxt2, sK1);
        if (nxt < wg_end) issue_v(nxt, sV0);
        step(cur, mc_lo, mc_hi, nxt, scB, scA, sK0, sV1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        cur = nxt; mc_lo = mn_lo; mc_hi = mn_hi;
        nxt = nxt2; mn_lo = m2_lo; mn_hi = m2_hi;
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
