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
template <int D>
__device__ __forceinline__ int swz(int row) {
    if constexpr (D == 64)
        return ((row >> 1) & 3) * 2 + ((row >> 3) & 1);
    else
        return (row & 7) * 2 + ((row >> 3) & 1);
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

    // ---- HBM -> LDS, no registers: each of the tile's 16 1-KB pieces is one
    // global_load_lds_dwordx4 (lane l fills bytes [16l, 16l+16) of its piece);
    // piece e*4 + wave is this wave's e-th.  Lane l therefore always fills the
    // same (row, chunk) of every tile: fetch the chunk the swizzle puts there.
    int ld_row[4], ld_chunk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int byte = (e * 4 + wave) * 1024 + 16 * lane;
        const int row = byte / (2 * D);
        const int pos = (byte % (2 * D)) / 16;
        ld_row[e] = row;
        ld_chunk[e] = pos ^ swz<D>(row);
    }
    auto issue = [&](int j0, uint8_t *dk, uint8_t *dv) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // keys past the end load the last key (finite data, masked below)
            const int j = min(j0 + ld_row[e], kv_len - 1);
            const int64_t off = key_row(j) + 8 * ld_chunk[e];
            const int piece = (e * 4 + wave) * 1024;
            __builtin_amdgcn_global_load_lds((const void *)(p.k + off), (lds_void *)(dk + piece),
                                             16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void *)(p.v + off), (lds_void *)(dv + piece),
                                             16, 0, 0);
        }
    };

    const float c = p.scale_log2;  // > 0

    // per-lane constants of the transposing V read: in each 16-lane group,
    // lane 4r+q points at row r (of 4) and d-columns 4q..4q+3 of its block
    const int tr_g = lane >> 4;
    const int tr_row = 4 * (tr_g >> 1) + ((lane & 15) >> 2);
    const int tr_col = 16 * (tr_g & 1) + 4 * (lane & 3);

    // ---- one tile of scores, online softmax and P.V for this wave's rows
    auto compute = [&](int j0, uint64_t mlo, uint64_t mhi, const uint8_t *sk,
                       const uint8_t *sv) {
        f32x16 s[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[t][r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const vec8 a = __builtin_bit_cast(
                    vec8, *(const u32x4 *)(sk + tile_off<D>(32 * t + l32, 2 * ks + hl)));
                s[t] = H::mfma(a, qf[ks], s[t]);
            }
        }

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
                    if (has_mask)
                        vis = vis && (((kk < 64 ? mlo >> kk : mhi >> (kk - 64)) & 1ull) != 0);
                    if (!vis) s[t][r] = -INFINITY;
                }
        }

        // row max of the raw scores (scaling by c >= 0 keeps the order)
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float tile_max = (mx == -INFINITY) ? -INFINITY : mx * c;
        if (__any(tile_max > m_run + kLazy)) {
            const float m_new = fmaxf(m_run, tile_max);
            const float corr = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
            l_run *= corr;
#pragma unroll
            for (int t = 0; t < DT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[t][r] *= corr;
            m_run = m_new;
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

        // P = exp2(c*s - m) rounded to 16 bits: the B operand of P.V; the row
        // sum adds the rounded values, the ones P.V actually uses
        vec8 pb[PSTEPS];
        float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
        for (int kk = 0; kk < PSTEPS; ++kk) {
            const int t = kk >> 1, u = kk & 1;
            u32x4 packed;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float e0 = fast_exp2(__builtin_fmaf(s[t][8 * u + 2 * e], c, -m_use));
                const float e1 = fast_exp2(__builtin_fmaf(s[t][8 * u + 2 * e + 1], c, -m_use));
                packed[e] = pack_half2<BF16>(e0, e1);
                if (e & 1)
                    rs1 = add_pair<BF16>(packed[e], rs1);
                else
                    rs0 = add_pair<BF16>(packed[e], rs0);
            }
            pb[kk] = __builtin_bit_cast(vec8, packed);
        }
        l_run += rs0 + rs1;

        // O^T += V^T P^T; the V^T operand comes from two transposing reads of
        // 4 keys each (k-slots 0..3 and 4..7 of this lane half)
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int kk = 0; kk < PSTEPS; ++kk) {
                const int row = 16 * kk + tr_row;
                const int col = 32 * t + tr_col;
                const int within = (col & 7) * 2;
                const s16x4 lo =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(sv + tile_off<D>(row, col >> 3) + within));
                const s16x4 hi =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(sv + tile_off<D>(row + 8, col >> 3) + within));
                const short vals[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                vec8 a;
                __builtin_memcpy(&a, vals, sizeof a);
                acc[t] = H::mfma(a, pb[kk], acc[t]);
            }
    };

    // ---- main loop: a two-stage LDS ring; while the waves compute one tile
    // the next one streams from HBM straight into the other stage
    uint64_t lo0 = ~0ull, hi0 = ~0ull, lo1 = ~0ull, hi1 = ~0ull;
    int cur = find_tile(kbeg, lo0, hi0);
    if (cur < wg_end) issue(cur, sK0, sV0);
    while (cur < wg_end) {
        // stage 0 holds tile `cur`
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        int nxt = find_tile(cur + BN, lo1, hi1);
        if (nxt < wg_end) issue(nxt, sK1, sV1);
        if (wave_active && cur < wave_end) compute(cur, lo0, hi0, sK0, sV0);
        cur = nxt;
        if (cur >= wg_end) break;
        // stage 1 holds tile `cur`
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        nxt = find_tile(cur + BN, lo0, hi0);
        if (nxt < wg_end) issue(nxt, sK0, sV0);
        if (wave_active && cur < wave_end) compute(cur, lo1, hi1, sK1, sV1);
        cur = nxt;
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
