// attn_bwd.hip -- grouped-query softmax attention backward for gfx950.
//
// TileOPs "Attention Operators", GQABwdOp: from q, k, v, o, do and the
// forward's natural-log lse, the gradients of O = softmax(alpha Q K^T + M) V:
//     P_ij = exp(alpha s_ij - lse_i)   (s_ij = <q_i, k_j>, visible keys only)
//     dP_ij = <dO_i, v_j>,   D_i = <dO_i, o_i>,   dS_ij = P_ij (dP_ij - D_i)
//     dq_i = alpha sum_j dS_ij k_j,  dk_j = alpha sum_i dS_ij q_i,
//     dv_j = sum_i P_ij dO_i,
// a KV head's dk/dv summing over the query heads of its group (the standard
// softmax-attention backward, as in Dao 2023, "FlashAttention-2").
//
// Two kernels, no atomics (every output element has one writer, so the
// result is the same bits on every call):
//   bwd_dq:    per 128 packed query rows (4 waves x 32), streaming 32-key
//              tiles: S^T = K Q^T and dP^T = V dO^T (K, V tiles as the A
//              operand, the wave's Q and dO rows in registers as B), then
//              dQ^T += K^T dS^T (K^T through the transposing LDS read, dS^T
//              straight from the score registers) -- the forward's layout.
//              It also forms D_i and lse_i log2(e) of its rows (+inf for a
//              row without a visible key, so that its P is exactly 0 without
//              a branch) and leaves them for bwd_dkdv;
//   bwd_dkdv:  per 128 keys of a KV head (4 waves x 32 keys, the wave's K and
//              V rows in registers), streaming 32-row tiles of the packed
//              query rows of all g heads: S = Q K^T and dP = dO V^T, then
//              dV^T += dO^T P and dK^T += Q^T dS (dO^T, Q^T transposed reads).
// Tiles go global -> registers -> LDS (swizzled like the forward's K/V tiles)
// with a two-buffer ring and one workgroup barrier per tile.
#include "attn_kernels.h"

#include <type_traits>

#include "attn_device.h"

namespace miattn {
namespace {

using namespace dev;

constexpr int kBwdRows = 32;   // rows of a streamed tile (keys for dq, packed rows for dk/dv)
constexpr int kBwdWaves = 4;

// ---- shared tile machinery
template <int D>
struct TileGeom {
    static constexpr int CHUNKS = kBwdRows * D / 8;        // 16-byte chunks per tile
    static constexpr int CPT = CHUNKS / (64 * kBwdWaves);  // chunks per thread
    static constexpr int KSTEPS = D / 16;
    static constexpr int DT = D / 32;
    static constexpr int PSTEPS = kBwdRows / 16;
    static constexpr int BYTES = kBwdRows * D * 2;
};

// LDS read addresses fixed per lane (the forward's patterns): the plain
// operand read (row l32, chunk 2ks + hl) and the transposing read.
template <int D>
struct LaneAddr {
    int k_addr[D / 16];
    int v_addr[D / 32][2];
    __device__ __forceinline__ void init(int lane) {
        const int l32 = lane & 31, hl = lane >> 5;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) k_addr[ks] = tile_off<D>(l32, 2 * ks + hl);
        const int tr_g = lane >> 4;
        const int tr_row = 4 * (tr_g >> 1) + ((lane & 15) >> 2);
        const int tr_col = 16 * (tr_g & 1) + 4 * (lane & 3);
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int col = 32 * t + tr_col;
                v_addr[t][h] = tile_off<D>(tr_row + 8 * h, col >> 3) + (col & 7) * 2;
            }
    }
};

// A (rows x d) product over a tile: C[32x32] += A(tile rows, plain reads) B(regs)
template <int D, bool BF16>
__device__ __forceinline__ f32x16 tile_times_regs(const uint8_t *tile, const LaneAddr<D> &la,
                                                  const typename Half<BF16>::vec8 (&b)[D / 16]) {
    using vec8 = typename Half<BF16>::vec8;
    constexpr int KS = D / 16;
    constexpr int CH = KS < 8 ? KS : 8;
    f32x16 c;
#pragma unroll
    for (int r = 0; r < 16; ++r) c[r] = 0.f;
#pragma unroll
    for (int k0 = 0; k0 < KS; k0 += CH) {
        vec8 a[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j)
            a[j] = __builtin_bit_cast(vec8, *(const u32x4 *)(tile + la.k_addr[k0 + j]));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < CH; ++j) c = Half<BF16>::mfma(a[j], b[k0 + j], c);
    }
    return c;
}

// acc[t] (d block t x 32 columns) += tile^T (d x tile rows, transposing reads) * pk
template <int D, bool BF16>
__device__ __forceinline__ void tileT_times_packed(const uint8_t *tile, const LaneAddr<D> &la,
                                                   const typename Half<BF16>::vec8 (&pk)[kBwdRows / 16],
                                                   f32x16 (&acc)[D / 32]) {
    using vec8 = typename Half<BF16>::vec8;
    constexpr int PS = kBwdRows / 16;
    constexpr int DTN = D / 32;
    constexpr int TB = (8 / PS) < DTN ? (8 / PS) : DTN;
#pragma unroll
    for (int t0 = 0; t0 < DTN; t0 += TB) {
        vec8 a[TB][PS];
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
            for (int kk = 0; kk < PS; ++kk) {
                const int step = 16 * kk * (2 * D);
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)(tile + la.v_addr[t0 + t][0] + step));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)(tile + la.v_addr[t0 + t][1] + step));
                a[t][kk] = __builtin_bit_cast(
                    vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < TB; ++t)
#pragma unroll
            for (int kk = 0; kk < PS; ++kk)
                acc[t0 + t] = Half<BF16>::mfma(a[t][kk], pk[kk], acc[t0 + t]);
    }
}

// 16 fp32 score registers -> the packed 16-bit B operand of the next product
// (register pairs 8u + 2e, 8u + 2e + 1 of k-step u; the forward's order)
template <bool BF16>
__device__ __forceinline__ void pack_scores(const f32x16 &x,
                                            typename Half<BF16>::vec8 (&pk)[kBwdRows / 16]) {
    using vec8 = typename Half<BF16>::vec8;
#pragma unroll
    for (int u = 0; u < kBwdRows / 16; ++u) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_half2<BF16>(x[8 * u + 2 * e], x[8 * u + 2 * e + 1]);
        pk[u] = __builtin_bit_cast(vec8, w);
    }
}

// store 32 rows x D of a 32x32-block accumulator set (lane = row, registers
// 4w..4w+3 of block t = d 32t + 8w + 4hl + 0..3), scaled.  The two lanes of
// a row (hl = 0, 1; both active or neither) trade halves with
// v_permlane32_swap, which swaps lanes 32..63 of its first operand with lanes
// 0..31 of its second, so that lane hl stores d = 32t + 8(w + hl) + 0..7 as
// one 16-byte store for w = 0, 2.
template <int D, bool BF16>
__device__ __forceinline__ void store_rows(uint16_t *row_ptr, const f32x16 (&acc)[D / 32],
                                           float s, int hl) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int w = 0; w < 4; w += 2) {
            auto pk = [&](int r) __attribute__((always_inline)) {
                return pack_half2<BF16>(acc[t][r] * s, acc[t][r + 1] * s);
            };
            const auto lo = __builtin_amdgcn_permlane32_swap(pk(4 * w), pk(4 * w + 4), false, false);
            const auto hi = __builtin_amdgcn_permlane32_swap(pk(4 * w + 2), pk(4 * w + 6), false, false);
            const u32x4 packed = {(uint32_t)lo[0], (uint32_t)hi[0], (uint32_t)lo[1], (uint32_t)hi[1]};
            *(u32x4 *)(row_ptr + 32 * t + 8 * (w + hl)) = packed;
        }
}

// sum over the 8 16-bit pairs of two 16-byte chunks of a * c, in FP32
template <bool BF16>
__device__ __forceinline__ float dot8(const u32x4 &a, const u32x4 &c) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        if constexpr (BF16) {
            acc = __builtin_fmaf(__builtin_bit_cast(float, a[w] << 16),
                                 __builtin_bit_cast(float, c[w] << 16), acc);
            acc = __builtin_fmaf(__builtin_bit_cast(float, a[w] & 0xffff0000u),
                                 __builtin_bit_cast(float, c[w] & 0xffff0000u), acc);
        } else {
            acc = __builtin_fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)a[w]),
                                 (float)__builtin_bit_cast(_Float16, (uint16_t)c[w]), acc);
            acc = __builtin_fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(a[w] >> 16)),
                                 (float)__builtin_bit_cast(_Float16, (uint16_t)(c[w] >> 16)), acc);
        }
    }
    return acc;
}

// ---- bwd_dq
template <int D, bool BF16>
__global__ __launch_bounds__(64 * kBwdWaves)
__attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(const BwdParams p) {
    using G = TileGeom<D>;
    using vec8 = typename Half<BF16>::vec8;
    __shared__ __attribute__((aligned(1024))) uint8_t sK[2][G::BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sV[2][G::BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int l32 = lane & 31, hl = lane >> 5;
    const int units = p.B * p.Hkv;
    const int rank = blockIdx.x / units;
    const int unit = blockIdx.x - rank * units;
    const int mblock = p.causal ? p.n_mblocks - 1 - rank : rank;  // heaviest first
    const int b = unit / p.Hkv, kvh = unit - b * p.Hkv;
    const int delta = p.Skv - p.Sq;
    const int row0 = mblock * (32 * kBwdWaves);
    const int row_last = min(p.rows, row0 + 32 * kBwdWaves) - 1;
    const int wg_end = p.causal ? min(p.Skv, row_last / p.G + delta + 1) : p.Skv;

    const int my_row = row0 + wave * 32 + l32;
    const bool row_ok = my_row < p.rows;
    const int my_i = (row_ok ? my_row : p.rows - 1) / p.G;
    const int my_gh = (row_ok ? my_row : p.rows - 1) - my_i * p.G;
    const int my_h = kvh * p.G + my_gh;
    const int my_last = !row_ok ? -1 : (p.causal ? min(p.Skv - 1, my_i + delta) : p.Skv - 1);
    // the wave's last visible key (uniform: the MFMAs below run on whole waves)
    const int wrow_last = min(p.rows, row0 + wave * 32 + 32) - 1;
    const bool wave_rows = row0 + wave * 32 < p.rows;
    const int wave_last = !wave_rows ? -1
                          : (p.causal ? min(p.Skv - 1, wrow_last / p.G + delta) : p.Skv - 1);
    // the last visible key of the wave's first row: no row of the wave sees
    // fewer keys (rows past the end have lse2 = +inf, so their P is 0 anyway)
    const int wave_first_last =
        p.causal ? min(p.Skv - 1, (row0 + wave * 32) / p.G + delta) : p.Skv - 1;
    const int64_t qoff = (((int64_t)b * p.Sq + my_i) * p.Hq + my_h) * D;
    vec8 qf[G::KSTEPS], df[G::KSTEPS];
    float dpart[G::KSTEPS];
#pragma unroll
    for (int ks = 0; ks < G::KSTEPS; ++ks) {
        qf[ks] = __builtin_bit_cast(vec8, *(const u32x4 *)(p.q + qoff + 16 * ks + 8 * hl));
        const u32x4 dw = *(const u32x4 *)(p.dout + qoff + 16 * ks + 8 * hl);
        const u32x4 ow = *(const u32x4 *)(p.o + qoff + 16 * ks + 8 * hl);
        df[ks] = __builtin_bit_cast(vec8, dw);
        dpart[ks] = dot8<BF16>(dw, ow);
    }
    // D_i = <dO_i, o_i>: this lane's half of the row (d 16 ks + 8 hl + 0..7),
    // summed pairwise, plus the other half from lane l32 + 32 (hl = 1)
#pragma unroll
    for (int w = 1; w < G::KSTEPS; w *= 2)
#pragma unroll
        for (int ks = 0; ks + w < G::KSTEPS; ks += 2 * w) dpart[ks] += dpart[ks + w];
    const float Di = row_ok ? dpart[0] + __shfl_xor(dpart[0], 32) : 0.f;
    const int64_t rat = ((int64_t)b * p.Hq + my_h) * p.Sq + my_i;
    const float l = row_ok ? p.lse[rat] : -INFINITY;
    const float lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
    if (row_ok && hl == 0) {
        p.d_rows[rat] = Di;
        p.lse2_rows[rat] = lse2;
    }
    const float c = p.scale_log2;  // alpha log2(e), any sign

    LaneAddr<D> la;
    la.init(lane);
    f32x16 acc[G::DT];
#pragma unroll
    for (int t = 0; t < G::DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;

    // tile loads: thread chunk e of the tile -> row, 16-byte chunk
    const int64_t kv_base = ((int64_t)b * p.Skv * p.Hkv + kvh) * D;
    // key tiles fetched two ahead into two register sets (tile n in set n & 1)
    u32x4 rk[2][G::CPT], rv[2][G::CPT];
    auto fetch = [&](auto set_tag, int j0) __attribute__((always_inline)) {
        constexpr int S = decltype(set_tag)::value;
#pragma unroll
        for (int e = 0; e < G::CPT; ++e) {
            const int ch = tid + e * 64 * kBwdWaves;
            const int r = ch / (D / 8), cc = ch % (D / 8);
            const int key = min(j0 + r, p.Skv - 1);
            const int64_t off = kv_base + (int64_t)key * p.Hkv * D + 8 * cc;
            rk[S][e] = *(const u32x4 *)(p.k + off);
            rv[S][e] = *(const u32x4 *)(p.v + off);
        }
    };
    auto stash = [&](auto set_tag, int buf) __attribute__((always_inline)) {
        constexpr int S = decltype(set_tag)::value;
#pragma unroll
        for (int e = 0; e < G::CPT; ++e) {
            const int ch = tid + e * 64 * kBwdWaves;
            const int r = ch / (D / 8), cc = ch % (D / 8);
            *(u32x4 *)(&sK[buf][tile_off<D>(r, cc)]) = rk[S][e];
            *(u32x4 *)(&sV[buf][tile_off<D>(r, cc)]) = rv[S][e];
        }
    };
    auto compute = [&](int j0, int cur) __attribute__((always_inline)) {
        if (j0 > wave_last) return;
        const f32x16 s = tile_times_regs<D, BF16>(sK[cur], la, qf);   // S^T
        const f32x16 dp = tile_times_regs<D, BF16>(sV[cur], la, df);  // dP^T
        f32x16 ds;
        // dS; when every row of the wave sees all 32 keys (wave-uniform) the
        // visibility test drops out
        auto grads = [&](auto full_tag) __attribute__((always_inline)) {
            const int lim = my_last - j0 - 4 * hl;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kc = 8 * (r >> 2) + (r & 3);
                const bool vis = decltype(full_tag)::value || kc <= lim;
                const float pr = vis ? fast_exp2(__builtin_fmaf(s[r], c, -lse2)) : 0.f;
                ds[r] = pr * (dp[r] - Di);
            }
        };
        if (j0 + kBwdRows - 1 <= wave_first_last)
            grads(std::true_type{});
        else
            grads(std::false_type{});
        vec8 dsb[G::PSTEPS];
        pack_scores<BF16>(ds, dsb);
        tileT_times_packed<D, BF16>(sK[cur], la, dsb, acc);  // dQ^T += K^T dS^T
    };
    using Z = std::integral_constant<int, 0>;
    using O = std::integral_constant<int, 1>;

    if (wg_end > 0) {
        // fetches and stashes run unconditionally (past the last tile they
        // move clamped keys that nothing reads), keeping the load counts static
        fetch(Z{}, 0);
        fetch(O{}, kBwdRows);
        stash(Z{}, 0);
        __syncthreads();
        for (int j0 = 0; j0 < wg_end; j0 += 2 * kBwdRows) {
            fetch(Z{}, j0 + 2 * kBwdRows);
            compute(j0, 0);
            stash(O{}, 1);
            __syncthreads();
            if (j0 + kBwdRows >= wg_end) break;
            fetch(O{}, j0 + 3 * kBwdRows);
            compute(j0 + kBwdRows, 1);
            stash(Z{}, 0);
            __syncthreads();
        }
    }
    if (!row_ok) return;
    store_rows<D, BF16>(p.dq + qoff, acc, p.scale, hl);
}

// ---- bwd_dkdv
template <int D, bool BF16>
__global__ __launch_bounds__(64 * kBwdWaves)
__attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dkdv_kernel(const BwdParams p) {
    using G = TileGeom<D>;
    using vec8 = typename Half<BF16>::vec8;
    __shared__ __attribute__((aligned(1024))) uint8_t sQ[2][G::BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sO[2][G::BYTES];  // dO rows
    __shared__ __attribute__((aligned(16))) float sL[2][kBwdRows];      // lse2 of the rows
    __shared__ __attribute__((aligned(16))) float sD[2][kBwdRows];      // D of the rows

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int l32 = lane & 31, hl = lane >> 5;
    const int units = p.B * p.Hkv;
    const int rank = blockIdx.x / units;
    const int unit = blockIdx.x - rank * units;
    const int kblock = rank;  // key block 0 (the most rows under the causal rule) first
    const int b = unit / p.Hkv, kvh = unit - b * p.Hkv;
    const int delta = p.Skv - p.Sq;
    const int key0 = kblock * (32 * kBwdWaves);
    const int wkey0 = key0 + 32 * wave;
    const int my_key = wkey0 + l32;
    const bool key_ok = my_key < p.Skv;
    const int64_t koff = (((int64_t)b * p.Skv + min(my_key, p.Skv - 1)) * p.Hkv + kvh) * D;
    vec8 kf[G::KSTEPS], vf[G::KSTEPS];
#pragma unroll
    for (int ks = 0; ks < G::KSTEPS; ++ks) {
        kf[ks] = __builtin_bit_cast(vec8, *(const u32x4 *)(p.k + koff + 16 * ks + 8 * hl));
        vf[ks] = __builtin_bit_cast(vec8, *(const u32x4 *)(p.v + koff + 16 * ks + 8 * hl));
    }
    // packed row r (query r / G) sees key j iff j <= r / G + delta, i.e. (for
    // the causal rule) r >= (j - delta) G: this lane's first visible row
    const int my_thr = p.causal ? max(0, (my_key - delta) * p.G) : 0;
    const int wave_thr_lo = p.causal ? max(0, (wkey0 - delta) * p.G) : 0;        // first key's
    const int wave_thr_hi = p.causal ? max(0, (wkey0 + 31 - delta) * p.G) : 0;   // last key's
    const int wg_row0 = p.causal ? max(0, (key0 - delta) * p.G) / kBwdRows * kBwdRows : 0;
    const float c = p.scale_log2;

    LaneAddr<D> la;
    la.init(lane);
    f32x16 adv[G::DT], adk[G::DT];
#pragma unroll
    for (int t = 0; t < G::DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            adv[t][r] = 0.f;
            adk[t][r] = 0.f;
        }

    // Tiles are fetched two ahead into two register sets (tile n in set n & 1)
    // so that a tile's global loads have two compute steps to arrive: with one
    // wave per SIMD nothing else hides their latency.  Tiles are fetched in
    // order, so each thread keeps the (query, head-in-group) pair of its rows
    // and steps it by kBwdRows packed rows per fetch instead of dividing.
    u32x4 rq[2][G::CPT], ro[2][G::CPT];
    float rl[2], rd[2];
    bool rok[2];
    // The row tiles [wg_row0, rows) in the order of the walk: tile n starts
    // at row first_r0 + n tstep.  The grid's first wave (down_wgs workgroups,
    // one per CU, which start together) walks down from the last tile: the
    // key blocks of one (batch, KV head) -- on one XCD, as the dispatch deals
    // workgroups to the 8 XCDs in turn -- then read the same q and dO tile at
    // about the same time, and all but the first find it in L2.  Workgroups
    // that start later, one by one as earlier ones finish, walk up from their
    // first visible tile.  (Measured on the causal prefill backward: 7x fewer
    // HBM bytes than every workgroup walking up, in the same time.)
    const bool down = (int)blockIdx.x < p.down_wgs;
    const int ntiles = wg_row0 < p.rows ? (p.rows - 1 - wg_row0) / kBwdRows + 1 : 0;
    const int first_r0 = down ? wg_row0 + (ntiles - 1) * kBwdRows : wg_row0;
    const int tstep = down ? -kBwdRows : kBwdRows;
    // one tile on: tstep = step_i G + step_h with 0 <= step_h < G
    int step_i = tstep / p.G, step_h = tstep - step_i * p.G;
    if (step_h < 0) {
        step_h += p.G;
        --step_i;
    }
    int ri[G::CPT], rh[G::CPT];  // chunk e's row: query ri[e], head kvh G + rh[e]
#pragma unroll
    for (int e = 0; e < G::CPT; ++e) {
        const int r = first_r0 + (tid + e * 64 * kBwdWaves) / (D / 8);
        ri[e] = r / p.G;
        rh[e] = r - ri[e] * p.G;
    }
    int li = (first_r0 + tid) / p.G, lh = first_r0 + tid - li * p.G;  // lse / D row (tid < 32)
    const int64_t q_base = ((int64_t)b * p.Sq * p.Hq + (int64_t)kvh * p.G) * D + 8 * (tid % (D / 8));
    const int64_t l_base = ((int64_t)b * p.Hq + (int64_t)kvh * p.G) * p.Sq;
    const int hqd = p.Hq * D;
    auto advance = [&](int &i, int &h) __attribute__((always_inline)) {
        i += step_i;
        h += step_h;
        if (h >= p.G) {
            h -= p.G;
            ++i;
        }
    };
    auto fetch = [&](auto set_tag) __attribute__((always_inline)) {
        constexpr int S = decltype(set_tag)::value;
#pragma unroll
        for (int e = 0; e < G::CPT; ++e) {
            // rows past the end read the last query's row (their P is 0);
            // rows before the first are fetched only beyond a downward walk's
            // last tile, and never used
            const int64_t off =
                q_base + (int64_t)min(max(ri[e], 0), p.Sq - 1) * hqd + rh[e] * D;
            rq[S][e] = *(const u32x4 *)(p.q + off);
            ro[S][e] = *(const u32x4 *)(p.dout + off);
            advance(ri[e], rh[e]);
        }
        // every thread loads (threads past the tile's rows read a clamped row
        // they never stash), so each fetch issues the same loads and the
        // waits before a stash count exactly the fetch issued after it
        // (the padding test is applied at the stash: a select here would wait
        // for the load at once)
        const int64_t at = l_base + (int64_t)lh * p.Sq + min(max(li, 0), p.Sq - 1);
        rl[S] = p.lse2_rows[at];
        rd[S] = p.d_rows[at];
        rok[S] = li >= 0 && li < p.Sq;
        advance(li, lh);
    };
    auto stash = [&](auto set_tag, int buf) __attribute__((always_inline)) {
        constexpr int S = decltype(set_tag)::value;
#pragma unroll
        for (int e = 0; e < G::CPT; ++e) {
            const int ch = tid + e * 64 * kBwdWaves;
            const int r = ch / (D / 8), cc = ch % (D / 8);
            *(u32x4 *)(&sQ[buf][tile_off<D>(r, cc)]) = rq[S][e];
            *(u32x4 *)(&sO[buf][tile_off<D>(r, cc)]) = ro[S][e];
        }
        if (tid < kBwdRows) {
            sL[buf][tid] = rok[S] ? rl[S] : INFINITY;  // a padding row: P = 0
            sD[buf][tid] = rok[S] ? rd[S] : 0.f;
        }
    };
    auto compute = [&](int r0, int cur) __attribute__((always_inline)) {
        // rows [r0, r0 + 32): skip when none of them sees any of the wave's keys
        if (r0 + kBwdRows - 1 < wave_thr_lo) return;
        const f32x16 s = tile_times_regs<D, BF16>(sQ[cur], la, kf);   // S
        const f32x16 dp = tile_times_regs<D, BF16>(sO[cur], la, vf);  // dP
        f32x16 pr, ds;
        // P and dS; in a tile every row of which sees all the wave's keys
        // (wave-uniform) the visibility test drops out
        auto probs = [&](auto full_tag) __attribute__((always_inline)) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                // registers 4 q4 .. 4 q4 + 3 hold rows 8 q4 + 4 hl + 0..3
                const f32x4 l4 = *(const f32x4 *)(&sL[cur][8 * q4 + 4 * hl]);
                const f32x4 d4 = *(const f32x4 *)(&sD[cur][8 * q4 + 4 * hl]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * q4 + e;
                    const bool vis =
                        decltype(full_tag)::value || (r0 + 8 * q4 + 4 * hl + e >= my_thr);
                    const float x = vis ? fast_exp2(__builtin_fmaf(s[r], c, -l4[e])) : 0.f;
                    pr[r] = x;
                    ds[r] = x * (dp[r] - d4[e]);
                }
            }
        };
        if (r0 >= wave_thr_hi)
            probs(std::true_type{});
        else
            probs(std::false_type{});
        vec8 pb[G::PSTEPS], dsb[G::PSTEPS];
        pack_scores<BF16>(pr, pb);
        pack_scores<BF16>(ds, dsb);
        tileT_times_packed<D, BF16>(sO[cur], la, pb, adv);   // dV^T += dO^T P
        tileT_times_packed<D, BF16>(sQ[cur], la, dsb, adk);  // dK^T += Q^T dS
    };
    // step on tile n (in LDS buffer n & 1, rows from r0): fetch tile n + 2
    // into set n & 1, compute tile n, stash tile n + 1 from set (n + 1) & 1
    using Z = std::integral_constant<int, 0>;
    using O = std::integral_constant<int, 1>;

    if (key0 < p.Skv && ntiles > 0) {
        // fetches and stashes run unconditionally (past the last tile they
        // move clamped rows that nothing reads), keeping the load counts static
        fetch(Z{});
        fetch(O{});
        stash(Z{}, 0);
        __syncthreads();
        for (int n = 0; n < ntiles; n += 2) {
            // tile n even: set 0 is free, tile n + 1 waits in set 1
            fetch(Z{});  // tile n + 2
            compute(first_r0 + n * tstep, 0);
            stash(O{}, 1);
            __syncthreads();
            if (n + 1 >= ntiles) break;
            // tile n + 1 (odd): set 1 is free, tile n + 2 waits in set 0
            fetch(O{});  // tile n + 3
            compute(first_r0 + (n + 1) * tstep, 1);
            stash(Z{}, 0);
            __syncthreads();
        }
    }
    if (!key_ok) return;
    store_rows<D, BF16>(p.dv + koff, adv, 1.f, hl);
    store_rows<D, BF16>(p.dk + koff, adk, p.scale, hl);
}

__global__ __launch_bounds__(256) void zero_fill_kernel(u32x4 *dst, size_t n16) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n16) dst[i] = u32x4{0u, 0u, 0u, 0u};
}

template <int D, bool BF16>
hipError_t launch_d(const BwdParams &p, hipStream_t stream) {
    const int units = p.B * p.Hkv;
    hipLaunchKernelGGL((bwd_dq_kernel<D, BF16>), dim3((unsigned)(units * p.n_mblocks)),
                       dim3(64 * kBwdWaves), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int kblocks = (p.Skv + 32 * kBwdWaves - 1) / (32 * kBwdWaves);
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, BF16>), dim3((unsigned)(units * kblocks)),
                       dim3(64 * kBwdWaves), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_zero_fill(void *ptr, size_t bytes, hipStream_t stream) {
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, stream,
                       (u32x4 *)ptr, n16);
    return hipGetLastError();
}

hipError_t launch_attn_bwd(const BwdParams &p, int D, bool bf16, hipStream_t stream) {
    if (D == 64) return bf16 ? launch_d<64, true>(p, stream) : launch_d<64, false>(p, stream);
    if (D == 128) return bf16 ? launch_d<128, true>(p, stream) : launch_d<128, false>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace miattn
