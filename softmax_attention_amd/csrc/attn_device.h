// attn_device.h -- device-side helpers shared by the attention kernels of
// libmiattn (internal): vector types, the 32x32x16 MFMA per input type,
// 16-bit packing, the LDS tile swizzle and the lazy-max threshold.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace miattn {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;

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

// Four E4M3FN codes (bytes 0..3 of w) -> four 16-bit values of the MFMA type,
// packed in pairs (bytes 0, 1 and 2, 3; the lower byte in the lower half).
// Exact: every E4M3FN value is both a bf16 and an fp16 value; NaN codes give
// NaN.  (gfx950's scaled packed conversion, with scale 1.)
template <bool BF16>
__device__ __forceinline__ u32x2 fp8x4_to_half4(uint32_t w) {
    if constexpr (BF16)
        return {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, false)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, true))};
    else
        return {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, false)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, true))};
}

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
// For D = 64 a row is half the banks (row parity picks the half) and has 8
// chunk positions: bits 1, 2, 3 of the row go to bits 2, 1, 0 of the mask, so
// the 8 rows of one parity among 16 consecutive rows take 8 distinct
// positions (K reads), and rows 4m and 4m + 2 -- which a transposing read
// gathers together with their 4 chunks -- take disjoint halves of the
// positions (SQ_LDS_BANK_CONFLICT 0; the earlier mapping had every
// transposing read conflict two ways).
template <int D>
__device__ __forceinline__ int swz(int row) {
    if constexpr (D == 64)
        return (((row >> 1) & 1) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1);
    else
        return ((row & 3) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1);
}

template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk) {  // bytes
    return row * (2 * D) + 16 * (chunk ^ swz<D>(row));
}

// Word 3 of a raw buffer resource (stride 0): a 32-bit data format, without
// which gfx9 buffer loads return zeros.
constexpr int kBufferFlags = 0x00020000;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Cache-policy operand of a buffer load: the non-temporal (streaming) hint,
// for data that no other workgroup reads again.
constexpr int kLoadNonTemporal = 2;

// One buffer_load_dwordx4 ... lds: lane l copies the 16 bytes at
// base + voffset(l) to dst + 16 l, bypassing registers; offsets at or past
// num_bytes read as zero.  POLICY is the load's cache-policy operand (0 or
// kLoadNonTemporal).  (The body exists in the device pass only: the host
// pass has no buffer-resource type and would otherwise drop the kernels'
// launch stubs.)
template <int POLICY = 0>
__device__ __forceinline__ void buffer_load_lds16(const void *base, int num_bytes, lds_void *dst,
                                                  int voffset) {
#if defined(__HIP_DEVICE_COMPILE__)
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, num_bytes, kBufferFlags);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voffset, 0, 0, POLICY);
#endif
}

// max(x, x of lane l ^ 32) in every lane: v_permlane32_swap exchanges the
// two 32-lane halves without going through LDS.
__device__ __forceinline__ float max_halves(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

// x + (x of lane l ^ 32) in every lane, as above.
__device__ __forceinline__ float sum_halves(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// ---- stream-K decode plan, computed by each wave that needs it.  Batch entry
// b holds ceil(len_b / bn) key tiles, len_b = seqlen[b] clamped into
// [0, cap] (skv for every entry when seqlen is null); the (batch, KV head)
// sequences, heads fastest, form one sequence of Hkv * (sum of tiles) tiles.
// Request extents, clamped so that malformed offsets or lengths cannot
// address rows outside the tensors: packed offsets into [0, total], lengths
// into [0, the per-request maximum], paged lengths into [0, cap].
//
// The tables are read as constant memory (the kernels never write them): with
// a wave-uniform index the read goes through the scalar cache and never
// waits on the vector memory counter, which the K/V rings count on.
__device__ __forceinline__ int32_t table_at(const int32_t *t, int i) {
    return ((__attribute__((address_space(4))) const int32_t *)t)[i];
}

__device__ __forceinline__ void q_span(const SeqDesc &s, int b, int64_t &row0, int &len) {
    if (!s.cu_q) {
        row0 = (int64_t)b * s.sq;
        len = s.sq;
        return;
    }
    const int a = min(max(table_at(s.cu_q, b), 0), s.total_q);
    const int e = min(max(table_at(s.cu_q, b + 1), a), s.total_q);
    row0 = a;
    len = min(e - a, s.sq);
}

__device__ __forceinline__ int seq_kv_len(const SeqDesc &s, int b) {
    if (s.seqlen) {
        int64_t len = table_at(s.seqlen, b);
        if (s.append) {  // the chunk's own keys follow the cached ones
            int64_t row0;
            int sq_b;
            q_span(s, b, row0, sq_b);
            len += sq_b;
        }
        return (int)min(max(len, (int64_t)0), (int64_t)s.cap);
    }
    if (!s.cu_kv) return s.skv;
    const int a = min(max(table_at(s.cu_kv, b), 0), s.total_kv);
    const int e = min(max(table_at(s.cu_kv, b + 1), a), s.total_kv);
    return min(e - a, s.skv);
}

// first key row of request b in a dense (possibly packed) K/V tensor
__device__ __forceinline__ int64_t seq_kv_row0(const SeqDesc &s, int b) {
    return s.cu_kv ? (int64_t)min(max(table_at(s.cu_kv, b), 0), s.total_kv) : (int64_t)b * s.skv;
}

// Stream-K plan over the key tiles of all requests.
struct SkBatch {
    SeqDesc sd;
    int bn;        // keys per tile
    int win_left;  // left window bound (-1: none)
    int piece;     // plan weight of starting a piece, in tiles (see sk_weight)
};

// first key tile any query of request b (sq_b queries, len keys) can see:
// with a left window the first query (at position len - sq_b) sees keys from
// len - sq_b - w_L on
__device__ __forceinline__ int sk_first_tile(const SkBatch &s, int len, int sq_b) {
    return s.win_left < 0 ? 0 : max(0, len - sq_b - s.win_left) / s.bn;
}

// key tiles of request b (none when it has no query)
__device__ __forceinline__ int sk_tiles(const SkBatch &s, int b) {
    int64_t row0;
    int sq_b;
    q_span(s.sd, b, row0, sq_b);
    if (sq_b == 0) return 0;
    const int len = seq_kv_len(s.sd, b);
    return (len + s.bn - 1) / s.bn - sk_first_tile(s, len, sq_b);
}

// Plan weight of each (request, KV head) unit: its key tiles plus `piece`
// for the cost of starting a piece of it (the page-table and first-tile
// round trips before the unit's first tile lands, the partial store after its
// last); none for a unit without tiles.  The unit's tiles sit at weight
// offsets [piece, piece + tiles), so the workgroups' equal shares of the
// weight give a workgroup that starts more pieces fewer tiles.
__device__ __forceinline__ int sk_weight(const SkBatch &s, int tiles) {
    return tiles > 0 ? tiles + s.piece : 0;
}

// inclusive prefix sum over the 64 lanes of a wave, with DPP moves (no LDS
// round trips): shifts by 1, 2, 4 and 8 lanes within each row of 16 (a lane
// whose source lies outside its row adds 0), then row 0's total into row 1
// and row 2's into row 3 (row_bcast:15), then the total of rows 0-1 into
// rows 2 and 3 (row_bcast:31)
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// plan weight of the whole batch (returned) and of the entries before `upto`
__device__ __forceinline__ int sk_sums(const SkBatch &s, int upto, int &before) {
    const int lane = threadIdx.x & 63;
    int total = 0, pre = 0;
    for (int c = 0; c < s.sd.B; c += 64) {
        const int b = c + lane;
        const int t = b < s.sd.B ? sk_weight(s, sk_tiles(s, b)) : 0;
        const int incl = wave_incl_scan(t);
        const int incl_before = wave_incl_scan(b < upto ? t : 0);
        total += __shfl(incl, 63);
        pre += __shfl(incl_before, 63);
    }
    // (wave-uniform values: scalar registers, so that addresses built from
    // them stay scalar -- a buffer descriptor in vector registers costs a
    // waterfall loop per load)
    before = __builtin_amdgcn_readfirstlane(pre);
    return __builtin_amdgcn_readfirstlane(total);
}

// the entry b whose weight holds position `at` of the sequence (hkv * pre_b <=
// at < hkv * (pre_b + t_b)), with pre_b (weight before it) and its weight t_b;
// `at` must be below the sequence's length
__device__ __forceinline__ void sk_find(const SkBatch &s, int hkv, int64_t at, int &b_out,
                                        int &pre_out, int &t_out) {
    const int lane = threadIdx.x & 63;
    int carry = 0;
    for (int c = 0; c < s.sd.B; c += 64) {
        const int b = c + lane;
        const int t = b < s.sd.B ? sk_weight(s, sk_tiles(s, b)) : 0;
        const int incl = carry + wave_incl_scan(t);
        const int excl = incl - t;
        const bool hit = b < s.sd.B && (int64_t)hkv * excl <= at && at < (int64_t)hkv * incl;
        const uint64_t m = __ballot(hit);
        if (m) {
            const int src = __builtin_ctzll(m);
            b_out = __builtin_amdgcn_readfirstlane(c + src);
            pre_out = __builtin_amdgcn_readfirstlane(__shfl(excl, src));
            t_out = __builtin_amdgcn_readfirstlane(__shfl(t, src));
            return;
        }
        carry = __shfl(incl, 63);
    }
    b_out = s.sd.B;
    pre_out = __builtin_amdgcn_readfirstlane(carry);
    t_out = 0;
}

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

// Unmasked tiles take their exponentials against the running max without
// forming their own max first; the max is formed (and the running max
// raised) only for a tile in which some lane's sum of exponentials exceeds
// this (so that every P <= 2^24, which keeps l and the FP32 output sums far
// from overflow for any |V| up to 2^70).
constexpr float kFastSum = 16777216.0f;  // 2^24

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// in bits 6:4, lgkmcnt in bits 11:8; a field at its maximum does not wait).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);

// Waits are issued through the s_waitcnt builtin rather than inline assembly
// because the compiler tracks which LDS array each direct-to-LDS load writes
// and inserts a wait of its own before any LDS read that might still be in
// flight; an assembly wait is opaque to it, so it would drain the whole ring
// (vmcnt(0)) before reads that the counted waits already cover.  The empty
// assembly statements keep memory accesses from moving across the wait.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(N));
    asm volatile("" ::: "memory");
}

// Workgroup barrier for the K/V rings.  __syncthreads() is a workgroup-scope
// release/acquire fence around s_barrier, and the release half waits for every
// outstanding global load (vmcnt(0)) -- which would drain the whole ring at
// each barrier.  The rings order their loads with explicit, counted vmcnt
// waits instead; the barrier itself only needs this wave's LDS reads done
// (so a stage can be refilled) and must keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void ring_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace dev
}  // namespace miattn
