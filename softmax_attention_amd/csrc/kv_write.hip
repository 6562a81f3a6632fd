// kv_write.hip -- scatter new K/V rows into paged KV-cache pools.
//
// TileOPs "Attention Operators", PagedKVCacheWriteFwdOp: token n's key and
// value rows ([Hkv, D]) go to the pool row its slot names (page * page_size +
// offset, -1 skipping the token); a 16-bit pool stores the rows as they are,
// an FP8 pool stores row / scale as E4M3FN with NaN preserved and finite
// overflow and infinities saturated to +-448.  For GQAPrefillPagedWithKVCache
// FwdOp the slots follow from the request layout instead: the packed chunk's
// token i of request b goes to logical position cache_seqlens[b] + i, i.e. pool
// row block_table[b, pos / page_size] * page_size + pos % page_size.
//
// One thread moves one 16-byte chunk (8 elements) of one token's K row and of
// its V row; consecutive threads take consecutive chunks of a row, so both the
// reads and the pool writes are contiguous per row.  HBM-bound.
#include "attn_kernels.h"

#include "attn_device.h"

namespace miattn {
namespace {

using namespace dev;

// E4M3FN code of a float (1 sign, 4 exponent bits with bias 7, 3 fraction
// bits; no infinities, S.1111.111 is NaN, largest finite 448), rounding to
// nearest with ties to the even code, written from the format's bit layout.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const uint32_t sign = (u >> 24) & 0x80u;
    if (x != x) return sign | 0x7fu;             // NaN stays NaN
    const float a = __builtin_fabsf(x);
    if (a >= 448.f) return sign | 0x7eu;         // saturate (infinities included)
    if (a < 0.015625f) {                         // below 2^-6: multiples of 2^-9
        // a * 512 is exact; rint rounds half to even; 8 gives code 0x08 = 2^-6
        return sign | (uint32_t)__builtin_rintf(a * 512.f);
    }
    const uint32_t ua = __builtin_bit_cast(uint32_t, a);
    int e = (int)(ua >> 23) - 127;               // -6 .. 8
    uint32_t keep = (ua >> 20) & 7u;             // the 3 fraction bits kept
    const uint32_t rest = ua & 0xfffffu;         // the 20 dropped
    if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
    if (keep == 8u) {
        keep = 0u;
        ++e;
    }
    return sign | ((uint32_t)(e + 7) << 3) | keep;  // a < 448 keeps this finite
}

template <bool BF16>
__device__ __forceinline__ float half_to_float(uint32_t bits16) {
    if constexpr (BF16)
        return __builtin_bit_cast(float, bits16 << 16);
    else
        return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// Slot of packed chunk token n in append mode (-1 when the metadata puts it
// outside the table or the pool): its request b is found by bisection over
// cu_q, which is clamped and made nondecreasing on the way.
__device__ __forceinline__ int64_t append_slot(const KvWriteParams &p, int n) {
    int lo = 0, hi = p.B;  // find the last b with cu_q[b] <= n
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.cu_q[mid] <= n) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int64_t pos = (int64_t)p.cache_seqlens[b] + (n - p.cu_q[b]);
    if (pos < 0 || pos >= (int64_t)p.max_pages * p.page_size || n >= p.cu_q[b + 1]) return -1;
    const int32_t page = p.block_table[(int64_t)b * p.max_pages + pos / p.page_size];
    if (page < 0 || (int64_t)page * p.page_size >= p.num_slots) return -1;
    return (int64_t)page * p.page_size + pos % p.page_size;
}

template <bool BF16, bool FP8, bool APPEND>
__global__ __launch_bounds__(256) void kv_write_kernel(const KvWriteParams p) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int chunks = p.row_elems / 8;  // 16-byte chunks of one input row
    const int n = (int)(gid / chunks);
    if (n >= p.tokens) return;
    const int c = (int)(gid - (int64_t)n * chunks);
    int64_t slot;
    if constexpr (APPEND)
        slot = append_slot(p, n);
    else
        slot = p.slot_mapping[n];
    if (slot < 0 || slot >= p.num_slots) return;  // skipped (or outside the pool)
    const int64_t src = (int64_t)n * p.row_elems + 8 * c;
    const int64_t dst = slot * p.row_elems + 8 * c;
    const u32x4 kv = *(const u32x4 *)(p.k + src);
    const u32x4 vv = *(const u32x4 *)(p.v + src);
    if constexpr (!FP8) {
        *(u32x4 *)(p.k_pool16 + dst) = kv;
        *(u32x4 *)(p.v_pool16 + dst) = vv;
    } else {
        // the pages divide by the scale (in float32, correctly rounded)
        const float ks = *p.k_scale, vs = *p.v_scale;
        u32x2 ko, vo;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            uint32_t kw = 0u, vw = 0u;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t word_k = kv[2 * w + e / 2], word_v = vv[2 * w + e / 2];
                const uint32_t hk = (e & 1) ? word_k >> 16 : word_k & 0xffffu;
                const uint32_t hv = (e & 1) ? word_v >> 16 : word_v & 0xffffu;
                kw |= e4m3_encode(__fdiv_rn(half_to_float<BF16>(hk), ks)) << (8 * e);
                vw |= e4m3_encode(__fdiv_rn(half_to_float<BF16>(hv), vs)) << (8 * e);
            }
            ko[w] = kw;
            vo[w] = vw;
        }
        *(u32x2 *)(p.k_pool8 + dst) = ko;
        *(u32x2 *)(p.v_pool8 + dst) = vo;
    }
}

template <bool BF16, bool FP8, bool APPEND>
hipError_t launch_one(const KvWriteParams &p, hipStream_t stream) {
    const int64_t threads = (int64_t)p.tokens * (p.row_elems / 8);
    const int64_t grid = (threads + 255) / 256;
    hipLaunchKernelGGL((kv_write_kernel<BF16, FP8, APPEND>), dim3((unsigned)grid), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dt(const KvWriteParams &p, bool fp8, bool append, hipStream_t stream) {
    if (fp8) return append ? launch_one<BF16, true, true>(p, stream)
                           : launch_one<BF16, true, false>(p, stream);
    return append ? launch_one<BF16, false, true>(p, stream)
                  : launch_one<BF16, false, false>(p, stream);
}

}  // namespace

hipError_t launch_kv_write(const KvWriteParams &p, bool bf16, bool fp8, bool append,
                           hipStream_t stream) {
    if (p.tokens <= 0) return hipSuccess;
    return bf16 ? launch_dt<true>(p, fp8, append, stream) : launch_dt<false>(p, fp8, append, stream);
}

}  // namespace miattn
