// miattn.hip -- the C ABI of libmiattn: argument validation, launch planning,
// the split-KV workspace and kernel timing.  The kernels live in attn_fwd.hip
// and lse_merge.hip; see include/miattn.h for the contract.
#include "miattn.h"

#include <limits.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <utility>
#include <vector>

#include "attn_kernels.h"

using miattn::FwdParams;
using miattn::MergeParams;

namespace miattn {

hipError_t launch_attn_fwd(const FwdParams &p, int D, bool bf16, bool paged, int waves,
                           bool cap, int grid, hipStream_t stream) {
    switch (D * 2 + (cap ? 1 : 0)) {
        case 128: return launch_attn_fwd_dc<64, false>(p, bf16, paged, waves, grid, stream);
        case 129: return launch_attn_fwd_dc<64, true>(p, bf16, paged, waves, grid, stream);
        case 256: return launch_attn_fwd_dc<128, false>(p, bf16, paged, waves, grid, stream);
        case 257: return launch_attn_fwd_dc<128, true>(p, bf16, paged, waves, grid, stream);
        case 512: return launch_attn_fwd_dc<256, false>(p, bf16, paged, waves, grid, stream);
        case 513: return launch_attn_fwd_dc<256, true>(p, bf16, paged, waves, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

int attn_fwd_decode_blocks_per_cu(const FwdParams &p, int D, bool bf16, bool paged, int waves,
                                  bool cap) {
    switch (D * 2 + (cap ? 1 : 0)) {
        case 128: return decode_blocks_per_cu_dc<64, false>(p, bf16, paged, waves);
        case 129: return decode_blocks_per_cu_dc<64, true>(p, bf16, paged, waves);
        case 256: return decode_blocks_per_cu_dc<128, false>(p, bf16, paged, waves);
        case 257: return decode_blocks_per_cu_dc<128, true>(p, bf16, paged, waves);
        default: return 0;
    }
}

}  // namespace miattn

namespace {

thread_local char g_err[512] = "";

miattn_status fail(miattn_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

miattn_status hip_fail(hipError_t e, const char *what) {
    return fail(MIATTN_ERR_HIP, "%s failed: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// ---------------------------------------------------------------- device state

constexpr int kMaxDevices = 64;

// The split-KV workspace of one device.  It grows by allocating a larger
// buffer; the old one is retired, not freed, because a HIP graph captured
// earlier may still name it in its kernel nodes.  Retired buffers are freed
// only by miattn_release_workspace().  Calls on different streams are
// ordered on the device: a call on another stream than the workspace's last
// user first waits for an event recorded behind that use (not under stream
// capture, where the caller orders graph replays).
struct DeviceState {
    void *ws = nullptr;  // split-KV partials
    size_t ws_bytes = 0;
    std::vector<void *> retired;
    hipStream_t last_stream = nullptr;  // last (non-capturing) stream that used ws
    hipEvent_t last_use = nullptr;      // recorded on last_stream after that use
    bool used = false;
    int cus = 0;
    // decode kernel occupancy: [D 128][bf16][paged][capped logits][16-bit, FP8 pools, paired,
    // paired over FP8 pools]
    int decode_per_cu[2][2][2][2][4] = {};
};

std::mutex g_mu;
DeviceState g_dev[kMaxDevices];
int g_split_keys = 0;  // 0 = automatic
constexpr int kSkPieceMax = 64;  // largest stream-K piece weight, in key tiles
// A piece of a stream-K unit that starts mid-kernel waits ~10 us for its
// page-table entry and first tile (measured with in-kernel timestamps), about
// six tiles' worth of streaming: the plan weighs each piece that much, so a
// workgroup that starts more pieces gets fewer tiles.
constexpr int kSkPieceDefault = 6;
// Fewest key tiles a planned (not forced) split of a prefill-shaped call holds.
constexpr int64_t kMinSplitTiles = 8;
int g_sk_piece = kSkPieceDefault;

int compute_units(int dev) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_dev[dev].cus == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        g_dev[dev].cus = n;
    }
    return g_dev[dev].cus;
}

// Decode workgroups one CU runs at once (occupancy API, cached).
int decode_per_cu(int dev, const miattn::FwdParams &p, int D, bool bf16, bool paged, bool cap,
                  int waves) {
    std::lock_guard<std::mutex> lock(g_mu);
    const int variant =
        (waves == miattn::kPairWaves ? 2 : 0) + (p.k_scale != nullptr ? 1 : 0);
    int &slot = g_dev[dev].decode_per_cu[D == 128][bf16][paged][cap][variant];
    if (slot == 0) {
        const int n = miattn::attn_fwd_decode_blocks_per_cu(p, D, bf16, paged, waves, cap);
        slot = n > 0 ? n : -1;
    }
    return slot > 0 ? slot : 1;
}

bool capturing(hipStream_t stream) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(stream, &st) == hipSuccess && st != hipStreamCaptureStatusNone;
}

// The workspace for a call on `stream`, at least `bytes` large; the call's
// kernels must then be followed by workspace_done(dev, stream).
miattn_status workspace(int dev, hipStream_t stream, size_t bytes, void **out) {
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceState &d = g_dev[dev];
    const bool cap = capturing(stream);
    if (d.ws_bytes < bytes) {
        if (cap)
            return fail(MIATTN_ERR_INVALID_ARG,
                        "the split-KV workspace must grow to %zu bytes, which cannot happen "
                        "under stream capture: run the call once before capturing it",
                        bytes);
        // grow with headroom so that a slightly larger call does not reallocate
        const size_t want = bytes + bytes / 4;
        void *fresh = nullptr;
        hipError_t e = hipMalloc(&fresh, want);
        if (e != hipSuccess) return hip_fail(e, "hipMalloc(split-KV workspace)");
        if (d.ws) d.retired.push_back(d.ws);
        d.ws = fresh;
        d.ws_bytes = want;
    }
    if (!cap && d.used && d.last_stream != stream) {
        // the previous user ran on another stream: order this call after it
        hipError_t e = hipStreamWaitEvent(stream, d.last_use, 0);
        if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent(workspace)");
    }
    *out = d.ws;
    return MIATTN_OK;
}

miattn_status workspace_done(int dev, hipStream_t stream) {
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceState &d = g_dev[dev];
    if (capturing(stream)) return MIATTN_OK;
    hipError_t e = hipSuccess;
    if (!d.last_use) e = hipEventCreateWithFlags(&d.last_use, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(d.last_use, stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord(workspace)");
    d.last_stream = stream;
    d.used = true;
    return MIATTN_OK;
}

// ---------------------------------------------------------------- fixed scratch

// Scratch of the allocation-free entry point (attn_fwd_paged_noalloc): the
// split-KV partials live in this file-scope device array instead of the
// workspace.  Every GPU the library runs on holds its own copy until the
// process ends.  Host code never uses the array's name as an address (on the
// host it is only a stand-in): the device address of each GPU's copy comes
// from hipGetSymbolAddress, looked up once per device with that device
// current, and only that address reaches the kernels.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

void *g_scratch_addr[kMaxDevices] = {};

miattn_status scratch_address(int dev, void **out) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch_addr[dev]) {
        void *ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(MIATTN_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_addr[dev] = ptr;
    }
    *out = g_scratch_addr[dev];
    return MIATTN_OK;
}

// Where a call's split-KV partials go: the library workspace (grown on
// demand), or the fixed scratch of this device (no allocation; a call that
// would need more is refused).
struct PartialsSource {
    bool fixed = false;
};

miattn_status partials(const PartialsSource &src, int dev, hipStream_t stream, size_t bytes,
                       void **out) {
    if (!src.fixed) return workspace(dev, stream, bytes, out);
    if (bytes > kScratchBytes)
        return fail(MIATTN_ERR_UNSUPPORTED,
                    "the call needs %zu bytes of split-KV scratch; the allocation-free entry "
                    "point holds at most %zu",
                    bytes, kScratchBytes);
    return scratch_address(dev, out);
}

miattn_status partials_done(const PartialsSource &src, int dev, hipStream_t stream) {
    return src.fixed ? MIATTN_OK : workspace_done(dev, stream);
}

// ---------------------------------------------------------------- timing

struct Timing {
    bool on = false;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> ev[2];  // [0] attention, [1] merge
};
std::mutex g_prof_mu;
Timing g_prof;

bool profiling() {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    return g_prof.on;
}

template <class Launch>
hipError_t timed_launch(int kind, hipStream_t stream, Launch &&launch) {
    if (!profiling()) return launch();
    hipEvent_t a, b;
    hipError_t e = hipEventCreate(&a);
    if (e != hipSuccess) return e;
    e = hipEventCreate(&b);
    if (e != hipSuccess) return e;
    (void)hipEventRecord(a, stream);
    e = launch();
    (void)hipEventRecord(b, stream);
    std::lock_guard<std::mutex> lock(g_prof_mu);
    g_prof.ev[kind].push_back({a, b});
    return e;
}

// ---------------------------------------------------------------- checks

miattn_status check_common(const void *q, const void *o, float *lse, int B, int Sq, int Hq,
                           int Hkv, int D, float scale, miattn_dtype dtype) {
    if (B < 0 || Sq < 0)
        return fail(MIATTN_ERR_INVALID_ARG, "negative dimension: B=%d Sq=%d", B, Sq);
    if (Hq <= 0 || Hkv <= 0)
        return fail(MIATTN_ERR_INVALID_ARG, "head counts must be positive: Hq=%d Hkv=%d", Hq,
                    Hkv);
    if (D <= 0) return fail(MIATTN_ERR_INVALID_ARG, "D=%d must be positive", D);
    if (Hq % Hkv != 0)
        return fail(MIATTN_ERR_INVALID_ARG, "Hq (%d) not divisible by Hkv (%d)", Hq, Hkv);
    if (D != 64 && D != 128 && D != 256)
        return fail(MIATTN_ERR_UNSUPPORTED, "D=%d unsupported (64, 128, 256)", D);
    if (dtype != MIATTN_BF16 && dtype != MIATTN_FP16)
        return fail(MIATTN_ERR_UNSUPPORTED, "dtype %d unsupported (MIATTN_BF16, MIATTN_FP16)",
                    (int)dtype);
    if (isinf(scale)) return fail(MIATTN_ERR_INVALID_ARG, "scale must be finite (or NaN for 1/sqrt(D))");
    if ((int64_t)Sq * (Hq / Hkv) > INT_MAX / 2)
        return fail(MIATTN_ERR_UNSUPPORTED, "Sq*Hq/Hkv = %lld exceeds %d packed rows",
                    (long long)Sq * (Hq / Hkv), INT_MAX / 2);
    if (B == 0 || Sq == 0) return MIATTN_OK;
    if (!q || !o) return fail(MIATTN_ERR_INVALID_ARG, "q and o must not be NULL");
    if (!aligned16(q)) return fail(MIATTN_ERR_INVALID_ARG, "q not 16-byte aligned");
    if (!aligned16(o)) return fail(MIATTN_ERR_INVALID_ARG, "o not 16-byte aligned");
    if (lse && ((uintptr_t)lse & 3u))
        return fail(MIATTN_ERR_INVALID_ARG, "lse not 4-byte aligned");
    return MIATTN_OK;
}

float resolve_scale(float scale, int D) {
    return isnan(scale) ? (float)(1.0 / sqrt((double)D)) : scale;
}

// The kernels take exp2 of scores scaled by a positive factor c = |alpha|
// log2(e).  A negative alpha is applied by negating q inside the kernel (an
// exact sign flip); alpha == 0 makes every visible score equal, which the
// kernel reproduces exactly by zeroing q (and using c = 1).
void set_scale(FwdParams &p, float alpha) {
    if (alpha == 0.f) {
        p.q_mode = 2;
        p.scale_log2 = 1.f;
    } else {
        p.q_mode = alpha < 0.f ? 1 : 0;
        p.scale_log2 = fabsf(alpha) * 1.4426950408889634f;
    }
}

// Sliding window and logit softcap (TileOPs "Attention Operators",
// GQADenseFwdOp stages 5 and 6; the init parameters: -1 = an unlimited window
// side, a cap of 0 disables capping, a negative cap is an error).  max_len is
// the longest key range a request can have.  A bound that cannot exclude any
// key becomes -1, which also keeps p_i + w_R within int range in the kernel.
miattn_status check_window_softcap(int window_left, int window_right, float softcap) {
    if (window_left < -1 || window_right < -1)
        return fail(MIATTN_ERR_INVALID_ARG,
                    "window_left=%d, window_right=%d: each must be -1 (unlimited) or >= 0",
                    window_left, window_right);
    if (!(softcap >= 0.f) || isinf(softcap))
        return fail(MIATTN_ERR_INVALID_ARG, "softcap must be 0 (none) or positive and finite");
    return MIATTN_OK;
}

miattn_status set_window_softcap(FwdParams &p, int window_left, int window_right,
                                 float softcap, int64_t max_len, float alpha) {
    // p_i lies in [-Sq, max_len - 1]: w_L >= max_len admits every key j >= 0,
    // w_R >= max_len + Sq every key j < max_len
    p.win_left = (window_left >= 0 && window_left < max_len) ? window_left : -1;
    p.win_right =
        (window_right >= 0 && window_right < max_len + p.Sq) ? window_right : -1;
    if (p.win_right >= 0 && 2 * max_len + p.Sq > INT_MAX)
        return fail(MIATTN_ERR_UNSUPPORTED,
                    "a right window needs 2 * keys + Sq <= %d (keys = %lld, Sq = %d)", INT_MAX,
                    (long long)max_len, p.Sq);
    p.cap_x = 0.f;
    p.cap_k2 = 0.f;
    if (softcap > 0.f) {
        const double l2e = 1.4426950408889634;
        p.cap_x = (float)(2.0 * l2e * fabs((double)alpha) / (double)softcap);
        p.cap_k2 = (float)((double)softcap * l2e);
    }
    return MIATTN_OK;
}

int env_int(const char *name, int dflt) {
    const char *s = getenv(name);
    if (!s || !*s) return dflt;
    return atoi(s);
}

// ---------------------------------------------------------------- plan + launch

// What the merge kernel needs of a call: its extents (as the attention kernel
// clamps them), the partials' layout and the sinks.
MergeParams merge_params(const FwdParams &p, bool paged) {
    MergeParams m = {};
    m.o_part = p.o_part;
    m.lse_part = p.lse_part;
    m.o = p.o;
    m.lse = p.lse;
    m.seqlen = paged ? p.seqlen : nullptr;
    m.cu_q = p.cu_q;
    m.cu_kv = paged ? nullptr : p.cu_kv;
    m.sinks = p.sinks;
    m.total_q = p.total_q;
    m.total_kv = p.total_kv;
    m.kv_append = p.kv_append;
    m.Skv = p.Skv;
    m.B = p.B;
    m.Sq = p.Sq;
    m.Hq = p.Hq;
    m.Hkv = p.Hkv;
    m.G = p.G;
    m.rows = p.rows;
    m.n_splits = p.n_splits;
    m.split_len = p.split_len;
    m.sk_cap = (paged && p.num_pages > 0) ? (p.max_pages << p.page_shift) : 0;
    m.sk_win_left = -1;
    m.sk_hpw = 1;
    return m;
}

miattn_status run(FwdParams p, int D, bool bf16, bool paged, int64_t capacity, bool cap,
                  hipStream_t stream, const PartialsSource &src = PartialsSource()) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MIATTN_ERR_UNSUPPORTED, "device %d", dev);

    p.G = p.Hq / p.Hkv;
    p.rows = p.Sq * p.G;
    // D <= 128: the 8-wave ping-pong schedule for prefill (at D = 64 over dense
    // K/V the 4-wave streaming schedule instead), a three-wave streaming
    // workgroup (one computing, two loading) for decode-shaped calls (all
    // packed rows in one MFMA column block) and for FP8 pools (there one
    // loading and two converting waves; decode-shaped calls may pair heads,
    // below); D = 256: the 4-wave streaming schedule.
    int waves = D == 256 ? 4 : (p.rows > miattn::kRowsPerWave ? ((D == 64 && !paged) ? 4 : 8) : 3);
    if (p.k_scale != nullptr) waves = 3;
    const int split_keys = g_split_keys > 0 ? g_split_keys : env_int("MIATTN_SPLIT_KEYS", 0);
    // Decode-shaped calls with an even number of KV heads run the paired
    // schedule (stream-K only): one workgroup reads both heads' rows of each
    // key as one contiguous segment (512 bytes at D = 128, 256 over FP8
    // pools), which streams faster than two segments read by two workgroups.
    auto streamk_fits = [&](int w) {
        const int64_t bn = miattn::keys_per_tile(D, w, p.k_scale != nullptr);
        const int64_t ct = capacity > 0 ? (capacity + bn - 1) / bn : 1;
        return (int64_t)p.B * (ct + kSkPieceMax) < INT_MAX;
    };
    if (waves == 3 && p.Hkv % 2 == 0 && D <= 128 &&
        p.rows <= miattn::kRowsPerWave && split_keys <= 0 && streamk_fits(miattn::kPairWaves))
        waves = miattn::kPairWaves;
    const int BN = miattn::keys_per_tile(D, waves, p.k_scale != nullptr);
    const int BM = miattn::rows_per_workgroup(waves);
    p.n_mblocks = (p.rows + BM - 1) / BM;
    const int64_t bhs = (int64_t)p.B * p.Hkv;
    const int64_t cap_tiles = capacity > 0 ? (capacity + BN - 1) / BN : 1;
    p.sk_grid = 0;

    // Decode-shaped calls run stream-K: a grid of what the GPU holds at once,
    // each workgroup an equal share of the plan weight of one KV head's
    // (request) units -- their key tiles plus a cost per piece -- so no
    // workgroup waits on a long request or for a dispatch slot.  A forced
    // split length selects the split plan below instead.  (The plan's sums
    // are 32-bit: B * the weight of a unit at the capacity.)
    if (waves == miattn::kPairWaves ||
        (waves == 3 && p.rows <= miattn::kRowsPerWave && split_keys <= 0 &&
         (int64_t)p.B * (cap_tiles + kSkPieceMax) < INT_MAX)) {
        const int per_cu = decode_per_cu(dev, p, D, bf16, paged, cap, waves);
        // whole groups of U workgroups: workgroup g serves head unit g % U (a
        // KV head, or a pair of them)
        const int hpw = waves == miattn::kPairWaves ? 2 : 1;
        const int U = p.Hkv / hpw;
        const int G = std::max(1, compute_units(dev) * per_cu / U) * U;
        p.n_mblocks = 1;
        p.n_splits = 1;
        p.split_len = 0;
        p.xcd_units = 0;
        p.heads_inner = 0;
        // partial slot of (KV head h, request b, share c): h (B + G / U) + b + c
        const int64_t slots = bhs + (int64_t)G * hpw;
        void *ws = nullptr;
        miattn_status st =
            partials(src, dev, stream, (size_t)slots * p.rows * (D + 1) * sizeof(float), &ws);
        if (st != MIATTN_OK) return st;
        p.o_part = (float *)ws;
        p.lse_part = p.o_part + slots * p.rows * D;
        p.sk_grid = G;
        p.sk_piece = g_sk_piece;
        e = timed_launch(0, stream, [&] {
            return miattn::launch_attn_fwd(p, D, bf16, paged, waves, cap, G, stream);
        });
        if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
        MergeParams m = merge_params(p, paged);
        m.sk_grid = G;
        m.sk_bn = BN;
        m.sk_win_left = p.win_left;
        m.sk_piece = p.sk_piece;
        m.sk_hpw = hpw;
        e = timed_launch(1, stream, [&] { return miattn::launch_lse_merge(m, D, bf16, stream); });
        if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
        return partials_done(src, dev, stream);
    }

    // Split the key axis when the (row block, batch, KV head) units alone
    // cannot fill the chip, or for decode-shaped calls, whose per-request
    // lengths vary and are only known on the device.
    // With a left window a row block sees at most w_L + its own query span
    // (+ w_R without the causal rule) keys: size the splits for that span.
    int64_t span_tiles = cap_tiles;
    if (p.win_left >= 0) {
        int64_t span = (int64_t)p.win_left + (BM + p.G - 1) / p.G + 1;
        if (!p.causal) span += p.win_right >= 0 ? (int64_t)p.win_right : capacity;
        span_tiles = std::min(cap_tiles, (span + BN - 1) / BN + 1);
    }
    int64_t tiles_per;
    if (split_keys > 0) {
        tiles_per = (split_keys + BN - 1) / BN;
    } else {
        const int64_t units0 = (int64_t)p.n_mblocks * bhs;
        const int cus = compute_units(dev);
        if (p.n_mblocks == 1 && p.rows <= miattn::kRowsPerWave) {
            tiles_per = (512 + BN - 1) / BN;  // 512-key splits
        } else if (units0 >= 2 * (int64_t)cus) {
            tiles_per = cap_tiles;
        } else {
            const int64_t want = (3 * (int64_t)cus + units0 - 1) / units0;
            tiles_per = (span_tiles + want - 1) / want;
        }
    }
    // (a planned split holds at least kMinSplitTiles key tiles: shorter ones
    // cost more in partial stores and the merge launch than they balance)
    if (split_keys <= 0 && tiles_per < kMinSplitTiles) tiles_per = kMinSplitTiles;
    if (tiles_per < 1) tiles_per = 1;
    if (tiles_per > cap_tiles) tiles_per = cap_tiles;
    const int64_t n_splits = (cap_tiles + tiles_per - 1) / tiles_per;
    p.n_splits = (int)n_splits;
    p.split_len = (int)(tiles_per * BN);
    if (n_splits == 1) p.split_len = (int)(cap_tiles * BN);

    const int64_t grid = (int64_t)p.n_mblocks * bhs * n_splits;
    if (grid > INT_MAX)
        return fail(MIATTN_ERR_UNSUPPORTED, "launch of %lld workgroups exceeds %d",
                    (long long)grid, INT_MAX);
    const int64_t units = bhs * n_splits;
    p.xcd_units = (units % 8 == 0) ? (int)(units / 8) : 0;
    // split decode: the KV heads of one key range run side by side
    p.heads_inner = (n_splits > 1 && p.n_mblocks == 1) ? 1 : 0;

    if (n_splits > 1) {
        const int64_t nrow = n_splits * bhs * p.rows;
        void *ws = nullptr;
        miattn_status st = partials(src, dev, stream, (size_t)nrow * (D + 1) * sizeof(float), &ws);
        if (st != MIATTN_OK) return st;
        p.o_part = (float *)ws;
        p.lse_part = p.o_part + nrow * D;
    }

    e = timed_launch(0, stream, [&] {
        return miattn::launch_attn_fwd(p, D, bf16, paged, waves, cap, (int)grid, stream);
    });
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch");

    if (n_splits > 1) {
        MergeParams m = merge_params(p, paged);
        e = timed_launch(1, stream, [&] { return miattn::launch_lse_merge(m, D, bf16, stream); });
        if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
        return partials_done(src, dev, stream);
    }
    return MIATTN_OK;
}

}  // namespace

extern "C" {

const char *miattn_last_error(void) { return g_err; }

}  // extern "C"

namespace {

// Packed offsets (MIATTN_VALIDATE=1 only; synchronises the stream): cu[0] = 0,
// nondecreasing, cu[B] = total, and no request longer than max_len.
miattn_status validate_offsets(const int32_t *cu, int B, int total, int max_len,
                               const char *name, hipStream_t s) {
    std::vector<int32_t> h((size_t)B + 1);
    hipError_t e = hipMemcpyAsync(h.data(), cu, sizeof(int32_t) * h.size(),
                                  hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "MIATTN_VALIDATE offsets copy");
    if (h[0] != 0 || h[B] != total)
        return fail(MIATTN_ERR_INVALID_ARG, "%s must start at 0 and end at %d (got %d .. %d)",
                    name, total, h[0], h[B]);
    for (int b = 0; b < B; ++b)
        if (h[b + 1] < h[b] || h[b + 1] - h[b] > max_len)
            return fail(MIATTN_ERR_INVALID_ARG,
                        "%s[%d..%d] = %d..%d: a request must hold 0..%d rows", name, b, b + 1,
                        h[b], h[b + 1], max_len);
    return MIATTN_OK;
}

// The dense call, uniform (cu_q == NULL: B blocks of Sq queries and Skv keys)
// or packed (THD: Sq and Skv are the per-request maxima, cu_q / cu_kv the
// request offsets, lse [Hq, total_q]).
miattn_status dense_call(const void *q, const void *k, const void *v, int B, int Hq, int Hkv,
                         int Sq, int Skv, int D, float scale, int causal, int window_left,
                         int window_right, float softcap, const uint8_t *key_padding_mask,
                         bool packed, const int32_t *cu_q, const int32_t *cu_kv, int total_q,
                         int total_kv, const float *sinks, void *o, float *lse,
                         miattn_dtype dtype, void *stream) {
    g_err[0] = '\0';
    // (a packed call without query rows has nothing to check q and o against)
    miattn_status st = check_common(q, o, lse, B, (packed && total_q == 0) ? 0 : Sq, Hq, Hkv,
                                    D, scale, dtype);
    if (st != MIATTN_OK) return st;
    st = check_window_softcap(window_left, window_right, softcap);
    if (st != MIATTN_OK) return st;
    if (Skv < 0) return fail(MIATTN_ERR_INVALID_ARG, "negative dimension: Skv=%d", Skv);
    if (causal != 0 && causal != 1)
        return fail(MIATTN_ERR_INVALID_ARG, "causal=%d must be 0 or 1", causal);
    if (packed && (total_q < 0 || total_kv < 0))
        return fail(MIATTN_ERR_INVALID_ARG, "total_q=%d, total_kv=%d must be >= 0", total_q,
                    total_kv);
    if (sinks && ((uintptr_t)sinks & 3u))
        return fail(MIATTN_ERR_INVALID_ARG, "sinks not 4-byte aligned");
    if (B == 0 || Sq == 0 || (packed && total_q == 0)) return MIATTN_OK;
    if (packed) {
        if (!cu_q || !cu_kv)
            return fail(MIATTN_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_kv must not be NULL");
        if (((uintptr_t)cu_q & 3u) || ((uintptr_t)cu_kv & 3u))
            return fail(MIATTN_ERR_INVALID_ARG, "cu_seqlens_q/cu_seqlens_kv not 4-byte aligned");
    }
    const int64_t kv_rows = packed ? (int64_t)total_kv : (int64_t)B * Skv;
    if (kv_rows > 0 && Skv > 0) {
        if (!k || !v) return fail(MIATTN_ERR_INVALID_ARG, "k and v must not be NULL");
        if (!aligned16(k)) return fail(MIATTN_ERR_INVALID_ARG, "k not 16-byte aligned");
        if (!aligned16(v)) return fail(MIATTN_ERR_INVALID_ARG, "v not 16-byte aligned");
    }
    if (kv_rows > INT_MAX)
        return fail(MIATTN_ERR_UNSUPPORTED, "B*Skv = %lld exceeds %d key rows",
                    (long long)kv_rows, INT_MAX);
    if (packed && env_int("MIATTN_VALIDATE", 0) == 1) {
        st = validate_offsets(cu_q, B, total_q, Sq, "cu_seqlens_q", (hipStream_t)stream);
        if (st == MIATTN_OK)
            st = validate_offsets(cu_kv, B, total_kv, Skv, "cu_seqlens_kv", (hipStream_t)stream);
        if (st != MIATTN_OK) return st;
    }

    FwdParams p = {};
    p.q = (const uint16_t *)q;
    p.k = (const uint16_t *)k;
    p.v = (const uint16_t *)v;
    p.o = (uint16_t *)o;
    p.lse = lse;
    p.mask = key_padding_mask;
    p.cu_q = cu_q;
    p.cu_kv = packed ? cu_kv : nullptr;
    p.total_q = total_q;
    p.total_kv = total_kv;
    p.sinks = sinks;
    p.B = B;
    p.Sq = Sq;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Skv = Skv;
    p.causal = causal;
    const float alpha = resolve_scale(scale, D);
    set_scale(p, alpha);
    st = set_window_softcap(p, window_left, window_right, softcap, Skv, alpha);
    if (st != MIATTN_OK) return st;
    return run(p, D, dtype == MIATTN_BF16, false, Skv, softcap > 0.f, (hipStream_t)stream);
}

// The paged call, uniform (cu_q == NULL: B blocks of Sq queries) or with
// packed queries (Sq the per-request maximum, lse [Hq, total_q]).
miattn_status paged_call(const void *q, const void *k_cache, const void *v_cache,
                         const int32_t *real_seqlen_kv, const int32_t *block_table,
                         int page_size, int causal, int window_left, int window_right,
                         float softcap, bool packed, const int32_t *cu_q, int total_q,
                         const float *sinks, void *o, float *lse, int B, int Sq, int Hq, int Hkv,
                         int D, int max_pages, int num_phys_pages, float scale,
                         miattn_dtype dtype, void *stream,
                         const miattn::KvWriteParams *append = nullptr,
                         int cache_dtype = -1,  // -1: 16-bit pools of the inputs' dtype
                         const float *k_scale = nullptr, const float *v_scale = nullptr,
                         const PartialsSource &src = PartialsSource()) {
    g_err[0] = '\0';
    // (a packed call without query rows has nothing to check q and o against)
    miattn_status st = check_common(q, o, lse, B, (packed && total_q == 0) ? 0 : Sq, Hq, Hkv,
                                    D, scale, dtype);
    if (st != MIATTN_OK) return st;
    st = check_window_softcap(window_left, window_right, softcap);
    if (st != MIATTN_OK) return st;
    if (page_size <= 0) return fail(MIATTN_ERR_INVALID_ARG, "page_size must be > 0 (got %d)",
                                    page_size);
    if (page_size < 16 || (page_size & (page_size - 1)) != 0)
        return fail(MIATTN_ERR_UNSUPPORTED,
                    "page_size=%d unsupported (a power of two >= 16)", page_size);
    if (max_pages <= 0)
        return fail(MIATTN_ERR_INVALID_ARG, "max_pages must be > 0 (got %d)", max_pages);
    if (num_phys_pages < 0)
        return fail(MIATTN_ERR_INVALID_ARG, "num_phys_pages=%d is negative", num_phys_pages);
    if (causal != 0 && causal != 1)
        return fail(MIATTN_ERR_INVALID_ARG, "causal=%d must be 0 or 1", causal);
    if (packed && total_q < 0)
        return fail(MIATTN_ERR_INVALID_ARG, "total_q=%d must be >= 0", total_q);
    if (cache_dtype < 0) cache_dtype = (int)dtype;
    const bool fp8 = cache_dtype == MIATTN_CACHE_FP8_E4M3;
    if (!fp8 && cache_dtype != (int)dtype)
        return fail(MIATTN_ERR_UNSUPPORTED,
                    "cache_dtype %d must equal dtype %d or be MIATTN_CACHE_FP8_E4M3",
                    cache_dtype, (int)dtype);
    if (fp8 && D > 128)
        return fail(MIATTN_ERR_UNSUPPORTED, "FP8 pools: D=%d unsupported (64, 128)", D);
    if (fp8 && (!k_scale || !v_scale || ((uintptr_t)k_scale & 3u) || ((uintptr_t)v_scale & 3u)))
        return fail(MIATTN_ERR_INVALID_ARG,
                    "an FP8 pool needs 4-byte aligned k_scale and v_scale");
    if (sinks && ((uintptr_t)sinks & 3u))
        return fail(MIATTN_ERR_INVALID_ARG, "sinks not 4-byte aligned");
    const int64_t capacity = (int64_t)max_pages * page_size;
    if (capacity > INT_MAX / 2)
        return fail(MIATTN_ERR_UNSUPPORTED, "max_pages*page_size = %lld exceeds %d keys",
                    (long long)capacity, INT_MAX / 2);
    if (B == 0 || Sq == 0 || (packed && total_q == 0)) return MIATTN_OK;
    if (!k_cache || !v_cache || !real_seqlen_kv || !block_table)
        return fail(MIATTN_ERR_INVALID_ARG,
                    "k_cache, v_cache, real_seqlen_kv and block_table must not be NULL");
    if (!aligned16(k_cache)) return fail(MIATTN_ERR_INVALID_ARG, "k_cache not 16-byte aligned");
    if (!aligned16(v_cache)) return fail(MIATTN_ERR_INVALID_ARG, "v_cache not 16-byte aligned");
    if (((uintptr_t)real_seqlen_kv & 3u) || ((uintptr_t)block_table & 3u))
        return fail(MIATTN_ERR_INVALID_ARG, "real_seqlen_kv/block_table not 4-byte aligned");
    if (packed && !cu_q) return fail(MIATTN_ERR_INVALID_ARG, "cu_seqlens_q must not be NULL");
    if (packed && ((uintptr_t)cu_q & 3u))
        return fail(MIATTN_ERR_INVALID_ARG, "cu_seqlens_q not 4-byte aligned");

    int page_shift = 0;
    while ((1 << page_shift) < page_size) ++page_shift;

    // (the allocation-free entry point skips it: the check copies to host
    // vectors and synchronises the stream)
    if (!src.fixed && env_int("MIATTN_VALIDATE", 0) == 1) {
        // opt-in check of the device metadata (synchronises the stream)
        std::vector<int32_t> lens(B), bt((size_t)B * max_pages);
        hipStream_t s = (hipStream_t)stream;
        hipError_t e = hipMemcpyAsync(lens.data(), real_seqlen_kv, sizeof(int32_t) * B,
                                      hipMemcpyDeviceToHost, s);
        if (e == hipSuccess)
            e = hipMemcpyAsync(bt.data(), block_table, sizeof(int32_t) * bt.size(),
                               hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_fail(e, "MIATTN_VALIDATE metadata copy");
        for (int b = 0; b < B; ++b) {
            if (lens[b] < 0 || lens[b] > capacity)
                return fail(MIATTN_ERR_INVALID_ARG,
                            "real_seqlen_kv[%d]=%d outside [0, max_pages*page_size=%lld]", b,
                            lens[b], (long long)capacity);
            const int used = (lens[b] + page_size - 1) / page_size;
            for (int pg = 0; pg < used; ++pg) {
                const int32_t ph = bt[(size_t)b * max_pages + pg];
                if (ph < 0 || ph >= num_phys_pages)
                    return fail(MIATTN_ERR_INVALID_ARG,
                                "block_table[%d,%d]=%d outside [0, num_phys_pages=%d)", b, pg,
                                ph, num_phys_pages);
            }
        }
        if (packed) {
            st = validate_offsets(cu_q, B, total_q, Sq, "cu_seqlens_q", s);
            if (st != MIATTN_OK) return st;
        }
        if (fp8) {
            float sc[2] = {1.f, 1.f};
            e = hipMemcpyAsync(&sc[0], k_scale, sizeof(float), hipMemcpyDeviceToHost, s);
            if (e == hipSuccess)
                e = hipMemcpyAsync(&sc[1], v_scale, sizeof(float), hipMemcpyDeviceToHost, s);
            if (e == hipSuccess) e = hipStreamSynchronize(s);
            if (e != hipSuccess) return hip_fail(e, "MIATTN_VALIDATE scale copy");
            if (!(sc[0] > 0.f) || !(sc[1] > 0.f) || isinf(sc[0]) || isinf(sc[1]))
                return fail(MIATTN_ERR_INVALID_ARG, "FP8 scales must be finite and positive");
        }
    }

    FwdParams p = {};
    p.q = (const uint16_t *)q;
    p.k = (const uint16_t *)k_cache;
    p.v = (const uint16_t *)v_cache;
    p.o = (uint16_t *)o;
    p.lse = lse;
    p.seqlen = real_seqlen_kv;
    p.block_table = block_table;
    p.cu_q = cu_q;
    p.total_q = total_q;
    p.sinks = sinks;
    p.k_scale = fp8 ? k_scale : nullptr;
    p.v_scale = fp8 ? v_scale : nullptr;
    p.B = B;
    p.Sq = Sq;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.page_shift = page_shift;
    p.max_pages = max_pages;
    p.num_pages = num_phys_pages;
    p.causal = causal;
    const float alpha = resolve_scale(scale, D);
    set_scale(p, alpha);
    st = set_window_softcap(p, window_left, window_right, softcap, capacity, alpha);
    if (st != MIATTN_OK) return st;
    if (append) {
        // the chunk's keys and values go into the pools first (same stream)
        miattn::KvWriteParams w = *append;
        w.k_pool16 = (uint16_t *)k_cache;
        w.v_pool16 = (uint16_t *)v_cache;
        w.k_pool8 = (uint8_t *)k_cache;
        w.v_pool8 = (uint8_t *)v_cache;
        w.k_scale = k_scale;
        w.v_scale = v_scale;
        w.cu_q = cu_q;
        w.cache_seqlens = real_seqlen_kv;
        w.block_table = block_table;
        w.B = B;
        w.page_size = page_size;
        w.max_pages = max_pages;
        w.num_slots = (int64_t)num_phys_pages * page_size;
        w.tokens = total_q;
        w.row_elems = Hkv * D;
        hipError_t e = miattn::launch_kv_write(w, dtype == MIATTN_BF16, fp8, true,
                                               (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "KV write kernel launch");
        p.kv_append = 1;
    }
    return run(p, D, dtype == MIATTN_BF16, true, capacity, softcap > 0.f, (hipStream_t)stream,
               src);
}

}  // namespace

extern "C" {

miattn_status attn_fwd_dense(const void *q, const void *k, const void *v, int B, int Hq,
                             int Hkv, int Sq, int Skv, int D, float scale, int causal,
                             const uint8_t *key_padding_mask, void *o, float *lse,
                             miattn_dtype dtype, void *stream) {
    return dense_call(q, k, v, B, Hq, Hkv, Sq, Skv, D, scale, causal, -1, -1, 0.f,
                      key_padding_mask, false, nullptr, nullptr, 0, 0, nullptr, o, lse, dtype,
                      stream);
}

miattn_status attn_fwd_dense_ex(const void *q, const void *k, const void *v, int B, int Hq,
                                int Hkv, int Sq, int Skv, int D, float scale, int causal,
                                const uint8_t *key_padding_mask, void *o, float *lse,
                                int window_left, int window_right, float softcap,
                                miattn_dtype dtype, void *stream) {
    return dense_call(q, k, v, B, Hq, Hkv, Sq, Skv, D, scale, causal, window_left,
                      window_right, softcap, key_padding_mask, false, nullptr, nullptr, 0, 0,
                      nullptr, o, lse, dtype, stream);
}

miattn_status attn_fwd_varlen(const void *q, const void *k, const void *v,
                              const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_kv, int B,
                              int total_q, int total_kv, int max_seqlen_q, int max_seqlen_kv,
                              int Hq, int Hkv, int D, float scale, int causal, int window_left,
                              int window_right, float softcap, const float *sinks, void *o,
                              float *lse, miattn_dtype dtype, void *stream) {
    return dense_call(q, k, v, B, Hq, Hkv, max_seqlen_q, max_seqlen_kv, D, scale, causal,
                      window_left, window_right, softcap, nullptr, true, cu_seqlens_q,
                      cu_seqlens_kv, total_q, total_kv, sinks, o, lse, dtype, stream);
}

miattn_status attn_fwd_paged(const void *q, const void *k_cache, const void *v_cache,
                             const int32_t *real_seqlen_kv, const int32_t *block_table,
                             int page_size, int causal, void *o, float *lse, int B, int Sq,
                             int Hq, int Hkv, int D, int max_pages, int num_phys_pages,
                             float scale, miattn_dtype dtype, void *stream) {
    return paged_call(q, k_cache, v_cache, real_seqlen_kv, block_table, page_size, causal, -1,
                      -1, 0.f, false, nullptr, 0, nullptr, o, lse, B, Sq, Hq, Hkv, D, max_pages,
                      num_phys_pages, scale, dtype, stream);
}

miattn_status attn_fwd_paged_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                     const int32_t *real_seqlen_kv, const int32_t *block_table,
                                     int page_size, int causal, void *o, float *lse, int B,
                                     int Sq, int Hq, int Hkv, int D, int max_pages,
                                     int num_phys_pages, float scale, miattn_dtype dtype,
                                     void *stream) {
    PartialsSource fixed;
    fixed.fixed = true;
    return paged_call(q, k_cache, v_cache, real_seqlen_kv, block_table, page_size, causal, -1,
                      -1, 0.f, false, nullptr, 0, nullptr, o, lse, B, Sq, Hq, Hkv, D, max_pages,
                      num_phys_pages, scale, dtype, stream, nullptr, -1, nullptr, nullptr, fixed);
}

miattn_status attn_fwd_paged_ex(const void *q, const void *k_cache, const void *v_cache,
                                const int32_t *real_seqlen_kv, const int32_t *block_table,
                                int page_size, int causal, void *o, float *lse, int B, int Sq,
                                int Hq, int Hkv, int D, int max_pages, int num_phys_pages,
                                float scale, int window_left, int window_right, float softcap,
                                miattn_dtype dtype, void *stream) {
    return paged_call(q, k_cache, v_cache, real_seqlen_kv, block_table, page_size, causal,
                      window_left, window_right, softcap, false, nullptr, 0, nullptr, o, lse, B,
                      Sq, Hq, Hkv, D, max_pages, num_phys_pages, scale, dtype, stream);
}

miattn_status attn_fwd_paged_varlen(const void *q, const void *k_cache, const void *v_cache,
                                    const int32_t *cache_seqlens, const int32_t *block_table,
                                    const int32_t *cu_seqlens_q, int page_size, int causal,
                                    int window_left, int window_right, float softcap,
                                    const float *sinks, void *o, float *lse, int B,
                                    int total_q, int max_seqlen_q, int Hq, int Hkv, int D,
                                    int max_pages, int num_phys_pages, float scale,
                                    miattn_dtype dtype, miattn_cache_dtype cache_dtype,
                                    const float *k_scale, const float *v_scale, void *stream) {
    if ((int)cache_dtype < 0 || (int)cache_dtype > MIATTN_CACHE_FP8_E4M3) {
        g_err[0] = '\0';
        return fail(MIATTN_ERR_INVALID_ARG, "cache_dtype %d unknown", (int)cache_dtype);
    }
    return paged_call(q, k_cache, v_cache, cache_seqlens, block_table, page_size, causal,
                      window_left, window_right, softcap, true, cu_seqlens_q, total_q, sinks, o,
                      lse, B, max_seqlen_q, Hq, Hkv, D, max_pages, num_phys_pages, scale, dtype,
                      stream, nullptr, cache_dtype, k_scale, v_scale);
}

miattn_status kv_cache_write(const void *k, const void *v, void *k_pages, void *v_pages,
                             const int64_t *slot_mapping, int tokens, int Hkv, int D,
                             int64_t num_slots, miattn_dtype dtype, miattn_cache_dtype cache_dtype,
                             const float *k_scale, const float *v_scale, void *stream) {
    g_err[0] = '\0';
    if (tokens < 0) return fail(MIATTN_ERR_INVALID_ARG, "tokens=%d is negative", tokens);
    if (Hkv <= 0 || D <= 0)
        return fail(MIATTN_ERR_INVALID_ARG, "Hkv=%d and D=%d must be positive", Hkv, D);
    if (num_slots < 0)
        return fail(MIATTN_ERR_INVALID_ARG, "num_slots=%lld is negative", (long long)num_slots);
    if (dtype != MIATTN_BF16 && dtype != MIATTN_FP16)
        return fail(MIATTN_ERR_UNSUPPORTED, "dtype %d unsupported (MIATTN_BF16, MIATTN_FP16)",
                    (int)dtype);
    if ((int)cache_dtype < 0 || (int)cache_dtype > MIATTN_CACHE_FP8_E4M3)
        return fail(MIATTN_ERR_INVALID_ARG, "cache_dtype %d unknown", (int)cache_dtype);
    const bool fp8 = cache_dtype == MIATTN_CACHE_FP8_E4M3;
    if (!fp8 && (int)cache_dtype != (int)dtype)
        return fail(MIATTN_ERR_UNSUPPORTED,
                    "cache_dtype %d must equal dtype %d or be MIATTN_CACHE_FP8_E4M3",
                    (int)cache_dtype, (int)dtype);
    if (((int64_t)Hkv * D) % 8 != 0 || (int64_t)Hkv * D > INT_MAX / 2)
        return fail(MIATTN_ERR_UNSUPPORTED, "Hkv*D = %lld must be a multiple of 8 (and < %d)",
                    (long long)Hkv * D, INT_MAX / 2);
    if ((int64_t)tokens * (Hkv * D / 8) > (int64_t)INT_MAX * 256)
        return fail(MIATTN_ERR_UNSUPPORTED, "tokens*Hkv*D too large for one launch");
    if (tokens == 0) return MIATTN_OK;
    if (!k || !v || !k_pages || !v_pages || !slot_mapping)
        return fail(MIATTN_ERR_INVALID_ARG,
                    "k, v, k_pages, v_pages and slot_mapping must not be NULL");
    if (!aligned16(k) || !aligned16(v))
        return fail(MIATTN_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
    const uintptr_t pool_align = fp8 ? 7u : 15u;
    if (((uintptr_t)k_pages & pool_align) || ((uintptr_t)v_pages & pool_align))
        return fail(MIATTN_ERR_INVALID_ARG, "k_pages/v_pages must be %d-byte aligned",
                    fp8 ? 8 : 16);
    if ((uintptr_t)slot_mapping & 7u)
        return fail(MIATTN_ERR_INVALID_ARG, "slot_mapping not 8-byte aligned");
    if (fp8 && (!k_scale || !v_scale || ((uintptr_t)k_scale & 3u) || ((uintptr_t)v_scale & 3u)))
        return fail(MIATTN_ERR_INVALID_ARG,
                    "an FP8 cache needs 4-byte aligned k_scale and v_scale");
    if (env_int("MIATTN_VALIDATE", 0) == 1) {
        std::vector<int64_t> sl(tokens);
        hipStream_t s = (hipStream_t)stream;
        hipError_t e = hipMemcpyAsync(sl.data(), slot_mapping, sizeof(int64_t) * tokens,
                                      hipMemcpyDeviceToHost, s);
        float sc[2] = {1.f, 1.f};
        if (e == hipSuccess && fp8)
            e = hipMemcpyAsync(&sc[0], k_scale, sizeof(float), hipMemcpyDeviceToHost, s);
        if (e == hipSuccess && fp8)
            e = hipMemcpyAsync(&sc[1], v_scale, sizeof(float), hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_fail(e, "MIATTN_VALIDATE metadata copy");
        for (int n = 0; n < tokens; ++n)
            if (sl[n] < -1 || sl[n] >= num_slots)
                return fail(MIATTN_ERR_INVALID_ARG,
                            "slot_mapping[%d]=%lld outside [-1, num_slots=%lld)", n,
                            (long long)sl[n], (long long)num_slots);
        if (!(sc[0] > 0.f) || !(sc[1] > 0.f) || isinf(sc[0]) || isinf(sc[1]))
            return fail(MIATTN_ERR_INVALID_ARG, "FP8 scales must be finite and positive");
    }
    miattn::KvWriteParams w = {};
    w.k = (const uint16_t *)k;
    w.v = (const uint16_t *)v;
    w.k_pool16 = (uint16_t *)k_pages;
    w.v_pool16 = (uint16_t *)v_pages;
    w.k_pool8 = (uint8_t *)k_pages;
    w.v_pool8 = (uint8_t *)v_pages;
    w.k_scale = k_scale;
    w.v_scale = v_scale;
    w.slot_mapping = slot_mapping;
    w.tokens = tokens;
    w.row_elems = Hkv * D;
    w.num_slots = num_slots;
    hipError_t e = miattn::launch_kv_write(w, dtype == MIATTN_BF16, fp8, false,
                                           (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "KV write kernel launch");
    return MIATTN_OK;
}

miattn_status attn_fwd_paged_append(const void *q, const void *k_new, const void *v_new,
                                    void *k_cache, void *v_cache, const int32_t *cache_seqlens,
                                    const int32_t *block_table, const int32_t *cu_seqlens_q,
                                    int page_size, int causal, float softcap, void *o,
                                    float *lse, int B, int total_q, int max_seqlen_q, int Hq,
                                    int Hkv, int D, int max_pages, int num_phys_pages,
                                    float scale, miattn_dtype dtype,
                                    miattn_cache_dtype cache_dtype, const float *k_scale,
                                    const float *v_scale, void *stream) {
    if ((int)cache_dtype < 0 || (int)cache_dtype > MIATTN_CACHE_FP8_E4M3) {
        g_err[0] = '\0';
        return fail(MIATTN_ERR_INVALID_ARG, "cache_dtype %d unknown", (int)cache_dtype);
    }
    if (B > 0 && total_q > 0 && max_seqlen_q > 0) {
        if (!k_new || !v_new) {
            g_err[0] = '\0';
            return fail(MIATTN_ERR_INVALID_ARG, "k_new and v_new must not be NULL");
        }
        if (!aligned16(k_new) || !aligned16(v_new)) {
            g_err[0] = '\0';
            return fail(MIATTN_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
        }
    }
    miattn::KvWriteParams w = {};
    w.k = (const uint16_t *)k_new;
    w.v = (const uint16_t *)v_new;
    return paged_call(q, k_cache, v_cache, cache_seqlens, block_table, page_size, causal, -1,
                      -1, softcap, true, cu_seqlens_q, total_q, nullptr, o, lse, B,
                      max_seqlen_q, Hq, Hkv, D, max_pages, num_phys_pages, scale, dtype, stream,
                      &w, cache_dtype, k_scale, v_scale);
}

miattn_status attn_bwd(const void *q, const void *k, const void *v, const void *o,
                       const void *dout, const float *lse, int B, int Hq, int Hkv, int Sq, int Skv,
                       int D, float scale, int causal, void *dq, void *dk, void *dv,
                       miattn_dtype dtype, void *stream) {
    g_err[0] = '\0';
    miattn_status st = check_common(q, dq, const_cast<float *>(lse), B, Sq, Hq, Hkv, D, scale, dtype);
    if (st != MIATTN_OK) return st;
    if (D == 256) return fail(MIATTN_ERR_UNSUPPORTED, "D=256 unsupported by the backward (64, 128)");
    if (Skv < 0) return fail(MIATTN_ERR_INVALID_ARG, "negative dimension: Skv=%d", Skv);
    if (causal != 0 && causal != 1)
        return fail(MIATTN_ERR_INVALID_ARG, "causal=%d must be 0 or 1", causal);
    if ((int64_t)B * Skv > INT_MAX || (int64_t)B * Sq * Hq > INT_MAX)
        return fail(MIATTN_ERR_UNSUPPORTED, "B*Skv or B*Sq*Hq exceeds %d rows", INT_MAX);
    if (B == 0 || (Sq == 0 && Skv == 0)) return MIATTN_OK;
    if (Skv > 0) {
        if (!k || !v || !dk || !dv)
            return fail(MIATTN_ERR_INVALID_ARG, "k, v, dk and dv must not be NULL");
        if (!aligned16(k) || !aligned16(v) || !aligned16(dk) || !aligned16(dv))
            return fail(MIATTN_ERR_INVALID_ARG, "k, v, dk and dv must be 16-byte aligned");
    }
    if (Sq > 0) {
        if (!o || !dout || !lse)
            return fail(MIATTN_ERR_INVALID_ARG, "o, do and lse must not be NULL");
        if (!aligned16(o) || !aligned16(dout))
            return fail(MIATTN_ERR_INVALID_ARG, "o and do must be 16-byte aligned");
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MIATTN_ERR_UNSUPPORTED, "device %d", dev);
    hipStream_t s = (hipStream_t)stream;
    if (Sq == 0) {
        // no query: every key gradient is zero
        const size_t bytes = (size_t)B * Skv * Hkv * D * 2;
        e = miattn::launch_zero_fill(dk, bytes, s);
        if (e == hipSuccess) e = miattn::launch_zero_fill(dv, bytes, s);
        return e == hipSuccess ? MIATTN_OK : hip_fail(e, "zero fill kernel launch");
    }
    miattn::BwdParams p = {};
    p.q = (const uint16_t *)q;
    p.k = (const uint16_t *)k;
    p.v = (const uint16_t *)v;
    p.o = (const uint16_t *)o;
    p.dout = (const uint16_t *)dout;
    p.lse = lse;
    p.dq = (uint16_t *)dq;
    p.dk = (uint16_t *)dk;
    p.dv = (uint16_t *)dv;
    p.B = B;
    p.Sq = Sq;
    p.Skv = Skv;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.G = Hq / Hkv;
    p.rows = Sq * p.G;
    p.n_mblocks = (p.rows + 127) / 128;
    p.causal = causal;
    const float alpha = resolve_scale(scale, D);
    p.scale = alpha;
    p.scale_log2 = alpha * 1.4426950408889634f;
    // bwd_dkdv runs one workgroup per CU: the first wave is one per CU
    p.down_wgs = compute_units(dev);
    const size_t nrows = (size_t)B * Hq * Sq;
    void *ws = nullptr;
    if (Skv == 0) {
        // no key: every query gradient is zero
        e = miattn::launch_zero_fill(dq, (size_t)B * Sq * Hq * D * 2, s);
        return e == hipSuccess ? MIATTN_OK : hip_fail(e, "zero fill kernel launch");
    }
    st = workspace(dev, s, nrows * 2 * sizeof(float), &ws);
    if (st != MIATTN_OK) return st;
    p.d_rows = (float *)ws;
    p.lse2_rows = p.d_rows + nrows;
    e = timed_launch(0, s, [&] { return miattn::launch_attn_bwd(p, D, dtype == MIATTN_BF16, s); });
    if (e != hipSuccess) return hip_fail(e, "backward kernel launch");
    return workspace_done(dev, s);
}

miattn_status miattn_release_workspace(void) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MIATTN_ERR_UNSUPPORTED, "device %d", dev);
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceState &d = g_dev[dev];
    if (d.ws) d.retired.push_back(d.ws);
    d.ws = nullptr;
    d.ws_bytes = 0;
    miattn_status st = MIATTN_OK;
    for (void *ptr : d.retired) {
        e = hipFree(ptr);  // waits for work that may still use it
        if (e != hipSuccess && st == MIATTN_OK) st = hip_fail(e, "hipFree(workspace)");
    }
    d.retired.clear();
    if (d.last_use) (void)hipEventDestroy(d.last_use);
    d.last_use = nullptr;
    d.used = false;
    d.last_stream = nullptr;
    return st;
}

void miattn_set_split_keys(int keys_per_split) {
    g_split_keys = keys_per_split > 0 ? keys_per_split : 0;
}

void miattn_set_streamk_piece(int tiles) {
    g_sk_piece = tiles < 0 ? kSkPieceDefault : std::min(tiles, kSkPieceMax);
}

void miattn_profile_start(void) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    for (auto &v : g_prof.ev)
        for (auto &pr : v) {
            (void)hipEventDestroy(pr.first);
            (void)hipEventDestroy(pr.second);
        }
    g_prof.ev[0].clear();
    g_prof.ev[1].clear();
    g_prof.on = true;
}

miattn_status miattn_profile_stop(double *attn_ms, int *attn_launches, double *merge_ms,
                                  int *merge_launches) {
    std::vector<std::pair<hipEvent_t, hipEvent_t>> ev[2];
    {
        std::lock_guard<std::mutex> lock(g_prof_mu);
        g_prof.on = false;
        ev[0].swap(g_prof.ev[0]);
        ev[1].swap(g_prof.ev[1]);
    }
    double tot[2] = {0.0, 0.0};
    miattn_status st = MIATTN_OK;
    for (int kind = 0; kind < 2; ++kind)
        for (auto &pr : ev[kind]) {
            float ms = 0.f;
            hipError_t e = hipEventSynchronize(pr.second);
            if (e == hipSuccess) e = hipEventElapsedTime(&ms, pr.first, pr.second);
            if (e != hipSuccess && st == MIATTN_OK) st = hip_fail(e, "hipEventElapsedTime");
            tot[kind] += ms;
            (void)hipEventDestroy(pr.first);
            (void)hipEventDestroy(pr.second);
        }
    if (attn_ms) *attn_ms = tot[0];
    if (attn_launches) *attn_launches = (int)ev[0].size();
    if (merge_ms) *merge_ms = tot[1];
    if (merge_launches) *merge_launches = (int)ev[1].size();
    return st;
}

}  // extern "C"
