// segtopk.hip -- host side of libsegtopk: request validation, the launch plan
// (one workgroup per segment, or several per segment when the batch alone
// cannot fill the device), scratch for the multi-workgroup plan, and dispatch
// to the kernel of the key type.  The kernels and their method are described
// in topk_kernel.h.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>

#include <map>
#include <mutex>
#include <thread>

#include "topk_common.h"

using namespace segtopk_impl;

namespace {

__global__ void zero_kernel(uint32_t *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// Processing order for a batch with one workgroup per segment: segments by
// size class (floor(log2 n) + 1), largest class first, so that the longest
// segments start first and the short ones fill the workgroup slots as they
// free up.  One workgroup of 1024 threads, num_segments <= 2048.
__global__ __launch_bounds__(1024) void order_kernel(const int64_t *off, int64_t num_segments,
                                                    uint32_t *order) {
    __shared__ uint32_t cnt[33];
    const uint32_t t = threadIdx.x;
    if (t < 33) cnt[t] = 0u;
    __syncthreads();
    uint32_t cls[2];
    for (int j = 0; j < 2; ++j) {
        const int64_t i = (int64_t)t + (int64_t)j * 1024;
        cls[j] = 0u;
        if (i < num_segments) {
            const int64_t d = off[i + 1] - off[i];
            const uint32_t n = d > 0 ? (uint32_t)d : 0u;
            cls[j] = n ? 32u - (uint32_t)__clz((int)n) : 0u;
            atomicAdd(&cnt[cls[j]], 1u);
        }
    }
    __syncthreads();
    if (t == 0) {  // exclusive prefix, largest class first
        uint32_t run = 0;
        for (int c = 32; c >= 0; --c) {
            const uint32_t n = cnt[c];
            cnt[c] = run;
            run += n;
        }
    }
    __syncthreads();
    for (int j = 0; j < 2; ++j) {
        const int64_t i = (int64_t)t + (int64_t)j * 1024;
        if (i < num_segments) order[atomicAdd(&cnt[cls[j]], 1u)] = (uint32_t)i;
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
constexpr uint32_t kTargetWorkgroups = 2048;  // enough to fill 256 CUs several times
constexpr uint32_t kMaxWgPerSeg = 256;
constexpr uint32_t kMinSlice = 16384;
constexpr int64_t kOrderMinSegments = 256;  // fewer segments: no processing order

int key_bytes(int type) { return (type == SEGTOPK_KEY_BF16 || type == SEGTOPK_KEY_F16) ? 2 : 4; }

uint32_t next_pow2(uint32_t x) {
    uint32_t p = 1;
    while (p < x) p <<= 1;
    return p;
}

std::mutex g_pool_mu;
bool g_pool_ready[64];

// Keep freed scratch in the device's stream-ordered pool between calls.
void prepare_pool(int dev) {
    std::lock_guard<std::mutex> lk(g_pool_mu);
    if (dev < 0 || dev >= 64 || g_pool_ready[dev]) return;
    hipMemPool_t pool;
    if (hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) {
        uint64_t thr = UINT64_MAX;
        (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr);
    }
    g_pool_ready[dev] = true;
}

// Scratch reused across the calls on one stream.  Stream order keeps the
// calls on a stream from overlapping, so one buffer per (device, stream)
// suffices; a stream-ordered malloc/free pair in every call made the host
// wait for the device each time.  A call that needs more grows the buffer
// (the old one is freed in stream order); buffers are held until the process
// ends.  The per-thread default stream is one handle for many streams, so
// that key also holds the calling thread.  Each buffer carries an event
// recorded after its last use: a call first makes its stream wait for it,
// so that a stream created with the handle of a destroyed one that still
// has work queued cannot overlap that work.  The caller holds g_ws_mu from
// stream_scratch until it has queued its kernels and recorded the event.
struct WsKey {
    int dev;
    hipStream_t stream;
    std::thread::id thread;
    bool operator<(const WsKey &o) const {
        if (dev != o.dev) return dev < o.dev;
        if (stream != o.stream) return stream < o.stream;
        return thread < o.thread;
    }
};
struct WsBuf {
    void *ptr = nullptr;
    size_t bytes = 0;
    hipEvent_t done = nullptr;
    // Leading 32-bit words that are zero once the stream's queued work is
    // done: slice mode leaves its histograms and tickets cleared again.
    size_t clean_words = 0;
};
std::mutex g_ws_mu;
std::map<WsKey, WsBuf> g_ws;

hipError_t stream_scratch(int dev, hipStream_t stream, size_t bytes, WsBuf **out) {
    const WsKey key{dev, stream,
                    stream == hipStreamPerThread ? std::this_thread::get_id() : std::thread::id()};
    WsBuf &b = g_ws[key];
    if (!b.done) {
        const hipError_t e = hipEventCreateWithFlags(&b.done, hipEventDisableTiming);
        if (e != hipSuccess) {
            b.done = nullptr;
            return e;
        }
    } else {
        const hipError_t e = hipStreamWaitEvent(stream, b.done, 0);
        if (e != hipSuccess) return e;
    }
    if (b.bytes < bytes) {
        size_t want = bytes + (bytes >> 2);
        want = (want + ((size_t)1 << 20) - 1) & ~(((size_t)1 << 20) - 1);
        void *np = nullptr;
        const hipError_t e = hipMallocAsync(&np, want, stream);
        if (e != hipSuccess) return e;
        if (b.ptr) (void)hipFreeAsync(b.ptr, stream);
        b.ptr = np;
        b.bytes = want;
        b.clean_words = 0;
    }
    *out = &b;
    return hipSuccess;
}

// Workgroups of the split kernel of (key type, direction) that the device
// holds at once with `lds` bytes of dynamic LDS; cached per combination.
struct OccKey {
    int dev, kt, largest;
    size_t lds;
    uint32_t wgs;
};
std::mutex g_occ_mu;
OccKey g_occ[64];
int g_occ_n = 0;

int per_cu_for(int type, bool largest, size_t lds) {
    switch (type) {
    case SEGTOPK_KEY_F32: return topk_per_cu<SEGTOPK_KEY_F32>(largest, lds);
    case SEGTOPK_KEY_BF16: return topk_per_cu<SEGTOPK_KEY_BF16>(largest, lds);
    case SEGTOPK_KEY_U32: return topk_per_cu<SEGTOPK_KEY_U32>(largest, lds);
    case SEGTOPK_KEY_I32: return topk_per_cu<SEGTOPK_KEY_I32>(largest, lds);
    default: return topk_per_cu<SEGTOPK_KEY_F16>(largest, lds);
    }
}

uint32_t resident_wgs_for(int type, int dev, bool largest, size_t lds) {
    {
        std::lock_guard<std::mutex> lk(g_occ_mu);
        for (int i = 0; i < g_occ_n; ++i)
            if (g_occ[i].dev == dev && g_occ[i].kt == type && g_occ[i].largest == (int)largest &&
                g_occ[i].lds == lds)
                return g_occ[i].wgs;
    }
    const int per_cu = per_cu_for(type, largest, lds);
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        cus = 256;
    const uint32_t wgs = (uint32_t)per_cu * (uint32_t)cus;
    std::lock_guard<std::mutex> lk(g_occ_mu);
    if (g_occ_n < 64) g_occ[g_occ_n++] = OccKey{dev, type, (int)largest, lds, wgs};
    return wgs;
}

hipError_t launch(int type, const Params &p, bool largest, int variant, uint32_t grid, size_t lds,
                  hipStream_t st) {
    switch (type) {
    case SEGTOPK_KEY_F32: return launch_topk<SEGTOPK_KEY_F32>(p, largest, variant, grid, lds, st);
    case SEGTOPK_KEY_BF16: return launch_topk<SEGTOPK_KEY_BF16>(p, largest, variant, grid, lds, st);
    case SEGTOPK_KEY_U32: return launch_topk<SEGTOPK_KEY_U32>(p, largest, variant, grid, lds, st);
    case SEGTOPK_KEY_I32: return launch_topk<SEGTOPK_KEY_I32>(p, largest, variant, grid, lds, st);
    default: return launch_topk<SEGTOPK_KEY_F16>(p, largest, variant, grid, lds, st);
    }
}

}  // namespace

extern "C" int batched_topk(const segtopk_keys *keys, const segtopk_values *values,
                            const int64_t *segment_offsets, int64_t num_segments, int64_t k,
                            int direction, int determinism, int tie_break, int ordering,
                            hipStream_t stream) {
    // ---- validation (no HIP call before it passes) ----
    if (!keys) return SEGTOPK_INVALID_ARGUMENT;
    const int type = keys->type;
    if (type < SEGTOPK_KEY_F32 || type > SEGTOPK_KEY_F16) return SEGTOPK_INVALID_ARGUMENT;
    if (direction != SEGTOPK_MAX && direction != SEGTOPK_MIN) return SEGTOPK_INVALID_ARGUMENT;
    if (determinism < SEGTOPK_NOT_GUARANTEED || determinism > SEGTOPK_GPU_TO_GPU)
        return SEGTOPK_INVALID_ARGUMENT;
    if (tie_break < SEGTOPK_TIE_UNSPECIFIED || tie_break > SEGTOPK_PREFER_LARGER_INDEX)
        return SEGTOPK_INVALID_ARGUMENT;
    if (ordering < SEGTOPK_UNSORTED || ordering > SEGTOPK_STABLE_SORTED)
        return SEGTOPK_INVALID_ARGUMENT;
    // An explicit index tie-break pins the set across GPUs, so it must come
    // with gpu_to_gpu.   [docs "Top-K: Determinism ...", "Which items are selected?"]
    if (tie_break != SEGTOPK_TIE_UNSPECIFIED && determinism != SEGTOPK_GPU_TO_GPU)
        return SEGTOPK_INVALID_ARGUMENT;
    if (k < 0 || k > INT32_MAX || num_segments < 0 || num_segments > INT32_MAX)
        return SEGTOPK_INVALID_ARGUMENT;
    if (num_segments == 0 || k == 0) return SEGTOPK_OK;
    if (!keys->in || !keys->out || !segment_offsets) return SEGTOPK_INVALID_ARGUMENT;
    const bool pairs = values && values->in;
    if (pairs && !values->out) return SEGTOPK_INVALID_ARGUMENT;
    const int kb = key_bytes(type);
    if ((reinterpret_cast<uintptr_t>(keys->in) % kb) || (reinterpret_cast<uintptr_t>(keys->out) % kb))
        return SEGTOPK_INVALID_ARGUMENT;
    if (pairs && ((reinterpret_cast<uintptr_t>(values->in) & 3) ||
                  (reinterpret_cast<uintptr_t>(values->out) & 3)))
        return SEGTOPK_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(segment_offsets) & 7)) return SEGTOPK_INVALID_ARGUMENT;
    const bool sorted = ordering != SEGTOPK_UNSORTED;
    if (sorted && k > SEGTOPK_MAX_SORTED_K) return SEGTOPK_NOT_SUPPORTED;

    // ---- plan ----
    Params p = {};
    p.keys_in = keys->in;
    p.keys_out = keys->out;
    p.vals_in = pairs ? static_cast<const uint32_t *>(values->in) : nullptr;
    p.vals_out = pairs ? static_cast<uint32_t *>(values->out) : nullptr;
    p.offsets = segment_offsets;
    p.num_segments = num_segments;
    p.k = (uint32_t)k;
    p.det = determinism != SEGTOPK_NOT_GUARANTEED;
    p.prefer_larger = tie_break == SEGTOPK_PREFER_LARGER_INDEX;
    p.sorted = sorted;

    const uint32_t k32 = (uint32_t)k;
    // Output staging: sorted output is staged and sorted in LDS; unsorted
    // output only for small k (coalesced row writes), else written in place.
    uint32_t out_cap = next_pow2(k32 < 2 ? 2 : k32);
    if (!sorted && out_cap > 256) out_cap = 0;
    // Several workgroups per segment when the segments alone cannot fill the
    // device.  Stash: with one workgroup per segment, room for about eight
    // times k candidates in four wave regions; with several, the
    // segment-wide bound keeps each slice's candidates few, and the stash
    // only has to hold bucket b* of the last arriver (about 2k at most).
    const bool split = (uint64_t)num_segments < kTargetWorkgroups;
    uint32_t stash_cap = next_pow2((split ? 2 : 8) * k32);
    if (stash_cap < (split ? 2048u : 1024u)) stash_cap = split ? 2048u : 1024u;
    if (stash_cap > 8192) stash_cap = 8192;
    while (stash_cap > 1024 && 8 * (size_t)(stash_cap + out_cap) > kMaxDynLds) stash_cap >>= 1;
    if (8 * (size_t)(stash_cap + out_cap) > kMaxDynLds) return SEGTOPK_NOT_SUPPORTED;
    p.stash_cap = stash_cap;
    p.out_cap = out_cap;
    const size_t lds = 8 * (size_t)(stash_cap + out_cap);

    int dev = 0;
    uint32_t P = 1;
    if (split) {
        // As many workgroups as the device holds at once, so that all the
        // slices of a segment run together and share their bound.
        if (hipGetDevice(&dev) != hipSuccess) return SEGTOPK_HIP_ERROR;
        const uint32_t target = resident_wgs_for(type, dev, direction == SEGTOPK_MAX, lds);
        P = (uint32_t)((target + num_segments - 1) / num_segments);
        if (P > kMaxWgPerSeg) P = kMaxWgPerSeg;
        if (P < 1) P = 1;
    }
    uint32_t min_slice = kMinSlice;
    if ((uint64_t)8 * k32 > min_slice) min_slice = 8 * k32 > (1u << 30) ? (1u << 30) : 8 * k32;
    if (k32 * 2 > stash_cap) P = 1;  // slices could not hold their local candidates
    p.wg_per_seg = P;
    p.min_slice = min_slice;

    const uint64_t S8 = ((uint64_t)num_segments + 7) / 8 * 8;
    const uint64_t grid = S8 * P;
    if (grid > 0x7FFFFFFFull) return SEGTOPK_NOT_SUPPORTED;

    void *ws = nullptr;
    WsBuf *wsb = nullptr;
    size_t zero_words_used = 0;
    std::unique_lock<std::mutex> ws_lock(g_ws_mu, std::defer_lock);
    hipError_t err = hipSuccess;
    if (split && P == 1 && num_segments >= kOrderMinSegments) {
        // One workgroup per segment for many segments of unknown sizes:
        // process the largest first.
        if (hipGetDevice(&dev) != hipSuccess) return SEGTOPK_HIP_ERROR;
        prepare_pool(dev);
        ws_lock.lock();
        if (stream_scratch(dev, stream, (size_t)num_segments * sizeof(uint32_t), &wsb) != hipSuccess)
            return SEGTOPK_HIP_ERROR;
        ws = wsb->ptr;
        wsb->clean_words = 0;  // the order overwrites the front
        p.order = static_cast<const uint32_t *>(ws);
        hipLaunchKernelGGL(order_kernel, dim3(1), dim3(1024), 0, stream, segment_offsets,
                           num_segments, static_cast<uint32_t *>(ws));
        err = hipGetLastError();
    } else if (P > 1) {
        prepare_pool(dev);
        const size_t S = (size_t)num_segments;
        const size_t n_hist = S * kBuckets, n_ticket = S;
        const size_t zero_words = 2 * n_hist + n_ticket;
        zero_words_used = zero_words;
        const size_t info_words = S * P * 4;
        const size_t cum_words = S * P * kBuckets;
        size_t bytes = (zero_words + info_words + cum_words) * 4;
        bytes = (bytes + 255) & ~(size_t)255;
        const size_t data_off = bytes;
        bytes += S * P * (size_t)stash_cap * sizeof(uint2);
        ws_lock.lock();
        if (stream_scratch(dev, stream, bytes, &wsb) != hipSuccess) return SEGTOPK_HIP_ERROR;
        ws = wsb->ptr;
        uint32_t *wsw = static_cast<uint32_t *>(ws);
        p.ws_hist = wsw;
        p.ws_early = wsw + n_hist;
        p.ws_ticket = wsw + 2 * n_hist;
        p.ws_slot_info = wsw + zero_words;
        p.ws_slot_cum = wsw + zero_words + info_words;
        p.ws_slot_data = reinterpret_cast<uint2 *>(static_cast<char *>(ws) + data_off);
        if (wsb->clean_words < zero_words) {
            size_t zb = (zero_words + 255) / 256;
            if (zb > 1024) zb = 1024;
            hipLaunchKernelGGL(zero_kernel, dim3((unsigned)zb), dim3(256), 0, stream, wsw, zero_words);
            err = hipGetLastError();
        }
        // The slots (after the cleared words) are written by this call; the
        // sliced kernel clears the histograms and tickets it used.
        wsb->clean_words = 0;
    }
    if (err == hipSuccess) {
        const bool largest = direction == SEGTOPK_MAX;
        const int variant = !split ? kVariantOne : (P > 1 ? kVariantSliced : kVariantSplit);
        err = launch(type, p, largest, variant, (uint32_t)grid, lds, stream);
        if (err == hipSuccess && variant == kVariantSliced) wsb->clean_words = zero_words_used;
    }
    if (wsb) {
        const hipError_t e = hipEventRecord(wsb->done, stream);
        if (err == hipSuccess) err = e;
    }
    return err == hipSuccess ? SEGTOPK_OK : SEGTOPK_HIP_ERROR;
}

extern "C" const char *segtopk_status_string(int status) {
    switch (status) {
    case SEGTOPK_OK: return "ok";
    case SEGTOPK_INVALID_ARGUMENT: return "invalid argument";
    case SEGTOPK_NOT_SUPPORTED: return "not supported";
    case SEGTOPK_HIP_ERROR: return "HIP error";
    default: return "unknown status";
    }
}

extern "C" int segtopk_version(void) { return 200; }
