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

// 8-byte payloads: the selection left each winner's source index in the low
// half of its 8-byte output slot; replace it by the payload.  Slots past k_i
// are not touched.  One thread per slot of the S x k output.
__global__ void gather64_kernel(const int64_t *off, const int32_t *kseg, int64_t num_segments,
                                uint32_t k, const uint64_t *vals_in, uint64_t *vals_out) {
    const uint64_t total = (uint64_t)num_segments * k;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (uint64_t)gridDim.x * blockDim.x) {
        const uint64_t row = i / k;
        const uint32_t j = (uint32_t)(i - row * k);
        const int64_t b = off[row], e = off[row + 1];
        const uint64_t n = e > b ? (uint64_t)(e - b) : 0u;
        uint64_t k_i = n < k ? n : k;
        if (kseg) {
            const int32_t ks = kseg[row];
            const uint64_t ku = ks > 0 ? (uint64_t)ks : 0u;
            k_i = ku < k_i ? ku : k_i;
        }
        if (j >= k_i) continue;
        const uint32_t idx = (uint32_t)vals_out[i];
        if (idx < n) vals_out[i] = vals_in[b + idx];
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
constexpr uint32_t kTargetWorkgroups = 2048;  // enough to fill 256 CUs several times
constexpr uint32_t kMinSlice = 16384;
constexpr int64_t kOrderMinSegments = 256;  // fewer segments: no processing order
constexpr size_t kMaxCachedStreams = 16;    // scratch buffers kept (LRU beyond that)
constexpr uint32_t kPlainCand = 2048;  // LDS candidate list of the plain kernel

// Key types served by the plain kernel (64-bit and 8-bit keys).
bool is_plain_key(int type) {
    return type == SEGTOPK_KEY_U64 || type == SEGTOPK_KEY_I64 || type == SEGTOPK_KEY_F64 ||
           type == SEGTOPK_KEY_U8 || type == SEGTOPK_KEY_I8;
}

int key_bytes(int type) {
    switch (type) {
    case SEGTOPK_KEY_U8: case SEGTOPK_KEY_I8: return 1;
    case SEGTOPK_KEY_BF16: case SEGTOPK_KEY_F16: case SEGTOPK_KEY_U16: case SEGTOPK_KEY_I16: return 2;
    case SEGTOPK_KEY_U64: case SEGTOPK_KEY_I64: case SEGTOPK_KEY_F64: return 8;
    default: return 4;
    }
}

// Smallest power of two >= x, for 1 <= x <= 2^62.
uint64_t next_pow2(uint64_t x) {
    uint64_t p = 1;
    while (p < x) p <<= 1;
    return p;
}

// The library's own stream-ordered pool per device (freed scratch stays
// cached in it; the device's default pool is left as the process set it).
std::mutex g_pool_mu;
hipMemPool_t g_pool[64];

hipError_t pool_for(int dev, hipMemPool_t *out) {
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_pool_mu);
    if (!g_pool[dev]) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        hipError_t e = hipMemPoolCreate(&pool, &props);
        if (e != hipSuccess) return e;
        uint64_t thr = UINT64_MAX;
        (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr);
        g_pool[dev] = pool;
    }
    *out = g_pool[dev];
    return hipSuccess;
}

// Scratch reused across the calls on one stream.  Stream order keeps the
// calls on a stream from overlapping, so one buffer per (device, stream)
// suffices; a stream-ordered malloc/free pair in every call made the host
// wait for the device each time.  A call that needs more grows the buffer
// (the old one is freed in stream order).  The per-thread default stream is
// one handle for many streams, so that key also holds the calling thread.
// Each buffer carries an event recorded after its last use: a call first
// makes its stream wait for it, so that a stream created with the handle of a
// destroyed one that still has work queued cannot overlap that work.  At most
// kMaxCachedStreams buffers are kept; the least recently used one is freed
// in the order of the stream that evicts it, after its own last use.  The
// caller holds g_ws_mu from stream_scratch until it has queued its kernels
// and recorded the event.
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
    uint64_t last_use = 0;
};
std::mutex g_ws_mu;
std::map<WsKey, WsBuf> g_ws;
uint64_t g_ws_tick = 0;

hipError_t evict_lru(const WsKey &keep, hipStream_t stream) {
    auto victim = g_ws.end();
    for (auto it = g_ws.begin(); it != g_ws.end(); ++it)
        if (!(it->first.dev == keep.dev && it->first.stream == keep.stream &&
              it->first.thread == keep.thread) &&
            (victim == g_ws.end() || it->second.last_use < victim->second.last_use))
            victim = it;
    if (victim == g_ws.end()) return hipSuccess;
    WsBuf &v = victim->second;
    if (v.done) {
        const hipError_t e = hipStreamWaitEvent(stream, v.done, 0);
        if (e != hipSuccess) return e;
    }
    if (v.ptr) {
        const hipError_t e = hipFreeAsync(v.ptr, stream);
        if (e != hipSuccess) return e;
    }
    if (v.done) (void)hipEventDestroy(v.done);
    g_ws.erase(victim);
    return hipSuccess;
}

hipError_t stream_scratch(int dev, hipStream_t stream, size_t bytes, WsBuf **out) {
    const WsKey key{dev, stream,
                    stream == hipStreamPerThread ? std::this_thread::get_id() : std::thread::id()};
    hipMemPool_t pool;
    hipError_t e = pool_for(dev, &pool);
    if (e != hipSuccess) return e;
    WsBuf &b = g_ws[key];
    b.last_use = ++g_ws_tick;
    if (!b.done) {
        e = hipEventCreateWithFlags(&b.done, hipEventDisableTiming);
        if (e != hipSuccess) {
            b.done = nullptr;
            return e;
        }
    } else {
        e = hipStreamWaitEvent(stream, b.done, 0);
        if (e != hipSuccess) return e;
    }
    if (g_ws.size() > kMaxCachedStreams && (e = evict_lru(key, stream)) != hipSuccess) return e;
    WsBuf &bb = g_ws[key];
    if (bb.bytes < bytes) {
        size_t want = bytes + (bytes >> 2);
        want = (want + ((size_t)1 << 20) - 1) & ~(((size_t)1 << 20) - 1);
        void *np = nullptr;
        e = hipMallocFromPoolAsync(&np, want, pool, stream);
        if (e != hipSuccess) return e;
        if (bb.ptr) (void)hipFreeAsync(bb.ptr, stream);
        bb.ptr = np;
        bb.bytes = want;
        bb.clean_words = 0;
    }
    *out = &bb;
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
    case SEGTOPK_KEY_U16: return topk_per_cu<SEGTOPK_KEY_U16>(largest, lds);
    case SEGTOPK_KEY_I16: return topk_per_cu<SEGTOPK_KEY_I16>(largest, lds);
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
    case SEGTOPK_KEY_U64: return launch_topk_plain<SEGTOPK_KEY_U64>(p, largest, grid, lds, st);
    case SEGTOPK_KEY_I64: return launch_topk_plain<SEGTOPK_KEY_I64>(p, largest, grid, lds, st);
    case SEGTOPK_KEY_F64: return launch_topk_plain<SEGTOPK_KEY_F64>(p, largest, grid, lds, st);
    case SEGTOPK_KEY_U8: return launch_topk_plain<SEGTOPK_KEY_U8>(p, largest, grid, lds, st);
    case SEGTOPK_KEY_I8: return launch_topk_plain<SEGTOPK_KEY_I8>(p, largest, grid, lds, st);
    case SEGTOPK_KEY_F32: return launch_topk<SEGTOPK_KEY_F32>(p, largest, variant, grid, lds, st);
    case SEGTOPK_KEY_BF16: return launch_topk<SEGTOPK_KEY_BF16>(p, largest, variant, grid, lds, st);
    case SEGTOPK_KEY_U32: return launch_topk<SEGTOPK_KEY_U32>(p, largest, variant, grid, lds, st);
    case SEGTOPK_KEY_I32: return launch_topk<SEGTOPK_KEY_I32>(p, largest, variant, grid, lds, st);
    case SEGTOPK_KEY_U16: return launch_topk<SEGTOPK_KEY_U16>(p, largest, variant, grid, lds, st);
    case SEGTOPK_KEY_I16: return launch_topk<SEGTOPK_KEY_I16>(p, largest, variant, grid, lds, st);
    default: return launch_topk<SEGTOPK_KEY_F16>(p, largest, variant, grid, lds, st);
    }
}

struct Request {
    const segtopk_keys *keys;
    const segtopk_values *values;
    int32_t value_bytes;
    const int64_t *offsets;
    int64_t num_segments, k;
    const int32_t *kseg;
    int64_t max_seg;
    int direction, determinism, tie_break, ordering;
    hipStream_t stream;
};

// Everything the call queues, decided on the host from the request alone.
struct Plan {
    Params p;
    int type;
    bool largest;
    int variant;
    uint32_t grid;
    size_t lds;
    bool pairs, wide_values;
    // scratch: the order array (order), or the slice-mode layout (sliced)
    bool order, sliced;
    size_t scratch_bytes, zero_words, data_off, n_hist, n_early, info_words, stage_off;
};

int validate(const Request &r) {
    if (!r.keys) return SEGTOPK_INVALID_ARGUMENT;
    const int type = r.keys->type;
    if (type < SEGTOPK_KEY_F32 || type > SEGTOPK_KEY_I8) return SEGTOPK_INVALID_ARGUMENT;
    if (r.direction != SEGTOPK_MAX && r.direction != SEGTOPK_MIN) return SEGTOPK_INVALID_ARGUMENT;
    if (r.determinism < SEGTOPK_NOT_GUARANTEED || r.determinism > SEGTOPK_GPU_TO_GPU)
        return SEGTOPK_INVALID_ARGUMENT;
    if (r.tie_break < SEGTOPK_TIE_UNSPECIFIED || r.tie_break > SEGTOPK_PREFER_LARGER_INDEX)
        return SEGTOPK_INVALID_ARGUMENT;
    if (r.ordering < SEGTOPK_UNSORTED || r.ordering > SEGTOPK_STABLE_SORTED)
        return SEGTOPK_INVALID_ARGUMENT;
    // An explicit index tie-break pins the set across GPUs, so it must come
    // with gpu_to_gpu.   [docs "Top-K: Determinism ...", "Which items are selected?"]
    if (r.tie_break != SEGTOPK_TIE_UNSPECIFIED && r.determinism != SEGTOPK_GPU_TO_GPU)
        return SEGTOPK_INVALID_ARGUMENT;
    if (r.k < 0 || r.k > INT32_MAX || r.num_segments < 0 || r.num_segments > INT32_MAX)
        return SEGTOPK_INVALID_ARGUMENT;
    if (r.value_bytes != 4 && r.value_bytes != 8) return SEGTOPK_INVALID_ARGUMENT;
    if (r.num_segments == 0 || r.k == 0) return SEGTOPK_OK;
    if (!r.keys->in || !r.keys->out || !r.offsets) return SEGTOPK_INVALID_ARGUMENT;
    const bool pairs = r.values && r.values->in;
    if (pairs && !r.values->out) return SEGTOPK_INVALID_ARGUMENT;
    const uintptr_t kb = (uintptr_t)key_bytes(type);
    if ((reinterpret_cast<uintptr_t>(r.keys->in) % kb) ||
        (reinterpret_cast<uintptr_t>(r.keys->out) % kb))
        return SEGTOPK_INVALID_ARGUMENT;
    const uintptr_t vb = (uintptr_t)r.value_bytes;
    if (pairs && ((reinterpret_cast<uintptr_t>(r.values->in) % vb) ||
                  (reinterpret_cast<uintptr_t>(r.values->out) % vb)))
        return SEGTOPK_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(r.offsets) & 7)) return SEGTOPK_INVALID_ARGUMENT;
    if (r.kseg && (reinterpret_cast<uintptr_t>(r.kseg) & 3)) return SEGTOPK_INVALID_ARGUMENT;
    if (r.ordering != SEGTOPK_UNSORTED && r.k > SEGTOPK_MAX_SORTED_K) return SEGTOPK_NOT_SUPPORTED;
    return -1;  // valid, with work to do
}

// The launch plan.  Only host arithmetic and (for fewer than 2048 segments)
// the cached occupancy query of the sliced kernel.
int make_plan(const Request &r, int dev, Plan &pl) {
    const int type = r.keys->type;
    const bool pairs = r.values && r.values->in;
    const bool sorted = r.ordering != SEGTOPK_UNSORTED;
    const uint64_t k = (uint64_t)r.k;
    const uint64_t S = (uint64_t)r.num_segments;
    // The hint only sizes the plan, never a bound the kernels rely on.
    const uint64_t hint = r.max_seg > 0 ? (uint64_t)r.max_seg : 0u;
    const uint64_t k_eff = (hint && hint < k) ? hint : k;

    Params &p = pl.p;
    p = Params{};
    p.keys_in = r.keys->in;
    p.keys_out = r.keys->out;
    p.vals_in = pairs ? static_cast<const uint32_t *>(r.values->in) : nullptr;
    p.vals_out = pairs ? static_cast<uint32_t *>(r.values->out) : nullptr;
    p.offsets = r.offsets;
    p.num_segments = r.num_segments;
    p.kseg = r.kseg;
    p.k = (uint32_t)k;
    p.det = r.determinism != SEGTOPK_NOT_GUARANTEED;
    p.prefer_larger = r.tie_break == SEGTOPK_PREFER_LARGER_INDEX;
    p.sorted = sorted;
    pl.wide_values = pairs && r.value_bytes == 8;
    p.vindex = pl.wide_values ? 1u : 0u;
    p.vshift = pl.wide_values ? 1u : 0u;

    if (is_plain_key(type)) {
        // 64-bit and 8-bit keys: one workgroup per segment, no scratch;
        // dynamic LDS holds the candidate list and the output staging (16
        // bytes an entry).
        uint64_t oc = 0;
        if (sorted || k <= 256) oc = next_pow2(k < 2 ? 2 : k);
        p.out_cap = (uint32_t)oc;
        p.stash_cap = kPlainCand;
        p.wg_per_seg = 1;
        pl.lds = 16 * (size_t)(kPlainCand + oc);
        if (pl.lds > kMaxDynLds) return SEGTOPK_NOT_SUPPORTED;
        pl.largest = r.direction == SEGTOPK_MAX;
        pl.type = type;
        pl.pairs = pairs;
        pl.grid = (uint32_t)S;
        pl.variant = kVariantOne;
        pl.order = pl.sliced = false;
        pl.scratch_bytes = pl.zero_words = pl.data_off = pl.n_hist = pl.n_early = pl.info_words = pl.stage_off = 0;
        return SEGTOPK_OK;
    }

    // Output staging: sorted output is staged and sorted in LDS (k is at most
    // SEGTOPK_MAX_SORTED_K then); unsorted output only for small k (coalesced
    // row writes), else written in place.  Sized by k, never by the hint: a
    // segment may exceed the hint.
    uint64_t out_cap = next_pow2(k < 2 ? 2 : (k > 8192 ? 8192 : k));
    if (!sorted && out_cap > 256) out_cap = 0;
    // Several workgroups per segment when the segments alone cannot fill the
    // device, unless the hint says no segment is long enough to be split.
    const bool many = S >= kTargetWorkgroups;
    uint64_t min_slice = kMinSlice;
    if (8 * k > min_slice) min_slice = 8 * k > (1ull << 30) ? (1ull << 30) : 8 * k;
    const bool split = !many && !(hint && hint <= min_slice);
    // Stash: with one workgroup per segment, room for about eight times k
    // candidates in four wave regions; with several, the segment-wide bound
    // keeps each slice's candidates few, and the stash only has to hold
    // bucket b* of the last arriver (about 2k at most).
    uint64_t stash = (split ? 2 : 8) * k_eff;
    if (stash > 8192) stash = 8192;
    uint64_t stash_cap = next_pow2(stash < 1 ? 1 : stash);
    if (stash_cap < (split ? 2048u : 1024u)) stash_cap = split ? 2048u : 1024u;
    // The sliced kernel also keeps a workgroup's shared-histogram
    // contributions in LDS (kBuckets words after the stash and the staging).
    // The kernels for 16-bit keys with one workgroup per segment keep rings
    // of loads waiting to be tested there instead.
    const uint64_t extra = split ? 4u * kBuckets : 0u;
    const uint64_t ring = key_bytes(type) == 2 ? kRingBytes : 0u;
    const uint64_t more = extra > ring ? extra : ring;
    while (stash_cap > 1024 && 8 * (stash_cap + out_cap) + more > kMaxDynLds) stash_cap >>= 1;
    if (8 * (stash_cap + out_cap) + more > kMaxDynLds) return SEGTOPK_NOT_SUPPORTED;
    p.stash_cap = (uint32_t)stash_cap;
    p.out_cap = (uint32_t)out_cap;
    pl.lds = 8 * (size_t)(stash_cap + out_cap) + (size_t)ring;
    const size_t lds_sliced = 8 * (size_t)(stash_cap + out_cap) + (size_t)extra;
    pl.largest = r.direction == SEGTOPK_MAX;
    pl.type = type;
    pl.pairs = pairs;

    uint64_t P = 1;
    if (split) {
        // As many workgroups as the device holds at once, so that all the
        // slices of a segment run together and share their bound.
        const uint64_t target = resident_wgs_for(type, dev, pl.largest, lds_sliced);
        if (S < 8) {
            P = target / S;  // every slice of every segment resident at once
        } else {
            P = (target + S - 1) / S;
        }
        if (P > kMaxWgPerSeg) P = kMaxWgPerSeg;
        if (P < 1) P = 1;
        if (2 * k > stash_cap) P = 1;  // slices could not hold their local candidates
    }
    p.wg_per_seg = (uint32_t)P;
    p.min_slice = (uint32_t)min_slice;
    p.spread = (split && S < 8 && P > 1) ? 1u : 0u;
    // With one workgroup per segment workgroup b serves segment b; with
    // several, the XCD-local mapping rounds the batch up to a multiple of 8.
    const uint64_t grid = P == 1 ? S : (p.spread ? S * P : (S + 7) / 8 * 8 * P);
    if (grid > 0x7FFFFFFFull) return SEGTOPK_NOT_SUPPORTED;
    pl.grid = (uint32_t)grid;
    pl.variant = many ? kVariantOne : (P > 1 ? kVariantSliced : kVariantSplit);
    if (P > 1) pl.lds = lds_sliced;
    // Every segment within one load of four per lane in each wave (by the
    // hint): the kernel that holds only that path.
    const uint64_t small = key_bytes(type) == 2 ? kSmallKeys16 : kSmallKeys32;
    if (P == 1 && hint && hint <= small) {
        pl.variant = kVariantSmall;
        pl.grid = (uint32_t)S;
        pl.lds = 8 * (size_t)(stash_cap + out_cap);
    }

    // Scratch.  One workgroup per segment for many segments of unknown sizes
    // (not all within one chunk by the hint): process the largest first.
    pl.order = split && P == 1 && S >= (uint64_t)kOrderMinSegments && !(hint && hint <= 8192) &&
               pl.variant != kVariantSmall;
    pl.sliced = P > 1;
    pl.scratch_bytes = pl.zero_words = pl.data_off = pl.n_hist = pl.n_early = pl.info_words = pl.stage_off = 0;
    if (pl.order) {
        pl.scratch_bytes = S * sizeof(uint32_t);
    } else if (pl.sliced) {
        // A segment spread over every XCD keeps one shared histogram per XCD.
        pl.n_hist = S * kBuckets;
        pl.n_early = (p.spread ? 8u : 1u) * pl.n_hist;
        pl.zero_words = pl.n_hist + pl.n_early + S;  // merged and shared histograms, tickets
        pl.info_words = S * P * 4;
        const size_t cum_words = S * P * kBuckets;
        size_t bytes = (pl.zero_words + pl.info_words + cum_words) * 4;
        bytes = (bytes + 255) & ~(size_t)255;
        pl.data_off = bytes;
        pl.scratch_bytes = bytes + S * P * (size_t)stash_cap * sizeof(uint2);
        if (p.spread) {
            pl.stage_off = pl.scratch_bytes;
            pl.scratch_bytes += S * (size_t)kStageCap * sizeof(uint2);
        }
    }
    return SEGTOPK_OK;
}

// Points the plan's scratch fields into `ws`.
void bind_scratch(Plan &pl, void *ws) {
    Params &p = pl.p;
    uint32_t *wsw = static_cast<uint32_t *>(ws);
    if (pl.order) {
        p.order = wsw;
    } else if (pl.sliced) {
        p.ws_hist = wsw;
        p.ws_early = wsw + pl.n_hist;
        p.ws_ticket = wsw + pl.n_hist + pl.n_early;
        p.ws_slot_info = wsw + pl.zero_words;
        p.ws_slot_cum = wsw + pl.zero_words + pl.info_words;
        p.ws_slot_data = reinterpret_cast<uint2 *>(static_cast<char *>(ws) + pl.data_off);
        p.ws_stage = pl.stage_off ? reinterpret_cast<uint2 *>(static_cast<char *>(ws) + pl.stage_off)
                                  : nullptr;
    }
}

// Queues the plan's kernels on `stream`: the clearing kernel when asked, the
// order kernel, the selection, and the 8-byte value gather.
hipError_t queue(const Request &r, const Plan &pl, bool clear, hipStream_t stream) {
    hipError_t err = hipSuccess;
    if (clear) {
        size_t zb = (pl.zero_words + 255) / 256;
        if (zb > 1024) zb = 1024;
        if (zb < 1) zb = 1;
        hipLaunchKernelGGL(zero_kernel, dim3((unsigned)zb), dim3(256), 0, stream,
                           const_cast<uint32_t *>(pl.p.ws_hist), pl.zero_words);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (pl.order) {
        hipLaunchKernelGGL(order_kernel, dim3(1), dim3(1024), 0, stream, r.offsets,
                           r.num_segments, const_cast<uint32_t *>(pl.p.order));
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    err = launch(pl.type, pl.p, pl.largest, pl.variant, pl.grid, pl.lds, stream);
    if (err != hipSuccess) return err;
    if (pl.wide_values) {
        const uint64_t total = (uint64_t)r.num_segments * (uint64_t)r.k;
        uint64_t blocks = (total + 255) / 256;
        if (blocks > 4096) blocks = 4096;
        hipLaunchKernelGGL(gather64_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                           r.offsets, r.kseg, r.num_segments, (uint32_t)r.k,
                           static_cast<const uint64_t *>(r.values->in),
                           static_cast<uint64_t *>(r.values->out));
        err = hipGetLastError();
    }
    return err;
}

int run(const Request &r) {
    const int v = validate(r);
    if (v >= 0) return v;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SEGTOPK_HIP_ERROR;
    Plan pl;
    const int ps = make_plan(r, dev, pl);
    if (ps != SEGTOPK_OK) return ps;
    const hipStream_t stream = r.stream;
    if (pl.scratch_bytes == 0)
        return queue(r, pl, false, stream) == hipSuccess ? SEGTOPK_OK : SEGTOPK_HIP_ERROR;

    // The scratch cache decides on the host what the stream's buffer holds;
    // a captured graph would replay those decisions against a buffer that
    // may have been regrown or dirtied since.
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return SEGTOPK_HIP_ERROR;
    if (cs != hipStreamCaptureStatusNone) return SEGTOPK_NOT_SUPPORTED;

    std::lock_guard<std::mutex> lk(g_ws_mu);
    WsBuf *wsb = nullptr;
    if (stream_scratch(dev, stream, pl.scratch_bytes, &wsb) != hipSuccess) return SEGTOPK_HIP_ERROR;
    bind_scratch(pl, wsb->ptr);
    bool clear = false;
    if (pl.order) {
        wsb->clean_words = 0;  // the order overwrites the front
    } else {
        clear = wsb->clean_words < pl.zero_words;
        // The slots (after the cleared words) are written by this call; the
        // sliced kernel clears the histograms and tickets it used.
        wsb->clean_words = 0;
    }
    hipError_t err = queue(r, pl, clear, stream);
    if (err == hipSuccess && pl.sliced) wsb->clean_words = pl.zero_words;
    const hipError_t e = hipEventRecord(wsb->done, stream);
    if (err == hipSuccess) err = e;
    return err == hipSuccess ? SEGTOPK_OK : SEGTOPK_HIP_ERROR;
}

// ---------------------------------------------------------------------------
// Scratch without allocation: one file-scope device array.  The library never
// passes the array's name to a kernel or a copy (in host code it is a
// host-side stand-in, not a device address); it takes each device's address
// of it once, with hipGetSymbolAddress, and uses that.  Every call on a device
// shares the array, so calls that overlap on one device race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[SEGTOPK_STATIC_SCRATCH_BYTES];

std::mutex g_static_mu;
void *g_static_ptr[64];

hipError_t static_scratch(int dev, void **out) {
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_static_mu);
    if (!g_static_ptr[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_static_ptr[dev] = ptr;
    }
    *out = g_static_ptr[dev];
    return hipSuccess;
}

int run_noalloc(const Request &r) {
    const int v = validate(r);
    if (v >= 0) return v;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SEGTOPK_HIP_ERROR;
    Plan pl;
    const int ps = make_plan(r, dev, pl);
    if (ps != SEGTOPK_OK) return ps;
    if (pl.scratch_bytes > (size_t)SEGTOPK_STATIC_SCRATCH_BYTES) return SEGTOPK_SCRATCH_TOO_SMALL;
    bool clear = false;
    if (pl.scratch_bytes) {
        void *ptr = nullptr;
        if (static_scratch(dev, &ptr) != hipSuccess) return SEGTOPK_HIP_ERROR;
        bind_scratch(pl, ptr);
        // The array keeps whatever the last call left: clear the words that
        // must start at zero every time.
        clear = pl.sliced;
    }
    return queue(r, pl, clear, r.stream) == hipSuccess ? SEGTOPK_OK : SEGTOPK_HIP_ERROR;
}

}  // namespace

extern "C" int batched_topk(const segtopk_keys *keys, const segtopk_values *values,
                            const int64_t *segment_offsets, int64_t num_segments, int64_t k,
                            int direction, int determinism, int tie_break, int ordering,
                            hipStream_t stream) {
    const Request r{keys, values, 4, segment_offsets, num_segments, k, nullptr, 0,
                    direction, determinism, tie_break, ordering, stream};
    return run(r);
}

extern "C" int batched_topk_ex(const segtopk_keys *keys, const segtopk_values *values,
                               int32_t value_bytes, const int64_t *segment_offsets,
                               int64_t num_segments, int64_t k, const int32_t *k_per_segment,
                               int64_t max_segment_size, int direction, int determinism,
                               int tie_break, int ordering, hipStream_t stream) {
    const Request r{keys, values, value_bytes, segment_offsets, num_segments, k, k_per_segment,
                    max_segment_size, direction, determinism, tie_break, ordering, stream};
    return run(r);
}

extern "C" int batched_topk_ex_noalloc(const segtopk_keys *keys, const segtopk_values *values,
                                       int32_t value_bytes, const int64_t *segment_offsets,
                                       int64_t num_segments, int64_t k,
                                       const int32_t *k_per_segment, int64_t max_segment_size,
                                       int direction, int determinism, int tie_break,
                                       int ordering, hipStream_t stream) {
    const Request r{keys, values, value_bytes, segment_offsets, num_segments, k, k_per_segment,
                    max_segment_size, direction, determinism, tie_break, ordering, stream};
    return run_noalloc(r);
}

extern "C" const char *segtopk_status_string(int status) {
    switch (status) {
    case SEGTOPK_OK: return "ok";
    case SEGTOPK_INVALID_ARGUMENT: return "invalid argument";
    case SEGTOPK_NOT_SUPPORTED: return "not supported";
    case SEGTOPK_HIP_ERROR: return "HIP error";
    case SEGTOPK_SCRATCH_TOO_SMALL: return "request needs more scratch than the static buffer holds";
    default: return "unknown status";
    }
}

extern "C" int segtopk_version(void) { return 300; }
