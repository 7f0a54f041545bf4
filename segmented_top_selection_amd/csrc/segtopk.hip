// segtopk.hip -- segmented (batched) top-k for gfx950 (AMD Instinct MI355X).
//
// Method: most-significant-digit radix selection.  Each pass builds a histogram
// of one digit over the surviving candidates, scans it best-first to find the
// bucket that holds the k-th key, narrows k and the candidate set to that bucket
// and folds the digit into the splitter.  When the chosen bucket holds exactly
// the remaining k candidates the passes stop early.  A final filter writes every
// key beyond the splitter plus exactly enough splitter-equal keys.
//   [PR "Implement Segmented TopK using Thread-Block-Clusters", §1.2 Radix
//    (digit) top-k, §1.4 Early stop, §1.5 Final filter and output placement]
//
// How it is laid out on gfx950 (differences from the pages' cluster design):
//
//  * One read of the keys.  Pass 0 streams the keys from HBM once.  A key is
//    counted in the pass-0 histogram and copied, with its index, into an LDS
//    "stash" only if its bucket can still hold the k-th key: the bound is the
//    k-th best bucket of the keys seen so far, which can only improve as more
//    keys arrive, so every key that the final result needs is counted and
//    stashed, and the counts of all buckets at or before the final k-th bucket
//    are exact.  Later passes, the tie selection and the output read only the
//    stash.  If a segment's candidates do not fit the stash (heavy ties, huge k)
//    the later passes re-stream the keys from memory instead.
//  * Buckets are reversed for MAX (bucket = B-1-digit) instead of inverting the
//    key bits, after -0.0 has been folded onto +0.0 in the order-preserving bit
//    transform.   [PR "Fix BlockTopK +/-0.0 handling", Fix]
//  * Deterministic tie-break: the splitter-equal keys are narrowed further by
//    radix passes over their source index (ascending digits for
//    prefer_smaller_index, reversed for prefer_larger_index), so exactly the
//    required number of ties is picked without an index-ordered scan.
//    not_guaranteed takes ties in arrival order behind an `out < k` guard.
//    [PR "Implement Segmented TopK ...", §1.6 Determinism / tie-breaking]
//  * A batch of few, long segments spreads each segment over several
//    workgroups.  Each streams its slice with the scheme above, adds its
//    histogram to a per-segment global histogram with atomics, writes its
//    stash to a global slot and takes a ticket; the last arriver scans the merged
//    histogram and finishes the segment from the slots.  (CDNA4 has no thread
//    block clusters; this replaces the cluster's DSMEM merge into a leader.)
//  * sorted / stable_sorted output is a bitonic sort of the k results in LDS on
//    (ordered key best-first, source index ascending).
//    [docs "Top-K: Determinism, Tie-Breaking, and Output Ordering", Output
//     ordering]
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>

#include "segtopk.h"

namespace {

constexpr int kThreads = 256;           // four wave64 per workgroup
constexpr int kDigit = 11;              // digit width of every radix pass
constexpr int kBuckets = 1 << kDigit;   // 2048 histogram buckets
constexpr uint32_t kNone = 0xFFFFFFFFu; // "no element" / sort sentinel

// ---------------------------------------------------------------------------
// Order-preserving bit transform.  ord(a) < ord(b) exactly when a < b, and
// ord(-0.0) == ord(+0.0).  The original bits are kept for output.
// ---------------------------------------------------------------------------
template <int KT> struct Key;

template <> struct Key<SEGTOPK_KEY_F32> {
    static constexpr int kBits = 32, kBytes = 4;
    __device__ __forceinline__ static uint32_t ord(uint32_t r) {
        r = (r == 0x80000000u) ? 0u : r;  // -0.0 joins +0.0
        return r ^ ((uint32_t)((int32_t)r >> 31) | 0x80000000u);
    }
};
template <> struct Key<SEGTOPK_KEY_BF16> {
    static constexpr int kBits = 16, kBytes = 2;
    __device__ __forceinline__ static uint32_t ord(uint32_t r) {
        r = (r == 0x8000u) ? 0u : r;
        return r ^ ((r & 0x8000u) ? 0xFFFFu : 0x8000u);
    }
};
template <> struct Key<SEGTOPK_KEY_F16> {
    static constexpr int kBits = 16, kBytes = 2;
    __device__ __forceinline__ static uint32_t ord(uint32_t r) {
        r = (r == 0x8000u) ? 0u : r;
        return r ^ ((r & 0x8000u) ? 0xFFFFu : 0x8000u);
    }
};
template <> struct Key<SEGTOPK_KEY_U32> {
    static constexpr int kBits = 32, kBytes = 4;
    __device__ __forceinline__ static uint32_t ord(uint32_t r) { return r; }
};
template <> struct Key<SEGTOPK_KEY_I32> {
    static constexpr int kBits = 32, kBytes = 4;
    __device__ __forceinline__ static uint32_t ord(uint32_t r) { return r ^ 0x80000000u; }
};

// ---------------------------------------------------------------------------
// Wave helpers (wave64).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
    const int ln = (int)lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t y = __shfl_up(x, (unsigned)d, 64);
        if (ln >= d) x += y;
    }
    return x;
}

// Reserves one slot per lane with `pred` from an LDS counter, with one atomic
// per wave; returns this lane's slot (meaningless where !pred).
__device__ __forceinline__ uint32_t wave_reserve(uint32_t *ctr, bool pred) {
    const uint64_t m = __ballot(pred);
    if (m == 0) return 0;
    const uint32_t leader = (uint32_t)__ffsll((unsigned long long)m) - 1u;
    uint32_t base = 0;
    if (lane_id() == leader) base = atomicAdd(ctr, (uint32_t)__popcll(m));
    base = __shfl(base, (int)leader, 64);
    return base + lanes_below(m);
}

// ---------------------------------------------------------------------------
// Kernel arguments and per-workgroup LDS.
// ---------------------------------------------------------------------------
struct Params {
    const void *keys_in;
    void *keys_out;
    const uint32_t *vals_in;  // nullptr: keys only
    uint32_t *vals_out;
    const int64_t *offsets;
    int64_t num_segments;
    uint32_t k;              // output row stride
    uint32_t det;            // deterministic tie-break requested
    uint32_t prefer_larger;  // ties toward larger source indices
    uint32_t sorted;         // sorted or stable_sorted output
    uint32_t stash_cap;      // LDS stash entries
    uint32_t out_cap;        // LDS output staging entries (power of two), 0 = none
    uint32_t wg_per_seg;     // workgroups per segment (1: one workgroup each)
    uint32_t min_slice;      // smallest slice a segment is split into
    uint32_t *ws_hist;       // [num_segments][kBuckets]   merged pass-0 histograms
    uint32_t *ws_ticket;     // [num_segments]             arrival tickets
    uint32_t *ws_slot_info;  // [num_segments][wg_per_seg][2] (count, overflowed)
    uint2 *ws_slot_data;     // [num_segments][wg_per_seg][stash_cap]
};

struct alignas(16) Smem {
    uint32_t hist[kBuckets];
    uint32_t touched[3];     // a chunk changed the histogram (rotating flags)
    uint32_t pending[3];     // stash entries a chunk wants to add (rotating)
    uint32_t stash_count;
    uint32_t stash_bad;      // the stash lost candidates: re-stream instead
    uint32_t res[4];         // find_kth result: found, bucket, count before, count in
    uint32_t ctr[2];         // output placement counters (better, tie)
    uint32_t compact_ctr;
    uint32_t snap;           // stash_count as seen before a chunk's pushes
    uint32_t flag;
};

struct Seg {
    int64_t begin;  // first element of the segment in keys_in / vals_in
    uint32_t n;     // segment size
    uint32_t k_i;   // min(k, n)
    int64_t row;    // output row
};

// ---------------------------------------------------------------------------
// Smallest bucket b < nb with hist[0] + ... + hist[b] >= target, found by
// wave 0 alone.  res = {found, b, sum before b, hist[b]}; found = 0 when the
// buckets hold fewer than `target` keys.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void find_kth(const uint32_t *hist, uint32_t nb, uint32_t target, uint32_t *res) {
    const uint32_t ln = lane_id();
    uint32_t per = (nb + 63u) >> 6;
    per = (per + 3u) & ~3u;
    const uint32_t b0 = ln * per;
    uint32_t s = 0;
    for (uint32_t q = 0; q < per; q += 4) {
        const uint32_t b = b0 + q;
        if (b < nb) {
            const uint4 h = *reinterpret_cast<const uint4 *>(&hist[b]);
            s += h.x + (b + 1 < nb ? h.y : 0u) + (b + 2 < nb ? h.z : 0u) + (b + 3 < nb ? h.w : 0u);
        }
    }
    const uint32_t incl = wave_incl_sum(s);
    const uint32_t excl = incl - s;
    const uint64_t hit = __ballot(excl < target && incl >= target);
    if (hit == 0) {
        if (ln == 0) {
            res[0] = 0;
            res[1] = nb - 1;
            res[2] = 0;
            res[3] = 0;
        }
        return;
    }
    const uint32_t L = (uint32_t)__ffsll((unsigned long long)hit) - 1u;
    if (ln == L) {
        uint32_t acc = excl;
        for (uint32_t q = 0; q < per; ++q) {
            const uint32_t h = hist[b0 + q];
            if (acc + h >= target) {
                res[0] = 1;
                res[1] = b0 + q;
                res[2] = acc;
                res[3] = h;
                break;
            }
            acc += h;
        }
    }
}

// ---------------------------------------------------------------------------
// Coalesced reader of the keys [lo, hi) of one segment: an unaligned head and
// tail (fewer than 16 bytes each) are read element by element, the aligned body
// with 16-byte loads, kU loads per thread per chunk.
// ---------------------------------------------------------------------------
template <int KT> struct Range {
    static constexpr int kBytes = Key<KT>::kBytes;
    static constexpr int kVec = 16 / kBytes;  // keys per 16-byte load
    static constexpr int kU = 4;              // loads per thread per chunk
    static constexpr int kKpt = kU * kVec;    // keys per thread per chunk
    static constexpr uint32_t kChunkVecs = kThreads * kU;

    const unsigned char *ebase;  // element 0 of the segment
    const uint4 *vbase;          // first aligned vector of the range
    uint32_t lo, head, nvec, tail_lo, nscalar, nchunks;

    __device__ void init(const void *keys, int64_t begin, uint32_t lo_, uint32_t hi_) {
        ebase = static_cast<const unsigned char *>(keys) + begin * kBytes;
        lo = lo_;
        const uint32_t len = hi_ - lo_;
        const uintptr_t a = reinterpret_cast<uintptr_t>(ebase + (size_t)lo_ * kBytes);
        const uint32_t h = (uint32_t)(((16u - (a & 15u)) & 15u) / kBytes);
        head = h < len ? h : len;
        nvec = (len - head) / kVec;
        tail_lo = lo + head + nvec * kVec;
        nscalar = head + (hi_ - tail_lo);
        vbase = reinterpret_cast<const uint4 *>(ebase + (size_t)(lo + head) * kBytes);
        nchunks = (nvec + kChunkVecs - 1) / kChunkVecs;
    }
    __device__ __forceinline__ uint32_t scalar_idx(uint32_t s) const {
        return s < head ? lo + s : tail_lo + (s - head);
    }
    __device__ __forceinline__ uint32_t load_scalar(uint32_t idx) const {
        if (kBytes == 4) return reinterpret_cast<const uint32_t *>(ebase)[idx];
        return reinterpret_cast<const uint16_t *>(ebase)[idx];
    }
    // Thread t's part of chunk c: raw[u * kVec + e] is element vidx[u] + e;
    // vidx[u] == kNone marks a load past the end.
    __device__ __forceinline__ void load_chunk(uint32_t c, uint32_t t, uint32_t (&raw)[kKpt],
                                               uint32_t (&vidx)[kU]) const {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const uint32_t vj = c * kChunkVecs + (uint32_t)u * kThreads + t;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            vidx[u] = kNone;
            if (vj < nvec) {
                v = vbase[vj];
                vidx[u] = lo + head + vj * kVec;
            }
            if (kBytes == 4) {
                raw[u * 4 + 0] = v.x;
                raw[u * 4 + 1] = v.y;
                raw[u * 4 + 2] = v.z;
                raw[u * 4 + 3] = v.w;
            } else {
                raw[u * 8 + 0] = v.x & 0xFFFFu;
                raw[u * 8 + 1] = v.x >> 16;
                raw[u * 8 + 2] = v.y & 0xFFFFu;
                raw[u * 8 + 3] = v.y >> 16;
                raw[u * 8 + 4] = v.z & 0xFFFFu;
                raw[u * 8 + 5] = v.z >> 16;
                raw[u * 8 + 6] = v.w & 0xFFFFu;
                raw[u * 8 + 7] = v.w >> 16;
            }
        }
    }
    // Calls f(raw, idx, active) for every element, chunk by chunk; every lane
    // of every wave makes the same sequence of calls.
    template <class F> __device__ __forceinline__ void for_each(uint32_t t, F &&f) const {
        {
            const bool act = t < nscalar;
            const uint32_t idx = act ? scalar_idx(t) : 0u;
            f(act ? load_scalar(idx) : 0u, idx, act);
        }
        for (uint32_t c = 0; c < nchunks; ++c) {
            uint32_t raw[kKpt], vidx[kU];
            load_chunk(c, t, raw, vidx);
#pragma unroll
            for (int u = 0; u < kU; ++u)
#pragma unroll
                for (int e = 0; e < kVec; ++e)
                    f(raw[u * kVec + e], vidx[u] + (uint32_t)e, vidx[u] != kNone);
        }
    }
};

// Pass-0 bucket rank of an ordered key: 0 is the best bucket.
template <int KT, bool LARGEST> __device__ __forceinline__ uint32_t rank0(uint32_t o) {
    constexpr int sh = Key<KT>::kBits - kDigit;
    const uint32_t d = o >> sh;
    return LARGEST ? (uint32_t)(kBuckets - 1) - d : d;
}

// Ordered-key threshold of "rank0 <= R": for MAX o >= thr, for MIN o <= thr.
template <int KT, bool LARGEST> __device__ __forceinline__ uint32_t rank_thr(uint32_t R) {
    constexpr int sh = Key<KT>::kBits - kDigit;
    return LARGEST ? ((uint32_t)(kBuckets - 1) - R) << sh
                   : (R << sh) | ((1u << sh) - 1u);
}
template <bool LARGEST> __device__ __forceinline__ bool within(uint32_t o, uint32_t thr) {
    return LARGEST ? o >= thr : o <= thr;
}

// ---------------------------------------------------------------------------
// Stash maintenance.
// ---------------------------------------------------------------------------

// Drops, in place, every stash entry whose pass-0 rank is beyond R.
// All threads call it; it contains barriers.
template <int KT, bool LARGEST>
__device__ __forceinline__ uint32_t compact_stash(Smem &sm, uint2 *stash, uint32_t cnt, uint32_t R) {
    const uint32_t t = threadIdx.x;
    const uint32_t thr = rank_thr<KT, LARGEST>(R);
    if (t == 0) sm.compact_ctr = 0;
    __syncthreads();
    constexpr int kR = 4;
    for (uint32_t base = 0; base < cnt; base += kR * kThreads) {
        uint2 e[kR];
        bool keep[kR];
#pragma unroll
        for (int r = 0; r < kR; ++r) {
            const uint32_t i = base + (uint32_t)r * kThreads + t;
            keep[r] = false;
            if (i < cnt) {
                e[r] = stash[i];
                keep[r] = within<LARGEST>(Key<KT>::ord(e[r].x), thr);
            }
        }
        __syncthreads();  // every read of this round precedes every write
#pragma unroll
        for (int r = 0; r < kR; ++r) {
            const uint32_t pos = wave_reserve(&sm.compact_ctr, keep[r]);
            if (keep[r]) stash[pos] = e[r];
        }
    }
    __syncthreads();
    if (t == 0) sm.stash_count = sm.compact_ctr;
    __syncthreads();
    return sm.compact_ctr;  // unchanged until the next compaction
}

// ---------------------------------------------------------------------------
// Pass 0 over the keys [lo, hi) of a segment: the filtered histogram and the
// stash.  Returns the final bound R; sm.res holds the find result for R
// (res[0] == 0 when the range holds fewer than `target` keys, then R is the
// last bucket and every key was kept).  sm.stash_bad says whether the stash
// holds every key with rank <= R.
// ---------------------------------------------------------------------------
template <int KT, bool LARGEST>
__device__ __forceinline__ uint32_t pass0(Smem &sm, uint2 *stash, uint32_t cap, const Params &p, const Seg &sg,
                          uint32_t lo, uint32_t hi, uint32_t target) {
    using Rg = Range<KT>;
    constexpr int K = Rg::kKpt;
    const uint32_t t = threadIdx.x;
    const uint32_t wave = t >> 6;

    for (uint32_t i = t; i < (uint32_t)kBuckets; i += kThreads) sm.hist[i] = 0;
    if (t == 0) {
        sm.touched[0] = sm.touched[1] = sm.touched[2] = 0;
        sm.pending[0] = sm.pending[1] = sm.pending[2] = 0;
        sm.stash_count = 0;
        sm.stash_bad = 0;
        sm.res[0] = 0;
        sm.res[1] = kBuckets - 1;
        sm.res[2] = 0;
        sm.res[3] = 0;
    }

    Rg L;
    L.init(p.keys_in, sg.begin, lo, hi);
    const uint32_t nch = L.nchunks > 0 ? L.nchunks : 1u;

    uint32_t R = kBuckets - 1;  // until `target` keys are seen every bucket may hold the k-th
    bool bad = false;
    uint32_t raw[K], vidx[Rg::kU];
    L.load_chunk(0, t, raw, vidx);
    __syncthreads();

    for (uint32_t c = 0; c < nch; ++c) {
        // This chunk's keys, and in chunk 0 one key of the unaligned head/tail.
        uint32_t cur[K], cv[Rg::kU];
#pragma unroll
        for (int j = 0; j < K; ++j) cur[j] = raw[j];
#pragma unroll
        for (int u = 0; u < Rg::kU; ++u) cv[u] = vidx[u];
        const bool sv = (c == 0) && t < L.nscalar;
        const uint32_t si = sv ? L.scalar_idx(t) : 0u;
        const uint32_t sr = sv ? L.load_scalar(si) : 0u;

        // Prefetch the next chunk while this one is counted.
        if (c + 1 < nch) L.load_chunk(c + 1, t, raw, vidx);

        // 1. Count keys whose bucket can still hold the k-th key.
        const uint32_t thr = rank_thr<KT, LARGEST>(R);
        bool any = false;
#pragma unroll
        for (int u = 0; u < Rg::kU; ++u)
#pragma unroll
            for (int e = 0; e < Rg::kVec; ++e) {
                const uint32_t o = Key<KT>::ord(cur[u * Rg::kVec + e]);
                if (cv[u] != kNone && within<LARGEST>(o, thr)) {
                    atomicAdd(&sm.hist[rank0<KT, LARGEST>(o)], 1u);
                    any = true;
                }
            }
        if (sv) {
            const uint32_t o = Key<KT>::ord(sr);
            if (within<LARGEST>(o, thr)) {
                atomicAdd(&sm.hist[rank0<KT, LARGEST>(o)], 1u);
                any = true;
            }
        }
        if (__any(any) && lane_id() == 0) sm.touched[c % 3] = 1;
        if (t == 0) {
            sm.touched[(c + 1) % 3] = 0;
            sm.pending[(c + 1) % 3] = 0;
        }
        __syncthreads();
        if (!sm.touched[c % 3]) continue;  // uniform: bound and stash unchanged

        // 2. New bound: the k-th best bucket of everything counted so far.
        if (wave == 0) find_kth(sm.hist, R + 1, target, sm.res);
        __syncthreads();
        if (sm.res[0]) R = sm.res[1];
        if (bad) continue;

        // 3. Stash this chunk's keys within the new bound.
        const uint32_t thr2 = rank_thr<KT, LARGEST>(R);
        uint32_t cnt = (sv && within<LARGEST>(Key<KT>::ord(sr), thr2)) ? 1u : 0u;
#pragma unroll
        for (int u = 0; u < Rg::kU; ++u)
#pragma unroll
            for (int e = 0; e < Rg::kVec; ++e)
                cnt += (cv[u] != kNone && within<LARGEST>(Key<KT>::ord(cur[u * Rg::kVec + e]), thr2))
                           ? 1u : 0u;
        {
            const uint32_t wsum = __shfl(wave_incl_sum(cnt), 63, 64);
            if (lane_id() == 0 && wsum) atomicAdd(&sm.pending[c % 3], wsum);
        }
        // No push has started yet, so every thread sees the same count.
        if (t == 0) sm.snap = sm.stash_count;
        __syncthreads();
        const uint32_t need = sm.pending[c % 3];
        uint32_t have = sm.snap;
        if (have + need > cap) {
            have = compact_stash<KT, LARGEST>(sm, stash, have, R);
            if (have + need > cap) {
                bad = true;  // uniform: every thread read the same counts
                if (t == 0) sm.stash_bad = 1;
                continue;
            }
        }
        // Append (one LDS atomic per wave).
        const uint32_t incl = wave_incl_sum(cnt);
        const uint32_t total = __shfl(incl, 63, 64);
        if (total) {
            uint32_t base = 0;
            if (lane_id() == 0) base = atomicAdd(&sm.stash_count, total);
            uint32_t pos = __shfl(base, 0, 64) + incl - cnt;
            if (sv && within<LARGEST>(Key<KT>::ord(sr), thr2)) stash[pos++] = make_uint2(sr, si);
#pragma unroll
            for (int u = 0; u < Rg::kU; ++u)
#pragma unroll
                for (int e = 0; e < Rg::kVec; ++e) {
                    const uint32_t r = cur[u * Rg::kVec + e];
                    if (cv[u] != kNone && within<LARGEST>(Key<KT>::ord(r), thr2))
                        stash[pos++] = make_uint2(r, cv[u] + (uint32_t)e);
                }
        }
    }
    __syncthreads();
    return R;
}

// ---------------------------------------------------------------------------
// Candidate sources for the passes after pass 0.
// ---------------------------------------------------------------------------
template <int KT> struct Cands {
    // LDS stash ...
    const uint2 *stash;
    uint32_t count;
    bool lds;
    // ... or global memory: nslots slices of `slice` keys; a slice whose slot
    // overflowed (or every slice, when there are no slots) is re-read from the
    // keys.
    const void *keys_in;
    int64_t begin;
    uint32_t n, nslots, slice, slot_cap;
    const uint32_t *slot_info;  // nullptr: no slots, stream the keys
    const uint2 *slot_data;

    template <class F> __device__ __forceinline__ void visit(F &&f) const {
        const uint32_t t = threadIdx.x;
        if (lds) {
            for (uint32_t base = 0; base < count; base += kThreads) {
                const uint32_t i = base + t;
                const bool act = i < count;
                const uint2 e = act ? stash[i] : make_uint2(0u, 0u);
                f(e.x, e.y, act);
            }
            return;
        }
        for (uint32_t q = 0; q < nslots; ++q) {
            const uint32_t lo = q * slice;
            const uint32_t hi = (n - lo) > slice ? lo + slice : n;
            const bool stream = slot_info == nullptr || slot_info[2 * q + 1] != 0;
            if (stream) {
                Range<KT> L;
                L.init(keys_in, begin, lo, hi);
                L.for_each(t, f);
            } else {
                uint32_t cnt = slot_info[2 * q];
                cnt = cnt < slot_cap ? cnt : slot_cap;
                const uint2 *d = slot_data + (size_t)q * slot_cap;
                for (uint32_t base = 0; base < cnt; base += kThreads) {
                    const uint32_t i = base + t;
                    const bool act = i < cnt;
                    const uint2 e = act ? d[i] : make_uint2(0u, 0u);
                    f(e.x, e.y, act);
                }
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Output.
// ---------------------------------------------------------------------------
template <int KT>
__device__ __forceinline__ void write_out(const Params &p, const Seg &sg, uint32_t pos,
                                          uint32_t raw, uint32_t idx) {
    // Both indices are in range by construction; the checks keep any slip
    // inside the segment's own row and input.
    if (pos >= sg.k_i) return;
    const size_t o = (size_t)sg.row * p.k + pos;
    if (Key<KT>::kBytes == 4)
        static_cast<uint32_t *>(p.keys_out)[o] = raw;
    else
        static_cast<uint16_t *>(p.keys_out)[o] = (uint16_t)raw;
    if (p.vals_in) p.vals_out[o] = idx < sg.n ? p.vals_in[sg.begin + idx] : kNone;
}

// a before b in the output: better key first, then smaller index; entries
// with idx == kNone are padding and go last.
template <int KT, bool LARGEST>
__device__ __forceinline__ bool out_before(uint2 a, uint2 b) {
    if (a.y == kNone) return false;
    if (b.y == kNone) return true;
    const uint32_t oa = Key<KT>::ord(a.x), ob = Key<KT>::ord(b.x);
    if (oa != ob) return LARGEST ? oa > ob : oa < ob;
    return a.y < b.y;
}

// Bitonic sort of buf[0, cnt) in LDS.  All threads call it.
template <int KT, bool LARGEST>
__device__ __forceinline__ void bitonic_sort(uint2 *buf, uint32_t cnt) {
    const uint32_t t = threadIdx.x;
    uint32_t P = 1;
    while (P < cnt) P <<= 1;
    for (uint32_t i = cnt + t; i < P; i += kThreads) buf[i] = make_uint2(0u, kNone);
    __syncthreads();
    for (uint32_t size = 2; size <= P; size <<= 1) {
        for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
            for (uint32_t i = t; i < (P >> 1); i += kThreads) {
                const uint32_t lo = 2 * i - (i & (stride - 1));
                const uint32_t hi = lo + stride;
                const bool asc = (lo & size) == 0;
                const uint2 a = buf[lo], b = buf[hi];
                if (out_before<KT, LARGEST>(b, a) == asc) {
                    buf[lo] = b;
                    buf[hi] = a;
                }
            }
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------------------
// Passes 1.. over the candidates, the tie selection and the output, given the
// pass-0 result (bucket b0, keys before it E0, keys in it c0).
// ---------------------------------------------------------------------------
template <int KT, bool LARGEST>
__device__ __forceinline__ void finish(Smem &sm, uint2 *outbuf, const Params &p, const Seg &sg,
                       const Cands<KT> &cand, uint32_t b0, uint32_t E0, uint32_t c0) {
    constexpr int KB = Key<KT>::kBits;
    const uint32_t t = threadIdx.x;
    const uint32_t wave = t >> 6;
    const bool pl = p.prefer_larger != 0;

    int hi = KB - kDigit;
    uint32_t kmask = (uint32_t)(kBuckets - 1) << hi;
    uint32_t kpref = (LARGEST ? (uint32_t)(kBuckets - 1) - b0 : b0) << hi;
    uint32_t krem = sg.k_i - E0;
    uint32_t front = E0;
    bool done = (c0 == krem);

    // Key digits.
    while (!done && hi > 0) {
        const int w = hi < kDigit ? hi : kDigit;
        const int sh = hi - w;
        const uint32_t nb = 1u << w;
        for (uint32_t i = t; i < nb; i += kThreads) sm.hist[i] = 0;
        __syncthreads();
        cand.visit([&](uint32_t raw, uint32_t idx, bool act) {
            const uint32_t o = Key<KT>::ord(raw);
            if (act && (o & kmask) == kpref) {
                const uint32_t d = (o >> sh) & (nb - 1);
                atomicAdd(&sm.hist[LARGEST ? nb - 1 - d : d], 1u);
            }
        });
        __syncthreads();
        if (wave == 0) find_kth(sm.hist, nb, krem, sm.res);
        __syncthreads();
        const uint32_t b = sm.res[1], E = sm.res[2], cnt = sm.res[3];
        krem -= E;
        front += E;
        kpref |= (LARGEST ? nb - 1 - b : b) << sh;
        kmask |= (nb - 1) << sh;
        done = (cnt == krem);
        hi = sh;
    }

    // Index digits among the splitter-equal keys (deterministic modes).  The
    // tie winners are the `ties` best of them by index; `krem` now counts
    // within the narrowing index prefix and `front` is left alone.
    const uint32_t ties = krem;
    bool by_index = false;
    uint32_t imask = 0, ipref = 0;
    if (!done && p.det) {
        by_index = true;
        hi = 32 - __clz((int)(sg.n - 1u));
        while (!done && hi > 0) {
            const int w = hi < kDigit ? hi : kDigit;
            const int sh = hi - w;
            const uint32_t nb = 1u << w;
            for (uint32_t i = t; i < nb; i += kThreads) sm.hist[i] = 0;
            __syncthreads();
            cand.visit([&](uint32_t raw, uint32_t idx, bool act) {
                if (act && (Key<KT>::ord(raw) & kmask) == kpref && (idx & imask) == ipref) {
                    const uint32_t d = (idx >> sh) & (nb - 1);
                    atomicAdd(&sm.hist[pl ? nb - 1 - d : d], 1u);
                }
            });
            __syncthreads();
            if (wave == 0) find_kth(sm.hist, nb, krem, sm.res);
            __syncthreads();
            const uint32_t b = sm.res[1], E = sm.res[2], cnt = sm.res[3];
            krem -= E;
            ipref |= (pl ? nb - 1 - b : b) << sh;
            imask |= (nb - 1) << sh;
            done = (cnt == krem);
            hi = sh;
        }
    }

    // Final filter: everything better than the splitter, then the ties.
    if (t == 0) {
        sm.ctr[0] = 0;
        sm.ctr[1] = 0;
    }
    __syncthreads();
    cand.visit([&](uint32_t raw, uint32_t idx, bool act) {
        const uint32_t km = Key<KT>::ord(raw) & kmask;
        const bool better = act && (LARGEST ? km > kpref : km < kpref);
        bool tie = act && km == kpref;
        if (by_index) {
            const uint32_t im = idx & imask;
            tie = tie && (pl ? im >= ipref : im <= ipref);
        }
        const uint32_t pb = wave_reserve(&sm.ctr[0], better);
        const uint32_t pt = wave_reserve(&sm.ctr[1], tie);
        uint32_t pos = kNone;
        if (better && pb < front) pos = pb;
        if (tie && pt < ties) pos = front + pt;
        if (pos != kNone) {
            if (outbuf)
                outbuf[pos] = make_uint2(raw, idx);
            else
                write_out<KT>(p, sg, pos, raw, idx);
        }
    });
    __syncthreads();
    if (outbuf) {
        if (p.sorted) bitonic_sort<KT, LARGEST>(outbuf, sg.k_i);
        for (uint32_t j = t; j < sg.k_i; j += kThreads) write_out<KT>(p, sg, j, outbuf[j].x, outbuf[j].y);
    }
}

// k >= n: every key of the segment is selected.
template <int KT, bool LARGEST>
__device__ __forceinline__ void select_all(uint2 *outbuf, const Params &p, const Seg &sg) {
    Range<KT> L;
    L.init(p.keys_in, sg.begin, 0u, sg.n);
    if (p.sorted) {
        // n <= k <= out_cap: stage, sort, write.
        L.for_each(threadIdx.x, [&](uint32_t raw, uint32_t idx, bool act) {
            if (act) outbuf[idx] = make_uint2(raw, idx);
        });
        __syncthreads();
        bitonic_sort<KT, LARGEST>(outbuf, sg.n);
        for (uint32_t j = threadIdx.x; j < sg.n; j += kThreads)
            write_out<KT>(p, sg, j, outbuf[j].x, outbuf[j].y);
    } else {
        L.for_each(threadIdx.x, [&](uint32_t raw, uint32_t idx, bool act) {
            if (act) write_out<KT>(p, sg, idx, raw, idx);
        });
    }
}

// ---------------------------------------------------------------------------
// The kernel.  Grid: ceil(S / 8) * 8 * wg_per_seg workgroups.  Workgroup b
// serves segment (b / 8 / P) * 8 + b % 8, slice (b / 8) % P, so that all the
// workgroups of one segment share b % 8 (the XCD a workgroup is dispatched to)
// and their atomics and slots stay within one L2.
// ---------------------------------------------------------------------------
template <int KT, bool LARGEST>
__global__ __launch_bounds__(kThreads) void topk_kernel(Params p) {
    __shared__ Smem sm;
    extern __shared__ uint2 dyn[];
    uint2 *stash = dyn;
    uint2 *outbuf = p.out_cap ? dyn + p.stash_cap : nullptr;

    const uint32_t P = p.wg_per_seg;
    const uint32_t b = blockIdx.x;
    const uint32_t qq = b >> 3;
    const int64_t s = (int64_t)(qq / P) * 8 + (b & 7u);
    const uint32_t q = qq % P;
    if (s >= p.num_segments) return;

    Seg sg;
    sg.begin = p.offsets[s];
    const int64_t end = p.offsets[s + 1];
    sg.n = end > sg.begin ? (uint32_t)(end - sg.begin) : 0u;
    sg.k_i = sg.n < p.k ? sg.n : p.k;
    sg.row = s;
    if (sg.k_i == 0) return;

    // Workgroups that share this segment.
    uint32_t ps = 1, slice = sg.n;
    if (P > 1 && sg.n > p.k) {
        uint32_t sl = (uint32_t)(((uint64_t)sg.n + P - 1) / P);
        if (sl < p.min_slice) sl = p.min_slice;
        sl = (sl + 63u) & ~63u;
        ps = (uint32_t)(((uint64_t)sg.n + sl - 1) / sl);
        slice = sl;
    }
    if (q >= ps) return;

    if (sg.n <= p.k) {  // select-all
        if (q == 0) select_all<KT, LARGEST>(outbuf, p, sg);
        return;
    }

    const uint32_t lo = q * slice;
    const uint32_t hi = (sg.n - lo) > slice ? lo + slice : sg.n;
    const uint32_t R = pass0<KT, LARGEST>(sm, stash, p.stash_cap, p, sg, lo, hi, sg.k_i);

    Cands<KT> cand;
    cand.stash = stash;
    cand.keys_in = p.keys_in;
    cand.begin = sg.begin;
    cand.n = sg.n;
    cand.slot_cap = p.stash_cap;

    if (ps == 1) {
        cand.lds = sm.stash_bad == 0;
        cand.count = sm.stash_count;
        cand.nslots = 1;
        cand.slice = sg.n;
        cand.slot_info = nullptr;
        cand.slot_data = nullptr;
        finish<KT, LARGEST>(sm, outbuf, p, sg, cand, R, sm.res[2], sm.res[3]);
        return;
    }

    // ---- several workgroups per segment: publish this slice ----
    const uint32_t t = threadIdx.x;
    uint32_t *gh = p.ws_hist + (size_t)s * kBuckets;
    for (uint32_t r = t; r <= R; r += kThreads) {
        const uint32_t h = sm.hist[r];
        if (h) atomicAdd(&gh[r], h);
    }
    uint32_t *info = p.ws_slot_info + ((size_t)s * P) * 2;
    uint2 *slots = p.ws_slot_data + ((size_t)s * P) * p.stash_cap;
    const bool bad = sm.stash_bad != 0;
    if (t == 0) sm.ctr[0] = 0;
    __syncthreads();
    if (!bad) {
        const uint32_t thr = rank_thr<KT, LARGEST>(R);
        const uint32_t cnt = sm.stash_count;
        uint2 *mine = slots + (size_t)q * p.stash_cap;
        for (uint32_t base = 0; base < cnt; base += kThreads) {
            const uint32_t i = base + t;
            const bool act = i < cnt;
            const uint2 e = act ? stash[i] : make_uint2(0u, 0u);
            const bool keep = act && within<LARGEST>(Key<KT>::ord(e.x), thr);
            const uint32_t pos = wave_reserve(&sm.ctr[0], keep);
            if (keep) mine[pos] = e;
        }
    }
    __syncthreads();
    if (t == 0) {
        info[2 * q] = bad ? 0u : sm.ctr[0];
        info[2 * q + 1] = bad ? 1u : 0u;
    }
    __threadfence();
    __syncthreads();
    if (t == 0) sm.flag = (atomicAdd(&p.ws_ticket[s], 1u) == ps - 1) ? 1u : 0u;
    __syncthreads();
    if (!sm.flag) return;
    __threadfence();

    // ---- last arriver: merged histogram, then the segment's candidates ----
    for (uint32_t r = t; r < (uint32_t)kBuckets; r += kThreads)
        sm.hist[r] = __hip_atomic_load(&gh[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if ((t >> 6) == 0) find_kth(sm.hist, kBuckets, sg.k_i, sm.res);
    __syncthreads();
    const uint32_t bstar = sm.res[1], E0 = sm.res[2], c0 = sm.res[3];

    cand.lds = false;
    cand.nslots = ps;
    cand.slice = slice;
    cand.slot_info = info;
    cand.slot_data = slots;
    // Gather the candidates into the LDS stash when they fit.
    if (t == 0) {
        sm.stash_count = 0;
        sm.stash_bad = 0;
    }
    __syncthreads();
    {
        const uint32_t thr = rank_thr<KT, LARGEST>(bstar);
        const uint32_t cap = p.stash_cap;
        cand.visit([&](uint32_t raw, uint32_t idx, bool act) {
            const bool keep = act && within<LARGEST>(Key<KT>::ord(raw), thr);
            const uint32_t pos = wave_reserve(&sm.stash_count, keep);
            if (keep) {
                if (pos < cap)
                    stash[pos] = make_uint2(raw, idx);
                else
                    sm.stash_bad = 1;
            }
        });
    }
    __syncthreads();
    if (sm.stash_bad == 0) {
        cand.lds = true;
        cand.count = sm.stash_count;
    }
    __syncthreads();
    finish<KT, LARGEST>(sm, outbuf, p, sg, cand, bstar, E0, c0);
}

__global__ void zero_kernel(uint32_t *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
constexpr uint32_t kTargetWorkgroups = 2048;  // enough to fill 256 CUs several times
constexpr uint32_t kMaxWgPerSeg = 256;
constexpr uint32_t kMinSlice = 16384;
constexpr size_t kMaxLds = 64 * 1024;

int key_bytes(int type) {
    return (type == SEGTOPK_KEY_BF16 || type == SEGTOPK_KEY_F16) ? 2 : 4;
}

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

template <int KT>
hipError_t launch(const Params &p, bool largest, uint32_t grid, size_t lds, hipStream_t st) {
    if (largest)
        hipLaunchKernelGGL((topk_kernel<KT, true>), dim3(grid), dim3(kThreads), lds, st, p);
    else
        hipLaunchKernelGGL((topk_kernel<KT, false>), dim3(grid), dim3(kThreads), lds, st, p);
    return hipGetLastError();
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
    const size_t fixed = sizeof(Smem);
    // Sorted output is staged and sorted in LDS; unsorted output is staged only
    // for small k (coalesced row writes) and otherwise written in place.
    uint32_t out_cap = next_pow2(k32 < 2 ? 2 : k32);
    if (!sorted && out_cap > 256) out_cap = 0;
    uint32_t stash_cap = next_pow2(4 * k32);
    if (stash_cap < 1024) stash_cap = 1024;
    if (stash_cap > 4096) stash_cap = 4096;
    while (stash_cap > 256 && fixed + 8 * (size_t)(stash_cap + out_cap) > kMaxLds) stash_cap >>= 1;
    if (fixed + 8 * (size_t)(stash_cap + out_cap) > kMaxLds) return SEGTOPK_NOT_SUPPORTED;
    p.stash_cap = stash_cap;
    p.out_cap = out_cap;
    const size_t lds = 8 * (size_t)(stash_cap + out_cap);

    uint32_t P = 1;
    if ((uint64_t)num_segments < kTargetWorkgroups) {
        P = (uint32_t)((kTargetWorkgroups + num_segments - 1) / num_segments);
        if (P > kMaxWgPerSeg) P = kMaxWgPerSeg;
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
    hipError_t err = hipSuccess;
    if (P > 1) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return SEGTOPK_HIP_ERROR;
        prepare_pool(dev);
        const size_t S = (size_t)num_segments;
        const size_t n_hist = S * kBuckets, n_ticket = S;
        const size_t zero_words = n_hist + n_ticket;
        const size_t info_words = S * P * 2;
        size_t bytes = (zero_words + info_words) * 4;
        bytes = (bytes + 255) & ~(size_t)255;
        const size_t data_off = bytes;
        bytes += S * P * (size_t)stash_cap * sizeof(uint2);
        if (hipMallocAsync(&ws, bytes, stream) != hipSuccess) return SEGTOPK_HIP_ERROR;
        uint32_t *w = static_cast<uint32_t *>(ws);
        p.ws_hist = w;
        p.ws_ticket = w + n_hist;
        p.ws_slot_info = w + zero_words;
        p.ws_slot_data = reinterpret_cast<uint2 *>(static_cast<char *>(ws) + data_off);
        size_t zb = (zero_words + 255) / 256;
        if (zb > 1024) zb = 1024;
        hipLaunchKernelGGL(zero_kernel, dim3((unsigned)zb), dim3(256), 0, stream, w, zero_words);
        err = hipGetLastError();
    }
    if (err == hipSuccess) {
        const bool largest = direction == SEGTOPK_MAX;
        switch (type) {
        case SEGTOPK_KEY_F32: err = launch<SEGTOPK_KEY_F32>(p, largest, (uint32_t)grid, lds, stream); break;
        case SEGTOPK_KEY_BF16: err = launch<SEGTOPK_KEY_BF16>(p, largest, (uint32_t)grid, lds, stream); break;
        case SEGTOPK_KEY_U32: err = launch<SEGTOPK_KEY_U32>(p, largest, (uint32_t)grid, lds, stream); break;
        case SEGTOPK_KEY_I32: err = launch<SEGTOPK_KEY_I32>(p, largest, (uint32_t)grid, lds, stream); break;
        default: err = launch<SEGTOPK_KEY_F16>(p, largest, (uint32_t)grid, lds, stream); break;
        }
    }
    if (ws) {
        if (hipFreeAsync(ws, stream) != hipSuccess && err == hipSuccess) err = hipErrorUnknown;
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

extern "C" int segtopk_version(void) { return 100; }
