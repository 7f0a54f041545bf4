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
// How it maps onto gfx950 (where it departs from the pages' cluster design):
//
//  * One workgroup of four wave64 serves a segment (or a slice of one).  The
//    four waves stream disjoint quarters of the keys from HBM once each, with
//    no workgroup barrier inside the streaming loop.
//  * Pass 0 counts a key in the workgroup's LDS histogram, and copies it with
//    its index into its wave's LDS stash, only if its bucket can still hold the
//    k-th key.  The bound each wave uses is the k-th best bucket of what the
//    shared histogram held when the wave last looked: counts only grow, so a
//    bound read from a histogram other waves are still filling is merely loose,
//    never wrong.  Hence every key the answer needs is counted and stashed, and
//    the counts of every bucket up to the final k-th bucket are exact.  Later
//    passes, the tie selection and the output read only the stashes; a wave
//    whose stash overflows (heavy ties, large k) has its quarter re-read.
//  * After one barrier, wave 0 finishes the segment alone, synchronising its
//    lanes with wave fences only.
//  * Buckets are reversed for MAX (bucket = B-1-digit) instead of inverting the
//    key bits, after -0.0 has been folded onto +0.0 in the order-preserving bit
//    transform.   [PR "Fix BlockTopK +/-0.0 handling", Fix]
//  * Deterministic tie-break: the splitter-equal keys are narrowed by further
//    radix passes over their source index (digits ascending for
//    prefer_smaller_index, reversed for prefer_larger_index), which picks
//    exactly the required ties without an index-ordered scan; not_guaranteed
//    takes ties in arrival order behind an `out < k` guard.
//    [PR "Implement Segmented TopK ...", §1.6 Determinism / tie-breaking]
//  * A batch of few, long segments spreads each segment over several
//    workgroups (CDNA4 has no thread-block clusters).  Each finishes pass 0 on
//    its slice, adds its histogram to a per-segment global histogram with
//    atomics, and writes its candidates to a global slot sorted by bucket
//    together with their cumulative bucket counts; the last workgroup to take
//    the segment's ticket scans the merged histogram and reads from every slot
//    only the prefix that can still win.
//  * sorted / stable_sorted output is a bitonic sort in LDS of the k results on
//    (ordered key best-first, source index ascending).
//    [docs "Top-K: Determinism, Tie-Breaking, and Output Ordering", Output
//     ordering]
#pragma once

#include <atomic>

#include "topk_common.h"

namespace segtopk_impl {
namespace {

// ---------------------------------------------------------------------------
// Order-preserving bit transform: ord(a) < ord(b) exactly when a < b, and
// ord(-0.0) == ord(+0.0).  The original bits are kept for output.  Keys are
// held as their raw bits, zero-extended to 32 bits.
// ---------------------------------------------------------------------------
template <int KT> struct Key;

// kSignMag: the raw bits are sign and magnitude (IEEE floats), so the raw
// bits read as signed integers order the non-negative keys and read as
// unsigned integers order the non-positive keys in reverse.
template <> struct Key<SEGTOPK_KEY_F32> {
    static constexpr int kBits = 32, kBytes = 4;
    static constexpr bool kSignMag = true;
    __host__ __device__ __forceinline__ static uint32_t ord(uint32_t r) {
        r = (r == 0x80000000u) ? 0u : r;  // -0.0 joins +0.0
        return r ^ ((uint32_t)((int32_t)r >> 31) | 0x80000000u);
    }
    // The raw bits of an ordered key (+0.0 for the ordered bits of zero).
    __host__ __device__ __forceinline__ static uint32_t inv_ord(uint32_t o) {
        return (o & 0x80000000u) ? (o ^ 0x80000000u) : ~o;
    }
};
template <> struct Key<SEGTOPK_KEY_BF16> {
    static constexpr int kBits = 16, kBytes = 2;
    static constexpr bool kSignMag = true;
    __host__ __device__ __forceinline__ static uint32_t ord(uint32_t r) {
        r = (r == 0x8000u) ? 0u : r;
        return r ^ ((r & 0x8000u) ? 0xFFFFu : 0x8000u);
    }
    __host__ __device__ __forceinline__ static uint32_t inv_ord(uint32_t o) {
        o &= 0xFFFFu;
        return (o & 0x8000u) ? (o ^ 0x8000u) : (~o & 0xFFFFu);
    }
};
template <> struct Key<SEGTOPK_KEY_F16> {
    static constexpr int kBits = 16, kBytes = 2;
    static constexpr bool kSignMag = true;
    __host__ __device__ __forceinline__ static uint32_t ord(uint32_t r) {
        r = (r == 0x8000u) ? 0u : r;
        return r ^ ((r & 0x8000u) ? 0xFFFFu : 0x8000u);
    }
    __host__ __device__ __forceinline__ static uint32_t inv_ord(uint32_t o) {
        o &= 0xFFFFu;
        return (o & 0x8000u) ? (o ^ 0x8000u) : (~o & 0xFFFFu);
    }
};
template <> struct Key<SEGTOPK_KEY_U32> {
    static constexpr int kBits = 32, kBytes = 4;
    static constexpr bool kSignMag = false;
    __host__ __device__ __forceinline__ static uint32_t ord(uint32_t r) { return r; }
    __host__ __device__ __forceinline__ static uint32_t inv_ord(uint32_t o) { return o; }
};
template <> struct Key<SEGTOPK_KEY_U16> {
    static constexpr int kBits = 16, kBytes = 2;
    static constexpr bool kSignMag = false;
    __host__ __device__ __forceinline__ static uint32_t ord(uint32_t r) { return r & 0xFFFFu; }
    __host__ __device__ __forceinline__ static uint32_t inv_ord(uint32_t o) { return o & 0xFFFFu; }
};
template <> struct Key<SEGTOPK_KEY_I16> {
    static constexpr int kBits = 16, kBytes = 2;
    static constexpr bool kSignMag = false;
    __host__ __device__ __forceinline__ static uint32_t ord(uint32_t r) { return (r ^ 0x8000u) & 0xFFFFu; }
    __host__ __device__ __forceinline__ static uint32_t inv_ord(uint32_t o) { return (o ^ 0x8000u) & 0xFFFFu; }
};
template <> struct Key<SEGTOPK_KEY_I32> {
    static constexpr int kBits = 32, kBytes = 4;
    static constexpr bool kSignMag = false;
    __host__ __device__ __forceinline__ static uint32_t ord(uint32_t r) { return r ^ 0x80000000u; }
    __host__ __device__ __forceinline__ static uint32_t inv_ord(uint32_t o) { return o ^ 0x80000000u; }
};

// Pass-0 bucket rank of an ordered key: 0 is the best bucket.
template <int KT, bool LARGEST> __host__ __device__ __forceinline__ uint32_t rank0(uint32_t o) {
    constexpr int sh = Key<KT>::kBits - kDigit;
    const uint32_t d = o >> sh;
    return LARGEST ? (uint32_t)(kBuckets - 1) - d : d;
}
// Ordered-key threshold of "rank0 <= R": for MAX o >= thr, for MIN o <= thr.
template <int KT, bool LARGEST> __host__ __device__ __forceinline__ uint32_t rank_thr(uint32_t R) {
    constexpr int sh = Key<KT>::kBits - kDigit;
    return LARGEST ? ((uint32_t)(kBuckets - 1) - R) << sh : (R << sh) | ((1u << sh) - 1u);
}

// ---------------------------------------------------------------------------
// Test of raw keys against a bucket bound "rank0 <= R", without the
// ordered-bits transform; it passes exactly the keys that pass the test on
// the ordered bits (-0.0 with +0.0).
//
//  * Per chunk, each lane reduces its keys with one min or max per key
//    (packed pairs of 16-bit keys count as one operation) in the domain in
//    which the bound is a plain threshold, and compares the result once:
//      kPfMaxS  signed max   >= T      kPfMinU  unsigned min <= T
//      kPfMinS  signed min   <= T      kPfMaxU  unsigned max >= T
//    (for sign-magnitude keys a bound above zero is a signed threshold on the
//    non-negative keys, a bound below zero an unsigned one on the negative
//    keys, which every non-negative key passes for MAX or fails for MIN).
//  * A single key passes when (x ^ X) >= T2, the same test folded into one
//    unsigned comparison.
// All fields are wave-uniform (scalar registers).
// ---------------------------------------------------------------------------
enum : uint32_t { kPfMaxS = 0, kPfMinU = 1, kPfMinS = 2, kPfMaxU = 3 };

struct Prefilter {
    uint32_t mode, T;  // chunk reduction and its threshold
    uint32_t X, T2;    // single key: (x ^ X) >= T2
};

// The test for the ordered-key threshold thr (for MAX ord >= thr passes, for
// MIN ord <= thr).
template <int KT, bool LARGEST>
__host__ __device__ __forceinline__ Prefilter prefilter_thr(uint32_t thr) {
    constexpr int B = Key<KT>::kBits;
    constexpr uint32_t H = 1u << (B - 1);
    constexpr uint32_t M = B == 32 ? 0xFFFFFFFFu : 0xFFFFu;
    uint32_t mode, T;
    if constexpr (KT == SEGTOPK_KEY_U32 || KT == SEGTOPK_KEY_U16) {
        mode = LARGEST ? kPfMaxU : kPfMinU;
        T = thr;
    } else if constexpr (KT == SEGTOPK_KEY_I32 || KT == SEGTOPK_KEY_I16) {
        mode = LARGEST ? kPfMaxS : kPfMinS;
        T = thr ^ H;
    } else if (LARGEST) {
        // ord >= thr.  thr > H: positive keys with bits >= thr - H.  Else
        // every positive key and the negative keys with bits <= ~thr; a
        // bound of exactly +0.0 is widened by one step so that -0.0 (which
        // ord puts at H) passes with it, and nothing else.
        if (thr > H) {
            mode = kPfMaxS;
            T = thr - H;
        } else {
            mode = kPfMinU;
            T = ~(thr < H ? thr : H - 1u) & M;
        }
    } else {
        // ord <= thr.  thr >= H: every negative key (and -0.0) and the
        // positive keys with bits <= thr - H.  Else the negative keys with
        // bits >= ~thr, except -0.0 (bits H), which ord puts at H: no key has
        // ord H - 1, so a bound there is taken as "bits >= H + 1".
        if (thr >= H) {
            mode = kPfMinS;
            T = thr - H;
        } else {
            mode = kPfMaxU;
            T = thr == H - 1u ? H + 1u : ~thr & M;
        }
    }
    Prefilter f;
    f.mode = mode;
    f.T = T & M;
    // Signed tests become unsigned ones by flipping the sign bit; "<=" tests
    // become ">=" ones by complementing both sides.
    const uint32_t flip = (mode == kPfMaxS || mode == kPfMinS) ? H : 0u;
    const uint32_t neg = (mode == kPfMinU || mode == kPfMinS) ? M : 0u;
    f.X = flip ^ neg;
    f.T2 = (f.T ^ flip) ^ neg;
    return f;
}

// The test for "rank0 <= R", its fields in scalar registers.
template <int KT, bool LARGEST> __device__ __forceinline__ Prefilter prefilter(uint32_t R) {
    Prefilter f = prefilter_thr<KT, LARGEST>(rank_thr<KT, LARGEST>(R));
    f.mode = __builtin_amdgcn_readfirstlane(f.mode);
    f.T = __builtin_amdgcn_readfirstlane(f.T);
    f.X = __builtin_amdgcn_readfirstlane(f.X);
    f.T2 = __builtin_amdgcn_readfirstlane(f.T2);
    return f;
}

__host__ __device__ __forceinline__ bool pf_key(const Prefilter &f, uint32_t x) { return (x ^ f.X) >= f.T2; }

typedef short pf_s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short pf_u16x2 __attribute__((ext_vector_type(2)));

// Reduction of N dwords by op with four interleaved accumulators (enough
// independent operations in flight, few extra registers).
template <class T, int N, class Op>
__host__ __device__ __forceinline__ T pf_tree(const uint32_t (&d)[N], Op op) {
    constexpr int A = N < 4 ? N : 4;
    T acc[A];
#pragma unroll
    for (int j = 0; j < A; ++j) acc[j] = __builtin_bit_cast(T, d[j]);
#pragma unroll
    for (int j = A; j < N; ++j) acc[j % A] = op(acc[j % A], __builtin_bit_cast(T, d[j]));
#pragma unroll
    for (int w = 1; w < A; w *= 2)
#pragma unroll
        for (int j = 0; j + w < A; j += 2 * w) acc[j] = op(acc[j], acc[j + w]);
    return acc[0];
}

// Whether any of a lane's keys (N dwords, every key slot valid or zero) can
// be within the bound.  Zero slots past the end of a range may pass.
template <int KT, int N>
__host__ __device__ __forceinline__ bool pf_chunk(const Prefilter &f, const uint32_t (&d)[N]) {
    if constexpr (Key<KT>::kBytes == 4) {
        switch (f.mode) {
        case kPfMaxS:
            return pf_tree<int32_t>(d, [](int32_t a, int32_t b) { return a > b ? a : b; }) >=
                   (int32_t)f.T;
        case kPfMinS:
            return pf_tree<int32_t>(d, [](int32_t a, int32_t b) { return a < b ? a : b; }) <=
                   (int32_t)f.T;
        case kPfMinU:
            return pf_tree<uint32_t>(d, [](uint32_t a, uint32_t b) { return a < b ? a : b; }) <= f.T;
        default:
            return pf_tree<uint32_t>(d, [](uint32_t a, uint32_t b) { return a > b ? a : b; }) >= f.T;
        }
    } else {
        switch (f.mode) {
        case kPfMaxS: {
            const pf_s16x2 m = pf_tree<pf_s16x2>(
                d, [](pf_s16x2 a, pf_s16x2 b) { return __builtin_elementwise_max(a, b); });
            return (int32_t)(m.x > m.y ? m.x : m.y) >= (int32_t)(int16_t)f.T;
        }
        case kPfMinS: {
            const pf_s16x2 m = pf_tree<pf_s16x2>(
                d, [](pf_s16x2 a, pf_s16x2 b) { return __builtin_elementwise_min(a, b); });
            return (int32_t)(m.x < m.y ? m.x : m.y) <= (int32_t)(int16_t)f.T;
        }
        case kPfMinU: {
            const pf_u16x2 m = pf_tree<pf_u16x2>(
                d, [](pf_u16x2 a, pf_u16x2 b) { return __builtin_elementwise_min(a, b); });
            return (uint32_t)(m.x < m.y ? m.x : m.y) <= f.T;
        }
        default: {
            const pf_u16x2 m = pf_tree<pf_u16x2>(
                d, [](pf_u16x2 a, pf_u16x2 b) { return __builtin_elementwise_max(a, b); });
            return (uint32_t)(m.x > m.y ? m.x : m.y) >= f.T;
        }
        }
    }
}

// ---------------------------------------------------------------------------
// Wave helpers (wave64).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Inclusive prefix sum over the wave with DPP row shifts (within each row of
// 16 lanes), then row broadcasts of lane 15 and lane 31 across rows.  Lanes
// with no source lane add 0.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// Value of x in lane `src` (a wave-uniform lane index), in a scalar register.
__device__ __forceinline__ uint32_t wave_bcast(uint32_t x, uint32_t src) {
    return (uint32_t)__builtin_amdgcn_readlane((int)x, (int)src);
}

// Wave-wide OR and AND (every lane of the wave active): row scans with DPP
// shifts, then the four rows' last lanes combined on the scalar unit.
__device__ __forceinline__ void wave_or_and(uint32_t &o, uint32_t &a) {
    o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0x111, 0xF, 0xF, false);   // row_shr:1
    a &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)a, 0x111, 0xF, 0xF, false);
    o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0x112, 0xF, 0xF, false);   // row_shr:2
    a &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)a, 0x112, 0xF, 0xF, false);
    o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0x114, 0xF, 0xF, false);   // row_shr:4
    a &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)a, 0x114, 0xF, 0xF, false);
    o |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)o, 0x118, 0xF, 0xF, false);   // row_shr:8
    a &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)a, 0x118, 0xF, 0xF, false);
    o = wave_bcast(o, 15) | wave_bcast(o, 31) | wave_bcast(o, 47) | wave_bcast(o, 63);
    a = wave_bcast(a, 15) & wave_bcast(a, 31) & wave_bcast(a, 47) & wave_bcast(a, 63);
}

// Key bits [lo, hi) on which every candidate at the prefix agrees (their OR
// and AND over those bits are equal) need no digit pass: they extend the
// prefix at once.  `o` and `a` are the OR and AND of those candidates' ordered
// keys; lowers hi to just above the highest bit on which they differ.
__device__ __forceinline__ void skip_common_bits(uint32_t o, uint32_t a, int &hi, uint32_t &kmask,
                                                 uint32_t &kpref) {
    if (hi <= 0) return;
    const uint32_t low = hi >= 32 ? ~0u : ((1u << hi) - 1u);
    const uint32_t diff = (o ^ a) & low;
    const int hb = diff ? 32 - __clz((int)diff) : 0;
    if (hb >= hi) return;
    const uint32_t keep = hb == 0 ? 0u : ((1u << hb) - 1u);
    const uint32_t m = low & ~keep;
    kpref |= a & m;
    kmask |= m;
    hi = hb;
}

// Orders this wave's LDS accesses across lanes (lanes run in lockstep; this
// keeps the compiler from moving LDS traffic across the point).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct Kth {
    uint32_t found;   // 0: the buckets hold fewer than `target` keys
    uint32_t b;       // the bucket holding the target-th key
    uint32_t before;  // keys in buckets before b
    uint32_t count;   // keys in bucket b
};

// Smallest bucket b < nb with hist[0] + ... + hist[b] >= target, by one wave:
// every lane sums a run of buckets, a wave scan finds the lane whose run
// crosses the target, then the lanes take one bucket each of that run.
// hist may be filled concurrently by other waves: every count read is at most
// the final count, so the bucket found is at or after the final one.
// The runs are 4..32 buckets (a power of two); lane l reads its 16-byte
// pieces starting at piece l mod (run / 4), so that each read instruction
// spreads the wave over all LDS banks (runs are a multiple of 128 bytes
// apart, which would put every lane on the same banks).
__device__ __forceinline__ Kth wave_find(const uint32_t *hist, uint32_t nb, uint32_t target) {
    const uint32_t ln = lane_id();
    uint32_t per = (nb + 63u) >> 6;
    per = per <= 4u ? 4u : (per <= 8u ? 8u : (per <= 16u ? 16u : 32u));
    const uint32_t b0 = ln * per;
    const uint32_t pieces = per >> 2;
    uint32_t s = 0;
#pragma unroll
    for (uint32_t q = 0; q < 8; ++q) {
        const uint32_t b = b0 + 4u * ((q + ln) & (pieces - 1u));
        if (q < pieces && b < nb) {
            const uint4 h = *reinterpret_cast<const uint4 *>(&hist[b]);
            s += h.x + (b + 1 < nb ? h.y : 0u) + (b + 2 < nb ? h.z : 0u) + (b + 3 < nb ? h.w : 0u);
        }
    }
    const uint32_t incl = wave_incl_sum(s);
    const uint32_t excl = incl - s;
    const uint64_t hit = __ballot(excl < target && incl >= target);
    Kth r;
    if (hit == 0) {
        r.found = 0;
        r.b = nb - 1;
        r.before = 0;
        r.count = 0;
        return r;
    }
    const uint32_t L = (uint32_t)__ffsll((unsigned long long)hit) - 1u;
    const uint32_t baseL = wave_bcast(excl, L);
    const uint32_t bl = L * per + ln;
    const uint32_t v = (ln < per && bl < nb) ? hist[bl] : 0u;
    const uint32_t vi = wave_incl_sum(v);
    const uint64_t hit2 = __ballot(ln < per && baseL + vi >= target);
    const uint32_t j = (uint32_t)__ffsll((unsigned long long)hit2) - 1u;
    r.found = 1;
    r.b = L * per + j;
    r.count = wave_bcast(v, j);
    r.before = baseL + wave_bcast(vi, j) - r.count;
    return r;
}

// wave_find over a histogram in global memory that other workgroups are still
// adding to (relaxed agent-scope loads; any count read is at most the final
// count, so the bucket found is at or after the final one).
__device__ __forceinline__ Kth wave_find_global(const uint32_t *g, uint32_t nb, uint32_t target) {
    const uint32_t ln = lane_id();
    const uint32_t per = (nb + 63u) >> 6;  // 1 .. 32 buckets per lane
    const uint32_t b0 = ln * per;
    uint32_t s = 0;
    for (uint32_t q = 0; q < per; ++q) {
        const uint32_t b = b0 + q;
        if (b < nb) s += __hip_atomic_load(&g[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const uint32_t incl = wave_incl_sum(s);
    const uint32_t excl = incl - s;
    const uint64_t hit = __ballot(excl < target && incl >= target);
    Kth r;
    r.found = 0;
    r.b = nb - 1;
    r.before = 0;
    r.count = 0;
    if (hit == 0) return r;
    const uint32_t L = (uint32_t)__ffsll((unsigned long long)hit) - 1u;
    const uint32_t baseL = wave_bcast(excl, L);
    const uint32_t bl = L * per + ln;
    const uint32_t v = (ln < per && bl < nb)
                           ? __hip_atomic_load(&g[bl], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                           : 0u;
    const uint32_t vi = wave_incl_sum(v);
    const uint64_t hit2 = __ballot(ln < per && baseL + vi >= target);
    if (hit2 == 0) return r;  // the counts grew between the two reads: no tighter bound now
    const uint32_t j = (uint32_t)__ffsll((unsigned long long)hit2) - 1u;
    r.found = 1;
    r.b = L * per + j;
    return r;
}

// wave_find over the first nb <= 512 buckets of a global histogram that other
// workgroups are still adding to, in two steps so that the loads can be in
// flight while the wave does other work: find_global_issue reads each lane's
// run of `per` = ceil(nb / 64) buckets into registers; find_global_scan finds
// the bucket from them (one round of loads, where wave_find_global needs two).
struct GlobalRun {
    uint32_t v[8];
    uint32_t nb, per;
};
__device__ __forceinline__ void find_global_issue(const uint32_t *g, uint32_t nb, GlobalRun &gr) {
    const uint32_t ln = lane_id();
    gr.nb = nb;
    gr.per = (nb + 63u) >> 6;
#pragma unroll
    for (uint32_t i = 0; i < 8; ++i) {
        const uint32_t b = ln * gr.per + i;
        gr.v[i] = 0u;
        if (i < gr.per && b < nb)
            gr.v[i] = __hip_atomic_load(&g[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}
__device__ __forceinline__ Kth find_global_scan(const GlobalRun &gr, uint32_t target) {
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += gr.v[i];
    const uint32_t incl = wave_incl_sum(s);
    const uint32_t excl = incl - s;
    const uint64_t hit = __ballot(excl < target && incl >= target);
    Kth r;
    r.found = 0;
    r.b = gr.nb - 1;
    r.before = 0;
    r.count = 0;
    if (hit == 0) return r;
    const uint32_t L = (uint32_t)__ffsll((unsigned long long)hit) - 1u;
    uint32_t run = wave_bcast(excl, L);
#pragma unroll
    for (uint32_t i = 0; i < 8; ++i) {
        const uint32_t c = wave_bcast(gr.v[i], L);
        if (!r.found && i < gr.per && run + c >= target) {
            r.found = 1;
            r.b = L * gr.per + i;
            r.before = run;
            r.count = c;
        }
        run += c;
    }
    return r;
}

__device__ __forceinline__ void wave_clear(uint32_t *hist, uint32_t nb) {
    const uint32_t ln = lane_id();
    if (nb >= 256) {
        for (uint32_t i = ln * 4; i < nb; i += 4 * kWave)
            *reinterpret_cast<uint4 *>(&hist[i]) = make_uint4(0u, 0u, 0u, 0u);
    } else {
        for (uint32_t i = ln; i < nb; i += kWave) hist[i] = 0u;
    }
}


struct Seg {
    int64_t begin;  // first element of the segment in keys_in / vals_in
    uint32_t n;     // segment size
    uint32_t k_i;   // min(k, n)
    int64_t row;    // output row
};

// ---------------------------------------------------------------------------
// Coalesced reader of the keys [lo, hi) of one segment by NT threads: an
// unaligned head and tail (under 16 bytes each) element by element, the
// aligned body with 16-byte loads, U loads per thread per chunk.
// ---------------------------------------------------------------------------
template <int KT, int NT, int U> struct Range {
    static constexpr int kBytes = Key<KT>::kBytes;
    static constexpr int kVec = 16 / kBytes;  // keys per 16-byte load
    static constexpr int kU = U;
    static constexpr int kKpt = kU * kVec;    // keys per thread per chunk
    static constexpr int kDw = kU * 4;        // dwords per thread per chunk
    static constexpr uint32_t kChunkVecs = NT * kU;
    static constexpr uint32_t kChunkKeys = kChunkVecs * kVec;  // keys per chunk (all threads)

    const unsigned char *ebase;  // element 0 of the segment
    const uint4 *vbase;          // first aligned vector of the range
    uint32_t lo, head, nvec, tail_lo, nscalar, nchunks;

    __device__ __forceinline__ void init(const void *keys, int64_t begin, uint32_t lo_, uint32_t hi_) {
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
    // Thread t's part of chunk c: the loaded dwords; key j = u * kVec + e is
    // element vidx[u] + e (key_at extracts it); vidx[u] == kNone marks a load
    // past the end, whose dwords are zero.  STREAM: non-temporal loads, for a
    // single pass over keys that are not read again soon.
    template <bool STREAM = false>
    __device__ __forceinline__ void load_chunk(uint32_t c, uint32_t t, uint32_t (&raw)[kDw],
                                               uint32_t (&vidx)[kU]) const {
        typedef unsigned int v4u __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const uint32_t vj = c * kChunkVecs + (uint32_t)u * NT + t;
            v4u v = {0u, 0u, 0u, 0u};
            vidx[u] = kNone;
            if (vj < nvec) {
                const v4u *src = reinterpret_cast<const v4u *>(vbase) + vj;
                v = STREAM ? __builtin_nontemporal_load(src) : *src;
                vidx[u] = lo + head + vj * kVec;
            }
            raw[u * 4 + 0] = v.x;
            raw[u * 4 + 1] = v.y;
            raw[u * 4 + 2] = v.z;
            raw[u * 4 + 3] = v.w;
        }
    }
    // Chunk c without the element indices: the loads of a chunk wholly
    // inside the aligned body (every chunk but the last) take no bounds
    // tests; slots past the end are zero.
    template <bool STREAM = false>
    __device__ __forceinline__ void load_body(uint32_t c, uint32_t t, uint32_t (&raw)[kDw]) const {
        typedef unsigned int v4u __attribute__((ext_vector_type(4)));
        const v4u *src = reinterpret_cast<const v4u *>(vbase) + c * kChunkVecs + t;
        if ((c + 1) * kChunkVecs <= nvec) {
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const v4u v = STREAM ? __builtin_nontemporal_load(src + u * NT) : src[u * NT];
                raw[u * 4 + 0] = v.x;
                raw[u * 4 + 1] = v.y;
                raw[u * 4 + 2] = v.z;
                raw[u * 4 + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                v4u v = {0u, 0u, 0u, 0u};
                if (c * kChunkVecs + (uint32_t)u * NT + t < nvec)
                    v = STREAM ? __builtin_nontemporal_load(src + u * NT) : src[u * NT];
                raw[u * 4 + 0] = v.x;
                raw[u * 4 + 1] = v.y;
                raw[u * 4 + 2] = v.z;
                raw[u * 4 + 3] = v.w;
            }
        }
    }
    // Element index of the first key of thread t's load u of chunk c, kNone
    // past the end.
    __device__ __forceinline__ uint32_t vec_idx(uint32_t c, uint32_t t, int u) const {
        const uint32_t vj = c * kChunkVecs + (uint32_t)u * NT + t;
        return vj < nvec ? lo + head + vj * kVec : kNone;
    }
    // Key j of a thread's chunk as raw bits, zero-extended.
    __device__ __forceinline__ static uint32_t key_at(const uint32_t (&raw)[kDw], int j) {
        if (kBytes == 4) return raw[j];
        const uint32_t d = raw[j >> 1];
        return (j & 1) ? (d >> 16) : (d & 0xFFFFu);
    }
    // Calls f(raw, idx, active) for every element, chunk by chunk; every lane
    // of the thread group makes the same sequence of calls.
    template <class F> __device__ __forceinline__ void for_each(uint32_t t, F &&f) const {
        {
            const bool act = t < nscalar;
            const uint32_t idx = act ? scalar_idx(t) : 0u;
            f(act ? load_scalar(idx) : 0u, idx, act);
        }
        for (uint32_t c = 0; c < nchunks; ++c) {
            uint32_t raw[kDw], vidx[kU];
            load_chunk(c, t, raw, vidx);
#pragma unroll
            for (int u = 0; u < kU; ++u)
#pragma unroll
                for (int e = 0; e < kVec; ++e)
                    f(key_at(raw, u * kVec + e), vidx[u] + (uint32_t)e, vidx[u] != kNone);
        }
    }
};

// U 16-byte loads per lane per chunk: 4 where many workgroups each stream a
// short range, 8 (more bytes in flight per wave) where a few long slices do.
template <int KT, int U = 4> using WaveRange = Range<KT, kWave, U>;

// ---------------------------------------------------------------------------
// Pass 0 of one wave over keys [lo, hi) of a segment into a histogram shared
// with the other waves of the workgroup and into the wave's own stash.
// ---------------------------------------------------------------------------
// Bound sharing between the workgroups of one segment (slice mode): the
// workgroup adds an early snapshot of its histogram to a per-segment global
// "early" histogram once, and its waves periodically turn that histogram
// into a bound, published to the other waves through an LDS word.
// Bound sharing between the workgroups of one segment (slice mode).  Wave 0
// of each workgroup adds, every few chunks, what its histogram gained since
// its last contribution (buckets within the bound only) to a per-segment
// global histogram; it keeps what it has added so far in `glast`.  Every
// count there is of a distinct key, so the histogram undercounts the
// segment's and any bucket it yields is a valid bound.  The waves read a
// bound from it in turn and publish it to the workgroup through an LDS word.
struct Share {
    uint32_t *rg;        // LDS: best bound known to the workgroup
    uint32_t *gearly;    // global: the segment's shared histogram, or nullptr
    uint32_t *glast;     // LDS: this workgroup's contributions so far
    uint32_t wave;       // this wave's index in the workgroup
    uint32_t spread;     // the segment's workgroups span every XCD
    uint4 *ring;         // LDS: this wave's ring of loads to test (16-bit keys)
    uint32_t *ring_idx;  // LDS: element index of each ring entry's first key
};

struct Pass0 {
    uint32_t R;      // the wave's final bound (rank)
    uint32_t count;  // stash entries
    uint32_t defer;  // chunks [0, defer) were counted but not stashed
    uint32_t nch;    // chunks of the wave's range
};

// Drops, in place, the stash entries whose pass-0 rank is beyond the bound.
template <int KT, bool LARGEST>
__device__ __forceinline__ uint32_t wave_compact(uint2 *stash, uint32_t cnt, const Prefilter &pf) {
    const uint32_t ln = lane_id();
    uint32_t out = 0;
    for (uint32_t base = 0; base < cnt; base += kWave) {
        const uint32_t i = base + ln;
        const bool act = i < cnt;
        const uint2 e = act ? stash[i] : make_uint2(0u, 0u);
        const bool keep = act && pf_key(pf, e.x);
        const uint64_t m = __ballot(keep);
        wave_sync();  // this round's reads come before its writes
        if (keep) stash[out + lanes_below(m)] = e;
        out += (uint32_t)__popcll(m);
        wave_sync();
    }
    return out;
}

// Appends the lanes' entries with `ex` set to the stash; false when they do
// not fit even after dropping the entries that fail pf (the test for the
// current bound, which the caller holds already).
template <int KT, bool LARGEST>
__device__ __forceinline__ bool wave_push(uint2 *stash, uint32_t cap, uint32_t &count,
                                          const Prefilter &pf, bool ex, uint32_t x, uint32_t idx) {
    const uint64_t m = __ballot(ex);
    const uint32_t n = (uint32_t)__popcll(m);
    if (n == 0) return true;
    if (count + n > cap) {
        wave_sync();
        count = wave_compact<KT, LARGEST>(stash, count, pf);
        if (count + n > cap) return false;
    }
    if (ex) stash[count + lanes_below(m)] = make_uint2(x, idx);
    count += n;
    return true;
}

// Pass 0 of one wave over keys [lo, hi) of a segment.  Until the histogram
// shared by the workgroup's waves yields a bound, every key is counted and
// none is stashed.  From then on a key is counted and stashed only if its
// bucket is within the running bound R, which only tightens.  Chunks that were
// counted but not stashed (before the bound, or dropped when the stash
// overflowed) are read again by wave_reread once the workgroup's bound is
// final.  SLICED: the variant for slices of a segment shared by several
// workgroups (see kLazy below).
template <int KT, bool LARGEST, int U, bool SLICED>
__device__ __forceinline__ Pass0 wave_pass0(uint32_t *hist, uint2 *stash, uint32_t cap,
                                            const void *keys, int64_t begin, uint32_t lo,
                                            uint32_t hi, uint32_t target, const Share &sh) {
    using Rg = WaveRange<KT, U>;
    constexpr int K = Rg::kDw;
    constexpr int V = Rg::kVec;
    const uint32_t ln = lane_id();
    Rg L;
    L.init(keys, begin, lo, hi);
    const uint32_t nch = L.nchunks > 0 ? L.nchunks : 1u;
    Pass0 r;
    r.R = kBuckets - 1;  // until `target` keys are counted any bucket may hold the k-th
    r.count = 0;
    r.defer = 0;
    bool bounded = false;
    bool contributed = false;
    Prefilter pf = prefilter<KT, LARGEST>(kBuckets - 1);
    // 16-bit keys: when the bound was last computed from the histogram,
    // `below` keys of the workgroup lay in buckets before it; this wave has
    // counted `nbelow` more there since.  The bound can only move once
    // `below` plus the new counts of all four waves reach the target, so the
    // scan waits for that (taking the other waves to count about as many as
    // this one).  The 2-mantissa-bit buckets of 16-bit floats keep the bound
    // in one bucket for most of a long stream, and this saves a scan per
    // chunk there; so do the long slices of slice mode (f32 keys have the
    // same 2 mantissa bits in the pass-0 digit).  Otherwise 32-bit keys
    // rescan after every chunk that counted anything: with one workgroup per
    // segment the deferred path measured slower for them (code generation of
    // the whole kernel, not the extra work).
    constexpr bool kLazy = Key<KT>::kBytes == 2 || SLICED;
    uint32_t below = 0, nbelow = 0;
    // 16-bit keys also defer the histogram counts of the keys they stash:
    // stash entries [flushed, count) are not counted yet, and flush() counts
    // them 64 at a time, with every lane busy, instead of one sparse atomic
    // per passing key position.  A key position only appends to the stash
    // while there is room; a key that finds none is counted at once and the
    // stash is dropped after the chunk.  Counts are flushed after a chunk
    // before a rescan of the bound, a compaction or a drop, and at the end of
    // the stream; until then the histogram only undercounts, and any bound
    // found from an undercount is still valid.
    uint32_t flushed = 0;
    uint32_t compR = kBuckets;  // the bound at the last compaction
    auto flush = [&]() {
        for (uint32_t base = flushed; base < r.count; base += kWave) {
            const uint32_t i = base + ln;
            uint32_t rk = kBuckets;
            if (i < r.count) {
                rk = rank0<KT, LARGEST>(Key<KT>::ord(stash[i].x));
                atomicAdd(&hist[rk], 1u);
            }
            nbelow += (uint32_t)__popcll(__ballot(rk < r.R));
        }
        flushed = r.count;
    };

    // 16-bit keys with one workgroup per segment: about 0.4% of the keys of
    // a long stream pass the running bound, so most 16-byte loads of a wave
    // hold a passing key in some lane, yet few lanes do.  Testing such a load
    // key position by key position costs the wave eight tests for one or two
    // keys.  Instead the lanes whose load may pass append it (16 bytes and
    // the element index of its first key) to the wave's ring in LDS, and
    // once a wave's worth of loads wait, every lane tests one of them key by
    // key.  A load waiting in the ring is tested later under a bound that can
    // only be tighter, and its keys are counted when they are stashed (or at
    // once if the stash is full), so the histogram still only undercounts.
    constexpr bool kRing = Key<KT>::kBytes == 2 && !SLICED;
    uint32_t rhead = 0, rtail = 0;  // ring entries [rhead, rtail) wait
    // The deferred-count form of a key's test and stash push (see flush()).
    auto lazy_take = [&](uint32_t x, uint32_t idx, bool valid, bool &okr) {
        const bool pv = valid && pf_key(pf, x);
        if (!__any(pv)) return;
        if (okr) {
            const uint64_t m = __ballot(pv);
            const uint32_t n = (uint32_t)__popcll(m);
            if (r.count + n <= cap) {
                if (pv) stash[r.count + lanes_below(m)] = make_uint2(x, idx);
                r.count += n;
                return;
            }
            okr = false;
        }
        // Not stashed (the stash is dropped after this chunk): count now.
        const uint32_t rk = rank0<KT, LARGEST>(Key<KT>::ord(x));
        if (pv) atomicAdd(&hist[rk], 1u);
        nbelow += (uint32_t)__popcll(__ballot(pv && rk < r.R));
    };
    // Tests the n (at most 64) oldest loads of the ring, one per lane.
    auto drain = [&](uint32_t n, bool &okr) {
        wave_sync();
        const bool act = ln < n;
        const uint32_t slot = (rhead + ln) & (kRingLoads - 1u);
        uint32_t d[4] = {0u, 0u, 0u, 0u};
        uint32_t vi = 0;
        if (act) {
            const uint4 v = sh.ring[slot];
            d[0] = v.x;
            d[1] = v.y;
            d[2] = v.z;
            d[3] = v.w;
            vi = sh.ring_idx[slot];
        }
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const uint32_t dw = d[(e * Key<KT>::kBytes) >> 2];
            const uint32_t x = Key<KT>::kBytes == 4 ? dw : ((e & 1) ? (dw >> 16) : (dw & 0xFFFFu));
            lazy_take(x, vi + (uint32_t)e, act, okr);
        }
        rhead += n;
    };

    // The unaligned head and tail ride along with chunk 0.
    const bool sv = ln < L.nscalar;
    const uint32_t si = sv ? L.scalar_idx(ln) : 0u;
    const uint32_t sx = sv ? L.load_scalar(si) : 0u;

    uint32_t raw[K], vidx[Rg::kU];
    if constexpr (kLazy)
        L.template load_body<true>(0, ln, raw);
    else
        L.template load_chunk<true>(0, ln, raw, vidx);
    // Slice mode: a read of the shared histogram issued in the previous
    // iteration (1: into registers, 2: to be read in two rounds now).
    GlobalRun gr;
    uint32_t pending = 0;
    for (uint32_t c = 0; c < nch; ++c) {
        if constexpr (SLICED) {
            if (pending) {
                const Kth g = pending == 1u ? find_global_scan(gr, target)
                                            : wave_find_global(sh.gearly, r.R + 1, target);
                pending = 0;
                if (g.found && g.b < r.R) {
                    r.R = g.b;
                    below = 0;
                    pf = prefilter<KT, LARGEST>(r.R);
                    if (ln == 0) atomicMin(sh.rg, g.b);
                }
            }
        }
        uint32_t cur[K], cv[Rg::kU];
#pragma unroll
        for (int j = 0; j < K; ++j) cur[j] = raw[j];
        const bool s0 = sv && c == 0;  // this lane carries a head/tail key now
        if constexpr (kLazy) {
            // 16-bit keys: unchecked loads for full chunks, the element
            // indices computed from c (they are needed only where keys pass).
            if (c + 1 < nch) L.template load_body<true>(c + 1, ln, raw);  // prefetch
#pragma unroll
            for (int u = 0; u < Rg::kU; ++u) cv[u] = L.vec_idx(c, ln, u);
        } else {
#pragma unroll
            for (int u = 0; u < Rg::kU; ++u) cv[u] = vidx[u];
            if (c + 1 < nch) L.template load_chunk<true>(c + 1, ln, raw, vidx);  // prefetch
        }

        // Shared bounds, two ways.  A segment spread over every XCD reads the
        // shared histogram through device-wide atomics that take long: each
        // wave's turn issues the reads now, behind the prefetch, and uses them
        // at the top of the next iteration, where the prefetch has to be
        // waited for anyway.  A segment on one XCD reads it in place (the
        // reads are short, and this form measured faster there).  Spread
        // segments also share half as often (every 16 chunks of a wave): 768
        // workgroups' device-wide reads and adds cost more stream time than
        // the tighter bound saves (one segment of 2^28 keys: 383 -> 346 us),
        // while a segment on one XCD needs the 8-chunk rhythm to keep its
        // slices' stashes from overflowing.
        if constexpr (SLICED) {
            if (sh.gearly && sh.spread && bounded && c >= 2u &&
                ((c - 2u - 2u * sh.wave) & 15u) == 0u) {
                pending = r.R < 512u ? 1u : 2u;
                if (pending == 1u) find_global_issue(sh.gearly, r.R + 1, gr);
            }
        }
        if (sh.gearly && !(SLICED && sh.spread)) {
            const uint32_t rg = __builtin_amdgcn_readfirstlane(
                __hip_atomic_load(sh.rg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
            if (rg < r.R) {
                r.R = rg;
                below = 0;  // not known for a bound found elsewhere
                bounded = true;
                pf = prefilter<KT, LARGEST>(r.R);
            }
            if (bounded && c >= 1) {
                if (sh.wave == 0 && ((c - 1) & 7u) == 0u) {
                    // Add what the workgroup's histogram gained since the last
                    // time.  Later bounds are never looser, so every bucket
                    // read back from glast was written the first time.
                    const bool first = !contributed;
                    contributed = true;
                    for (uint32_t b = ln; b <= r.R; b += kWave) {
                        const uint32_t v = hist[b];
                        const uint32_t l = first ? 0u : sh.glast[b];
                        if (v > l) atomicAdd(&sh.gearly[b], v - l);
                        if (first || v != l) sh.glast[b] = v;
                    }
                }
                if (((c - 2u - 2u * sh.wave) & 7u) == 0u && c >= 2u) {
                    const Kth g = wave_find_global(sh.gearly, r.R + 1, target);
                    if (g.found && g.b < r.R) {
                        r.R = g.b;
                        below = 0;
                        pf = prefilter<KT, LARGEST>(r.R);
                        if (ln == 0) atomicMin(sh.rg, g.b);
                    }
                }
            }
        }

        if (SLICED && sh.gearly && sh.spread) {
            // Adopt a tighter bound found by another wave of this workgroup
            // (one lane reads it, so that the wave agrees on it).
            const uint32_t rg = __builtin_amdgcn_readfirstlane(
                __hip_atomic_load(sh.rg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
            if (rg < r.R) {
                r.R = rg;
                below = 0;  // not known for a bound found elsewhere
                bounded = true;
                pf = prefilter<KT, LARGEST>(r.R);
            }
            if (bounded && c >= 1 && sh.wave == 0 && ((c - 1) & 15u) == 0u) {
                // Add what the workgroup's histogram gained since the last
                // time.  Later bounds are never looser, so every bucket read
                // back from glast was written the first time.
                const bool first = !contributed;
                contributed = true;
                for (uint32_t b = ln; b <= r.R; b += kWave) {
                    const uint32_t v = hist[b];
                    const uint32_t l = first ? 0u : sh.glast[b];
                    if (v > l) atomicAdd(&sh.gearly[b], v - l);
                    if (first || v != l) sh.glast[b] = v;
                }
            }
        }

        if (!bounded) {
            // No bound yet: count every key, then look for the bound.
            bool any = false;
#pragma unroll
            for (int u = 0; u < Rg::kU; ++u)
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    if (cv[u] != kNone) {
                        atomicAdd(&hist[rank0<KT, LARGEST>(Key<KT>::ord(Rg::key_at(cur, u * V + e)))], 1u);
                        any = true;
                    }
                }
            if (s0) {
                atomicAdd(&hist[rank0<KT, LARGEST>(Key<KT>::ord(sx))], 1u);
                any = true;
            }
            r.defer = c + 1;
            if (!__any(any)) continue;
            wave_sync();
            const Kth f = wave_find(hist, kBuckets, target);
            if (!f.found) continue;
            r.R = f.b;
            below = f.before;
            bounded = true;
            pf = prefilter<KT, LARGEST>(r.R);
            // Stash this chunk's keys within the bound from the registers,
            // if they fit; earlier chunks stay deferred.
            const bool sin = s0 && pf_key(pf, sx);
            uint32_t cnt = sin ? 1u : 0u;
#pragma unroll
            for (int u = 0; u < Rg::kU; ++u)
#pragma unroll
                for (int e = 0; e < V; ++e)
                    cnt += (cv[u] != kNone && pf_key(pf, Rg::key_at(cur, u * V + e))) ? 1u : 0u;
            const uint32_t incl = wave_incl_sum(cnt);
            const uint32_t total = wave_bcast(incl, kWave - 1);
            if (r.count + total > cap) continue;  // the stash is empty: defer the chunk
            uint32_t pos = r.count + incl - cnt;
            if (sin) stash[pos++] = make_uint2(sx, si);
#pragma unroll
            for (int u = 0; u < Rg::kU; ++u)
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const uint32_t x = Rg::key_at(cur, u * V + e);
                    if (cv[u] != kNone && pf_key(pf, x))
                        stash[pos++] = make_uint2(x, cv[u] + (uint32_t)e);
                }
            r.count += total;
            if constexpr (kLazy) flushed = r.count;  // counted above already
            r.defer = c;
            continue;
        }

        // Bounded: one min or max per key decides whether any key of the
        // chunk can be within the bound; only then are the keys tested one
        // by one, and only a key position in which some lane passes takes
        // the exact rank test, the count and the stash push.
        // 16-bit keys test load by load, so that only the loads in which
        // some lane passes have their key positions tested one by one.
        bool lp[Rg::kU];
        if constexpr (kLazy) {
            bool cp = s0 && pf_key(pf, sx);
#pragma unroll
            for (int u = 0; u < Rg::kU; ++u) {
                lp[u] = pf_chunk<KT>(pf, *reinterpret_cast<const uint32_t(*)[4]>(&cur[u * 4]));
                cp = cp | lp[u];
            }
            if (!__any(cp)) continue;
        } else {
            const bool cp = pf_chunk<KT>(pf, cur);
            const bool sp = s0 && pf_key(pf, sx);
            if (!__any(cp || sp)) continue;
        }
        bool ok = true;
        auto take = [&](uint32_t x, uint32_t idx, bool valid) {
            const bool pv = valid && pf_key(pf, x);
            if (!__any(pv)) return;
            if constexpr (kLazy) {
                // The bound test is exact, so pv already means rank <= R.
                if (ok) {
                    const uint64_t m = __ballot(pv);
                    const uint32_t n = (uint32_t)__popcll(m);
                    if (r.count + n <= cap) {
                        if (pv) stash[r.count + lanes_below(m)] = make_uint2(x, idx);
                        r.count += n;
                        return;
                    }
                    ok = false;
                }
                // Not stashed (the stash is dropped after this chunk): count now.
                const uint32_t rk = rank0<KT, LARGEST>(Key<KT>::ord(x));
                if (pv) atomicAdd(&hist[rk], 1u);
                nbelow += (uint32_t)__popcll(__ballot(pv && rk < r.R));
                return;
            }
            const uint32_t rk = rank0<KT, LARGEST>(Key<KT>::ord(x));
            const bool ex = pv && rk <= r.R;
            if (ex) atomicAdd(&hist[rk], 1u);
            nbelow += (uint32_t)__popcll(__ballot(ex && (!kLazy || rk < r.R)));
            if (ok) ok = wave_push<KT, LARGEST>(stash, cap, r.count, pf, ex, x, idx);
        };
        if constexpr (kRing) {
            lazy_take(sx, si, s0, ok);
#pragma unroll
            for (int u = 0; u < Rg::kU; ++u) {
                const bool f = lp[u] && cv[u] != kNone;
                const uint64_t m = __ballot(f);
                if (m == 0) continue;
                if (f) {
                    const uint32_t slot = (rtail + lanes_below(m)) & (kRingLoads - 1u);
                    sh.ring[slot] = make_uint4(cur[u * 4], cur[u * 4 + 1], cur[u * 4 + 2], cur[u * 4 + 3]);
                    sh.ring_idx[slot] = cv[u];
                }
                rtail += (uint32_t)__popcll(m);
                if (rtail - rhead >= (uint32_t)kWave) drain(kWave, ok);
            }
            // A drop of the stash follows: every waiting load is tested (and
            // its passing keys counted) first.
            if (!ok)
                while (rtail != rhead)
                    drain(rtail - rhead < (uint32_t)kWave ? rtail - rhead : (uint32_t)kWave, ok);
        } else {
            take(sx, si, s0);
#pragma unroll
            for (int u = 0; u < Rg::kU; ++u) {
                if constexpr (kLazy)
                    if (!__any(lp[u])) continue;
#pragma unroll
                for (int e = 0; e < V; ++e)
                    take(Rg::key_at(cur, u * V + e), cv[u] + (uint32_t)e, cv[u] != kNone);
            }
        }
        if constexpr (kLazy) {
            // One place for the deferred counts: before a drop, before a
            // compaction (the stash half full and the bound tighter than at
            // the last one), and when the bound may move (unflushed entries
            // bound the uncounted keys before its bucket).
            const bool half = r.count > cap / 2u && r.R < compR;
            if (!ok || half ||
                below + (uint32_t)kWaves * (nbelow + (r.count - flushed)) >= target) {
                flush();
                if (ok && half) {
                    wave_sync();
                    r.count = wave_compact<KT, LARGEST>(stash, r.count, pf);
                    flushed = r.count;
                    compR = r.R;
                }
            }
        }
        if (!ok) {
            // The stash is full even within the bound: drop it and read this
            // and every earlier chunk again later.
            r.count = 0;
            r.defer = c + 1;
            if constexpr (kLazy) flushed = 0;
        }
        if (nbelow != 0 && (!kLazy || below + (uint32_t)kWaves * nbelow >= target)) {
            // The bound may move: recompute it from everything counted.
            nbelow = 0;
            wave_sync();
            const Kth f = wave_find(hist, r.R + 1, target);
            if (f.found) {
                below = f.before;
                if (f.b < r.R) {
                    r.R = f.b;
                    pf = prefilter<KT, LARGEST>(r.R);
                }
            }
        }
    }
    if constexpr (kRing) {
        // The loads still waiting; if their keys do not fit, the stash is
        // dropped and every chunk is read again later.
        bool ok = true;
        while (rtail != rhead)
            drain(rtail - rhead < (uint32_t)kWave ? rtail - rhead : (uint32_t)kWave, ok);
        if (!ok) {
            flush();
            r.count = 0;
            r.defer = nch;
            flushed = 0;
        }
    }
    if constexpr (kLazy) flush();
    r.nch = nch;
    return r;
}

// Stashes, under the workgroup's final bound R, the keys of the chunks [0,
// defer) of [lo, hi) (and the unaligned head and tail).  They were counted in
// pass 0 already.  Returns false when they do not fit.
template <int KT, bool LARGEST, int U>
__device__ __forceinline__ bool wave_reread(uint2 *stash, uint32_t cap, uint32_t &count,
                                            const void *keys, int64_t begin, uint32_t lo,
                                            uint32_t hi, uint32_t defer, uint32_t R) {
    using Rg = WaveRange<KT, U>;
    constexpr int K = Rg::kDw;
    constexpr int V = Rg::kVec;
    const uint32_t ln = lane_id();
    Rg L;
    L.init(keys, begin, lo, hi);
    const Prefilter pf = prefilter<KT, LARGEST>(R);
    bool ok;
    {
        const bool sv = ln < L.nscalar;
        const uint32_t si = sv ? L.scalar_idx(ln) : 0u;
        const uint32_t x = sv ? L.load_scalar(si) : 0u;
        ok = wave_push<KT, LARGEST>(stash, cap, count, pf, sv && pf_key(pf, x), x, si);
    }
    const uint32_t nre = defer < L.nchunks ? defer : L.nchunks;
    uint32_t raw[K], vidx[Rg::kU];
    if (nre > 0) L.load_chunk(0, ln, raw, vidx);
    for (uint32_t c = 0; c < nre && ok; ++c) {
        uint32_t cur[K], cv[Rg::kU];
#pragma unroll
        for (int j = 0; j < K; ++j) cur[j] = raw[j];
#pragma unroll
        for (int u = 0; u < Rg::kU; ++u) cv[u] = vidx[u];
        if (c + 1 < nre) L.load_chunk(c + 1, ln, raw, vidx);
        // A chunk in which no lane can be within the bound costs one
        // reduction and one ballot.
        if (!__any(pf_chunk<KT>(pf, cur))) continue;
#pragma unroll
        for (int u = 0; u < Rg::kU; ++u)
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const uint32_t x = Rg::key_at(cur, u * V + e);
                if (ok)
                    ok = wave_push<KT, LARGEST>(stash, cap, count, pf, cv[u] != kNone && pf_key(pf, x),
                                                x, cv[u] + (uint32_t)e);
            }
    }
    return ok;
}

// Pass 0 of one wave, then its deferred chunks read again at once under the
// wave's own final bound (valid for the workgroup: bounds only tighten), so
// that the re-read overlaps the other waves' streaming instead of following
// the workgroup barrier.  If they do not fit, every chunk stays deferred and
// is read again after the barrier under the workgroup's bound.
template <int KT, bool LARGEST, int U, bool SLICED>
__device__ __forceinline__ Pass0 wave_pass0_stash(uint32_t *hist, uint2 *stash, uint32_t cap,
                                                  const void *keys, int64_t begin, uint32_t lo,
                                                  uint32_t hi, uint32_t target, const Share &sh) {
    Pass0 r = wave_pass0<KT, LARGEST, U, SLICED>(hist, stash, cap, keys, begin, lo, hi, target, sh);
    if (r.defer != 0) {
        uint32_t cnt = r.count;
        if (wave_reread<KT, LARGEST, U>(stash, cap, cnt, keys, begin, lo, hi, r.defer, r.R)) {
            r.count = cnt;
            r.defer = 0;
        } else {
            r.count = 0;
            r.defer = r.nch;
        }
    }
    return r;
}

// ---------------------------------------------------------------------------
// Candidates after pass 0, visited by wave 0: an LDS list, or (when a stash
// overflowed) global sources -- per slice either the first `cnt` entries of a
// global slot or, for an overflowed slot, the slice's keys again.
// ---------------------------------------------------------------------------
template <int KT> struct Cands {
    const uint2 *list;      // LDS list ...
    uint32_t count;
    bool lds;
    const void *keys_in;    // ... or global sources
    int64_t begin;
    uint32_t n, nslices, slice;
    const uint32_t *slot_info;  // nullptr: every slice is re-read from the keys
    const uint32_t *slot_cum;
    const uint2 *slot_data;
    uint32_t slot_cap, bstar;

    template <class F> __device__ __forceinline__ void visit(F &&f) const {
        const uint32_t ln = lane_id();
        if (lds) {
            for (uint32_t base = 0; base < count; base += kWave) {
                const uint32_t i = base + ln;
                const bool act = i < count;
                const uint2 e = act ? list[i] : make_uint2(0u, 0u);
                f(e.x, e.y, act);
            }
            return;
        }
        for (uint32_t q = 0; q < nslices; ++q) {
            const uint32_t lo = q * slice;
            const uint32_t hi = (n - lo) > slice ? lo + slice : n;
            if (slot_info == nullptr || slot_info[4 * q + 1] != 0) {
                WaveRange<KT> L;
                L.init(keys_in, begin, lo, hi);
                L.for_each(ln, f);
            } else {
                uint32_t cnt = slot_cum[(size_t)q * kBuckets + bstar];
                cnt = cnt < slot_cap ? cnt : slot_cap;
                const uint2 *d = slot_data + (size_t)q * slot_cap;
                for (uint32_t base = 0; base < cnt; base += kWave) {
                    const uint32_t i = base + ln;
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
// The value of the segment's element idx: the payload, or (index mode, used
// for 8-byte payloads that a later pass gathers) the index itself.
__device__ __forceinline__ uint32_t val_load(const Params &p, const Seg &sg, uint32_t idx) {
    return p.vindex ? idx : p.vals_in[sg.begin + idx];
}
__device__ __forceinline__ void val_store(const Params &p, size_t o, uint32_t v) {
    p.vals_out[o << p.vshift] = v;
}

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
    if (p.vals_in) val_store(p, o, idx < sg.n ? val_load(p, sg, idx) : kNone);
}

// write_out for B entries per lane: every value load is issued before the
// first store, so that the loads' latencies overlap.
template <int KT, int B>
__device__ __forceinline__ void write_batch(const Params &p, const Seg &sg, const uint32_t (&pos)[B],
                                            const uint2 (&e)[B]) {
    uint32_t v[B];
#pragma unroll
    for (int u = 0; u < B; ++u)
        v[u] = (p.vals_in && pos[u] < sg.k_i && e[u].y < sg.n) ? val_load(p, sg, e[u].y) : kNone;
#pragma unroll
    for (int u = 0; u < B; ++u) {
        if (pos[u] >= sg.k_i) continue;
        const size_t o = (size_t)sg.row * p.k + pos[u];
        if (Key<KT>::kBytes == 4)
            static_cast<uint32_t *>(p.keys_out)[o] = e[u].x;
        else
            static_cast<uint16_t *>(p.keys_out)[o] = (uint16_t)e[u].x;
        if (p.vals_in) val_store(p, o, v[u]);
    }
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

// Bitonic sort of buf[0, cnt) in LDS by one wave.
template <int KT, bool LARGEST>
__device__ __forceinline__ void wave_bitonic(uint2 *buf, uint32_t cnt) {
    const uint32_t ln = lane_id();
    uint32_t P = 1;
    while (P < cnt) P <<= 1;
    for (uint32_t i = cnt + ln; i < P; i += kWave) buf[i] = make_uint2(0u, kNone);
    wave_sync();
    for (uint32_t size = 2; size <= P; size <<= 1) {
        for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
            for (uint32_t i = ln; i < (P >> 1); i += kWave) {
                const uint32_t lo = 2 * i - (i & (stride - 1));
                const uint32_t hi = lo + stride;
                const bool asc = (lo & size) == 0;
                const uint2 a = buf[lo], b = buf[hi];
                if (out_before<KT, LARGEST>(b, a) == asc) {
                    buf[lo] = b;
                    buf[hi] = a;
                }
            }
            wave_sync();
        }
    }
}

// x of lane (l ^ M), for a constant M: DPP quad permutes for 1 and 2, DPP row
// shifts limited to the receiving banks for 4 and 8, and the permlane swaps
// of gfx950 for 16 and 32 -- no trip through the LDS crossbar.
template <int M> __device__ __forceinline__ uint32_t lane_xor(uint32_t x) {
    if constexpr (M == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    } else if constexpr (M == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    } else if constexpr (M == 4) {
        const int t = __builtin_amdgcn_update_dpp((int)x, (int)x, 0x104, 0xF, 0x5, false);  // row_shl:4
        return (uint32_t)__builtin_amdgcn_update_dpp(t, (int)x, 0x114, 0xF, 0xA, false);   // row_shr:4
    } else if constexpr (M == 8) {
        const int t = __builtin_amdgcn_update_dpp((int)x, (int)x, 0x108, 0xF, 0x3, false);  // row_shl:8
        return (uint32_t)__builtin_amdgcn_update_dpp(t, (int)x, 0x118, 0xF, 0xC, false);   // row_shr:8
    } else if constexpr (M == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return (lane_id() & 16u) ? r[0] : r[1];
    } else {
        static_assert(M == 32, "lane_xor: M must be a power of two below 64");
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (lane_id() & 32u) ? r[0] : r[1];
    }
}

// One compare-exchange step (block SIZE, distance STRIDE) of a bitonic sort
// of 64*E register entries, lane l holding entries l*E .. l*E+E-1, ascending
// by (sk, id); NP payload arrays ride along (none when NP is 0).
template <int E, int NP, int SIZE, int STRIDE>
__device__ __forceinline__ void bitonic_step(uint32_t (&sk)[E], uint32_t (&id)[E], uint32_t (&pl)[NP ? NP : 1][E]) {
    const uint32_t ln = lane_id();
    if constexpr (STRIDE >= E) {
        constexpr int LM = STRIDE / E;
        const bool lower = ((ln * E) & STRIDE) == 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint32_t j = ln * E + e;
            const uint32_t psk = lane_xor<LM>(sk[e]);
            const uint32_t pid = lane_xor<LM>(id[e]);
            uint32_t ppl[NP ? NP : 1];
#pragma unroll
            for (int q = 0; q < NP; ++q) ppl[q] = lane_xor<LM>(pl[q][e]);
            const bool asc = (j & SIZE) == 0;
            const bool pfirst = psk < sk[e] || (psk == sk[e] && pid < id[e]);
            if ((lower == asc) ? pfirst : !pfirst) {
                sk[e] = psk;
                id[e] = pid;
#pragma unroll
                for (int q = 0; q < NP; ++q) pl[q][e] = ppl[q];
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (e & STRIDE) continue;
            const int f = e | STRIDE;
            const uint32_t j = ln * E + e;
            const bool asc = (j & SIZE) == 0;
            const bool ffirst = sk[f] < sk[e] || (sk[f] == sk[e] && id[f] < id[e]);
            if (ffirst == asc) {
                uint32_t t0 = sk[e]; sk[e] = sk[f]; sk[f] = t0;
                t0 = id[e]; id[e] = id[f]; id[f] = t0;
#pragma unroll
                for (int q = 0; q < NP; ++q) {
                    t0 = pl[q][e]; pl[q][e] = pl[q][f]; pl[q][f] = t0;
                }
            }
        }
    }
}

template <int E, int NP, int SIZE, int STRIDE>
__device__ __forceinline__ void bitonic_merge(uint32_t (&sk)[E], uint32_t (&id)[E], uint32_t (&pl)[NP ? NP : 1][E]) {
    bitonic_step<E, NP, SIZE, STRIDE>(sk, id, pl);
    if constexpr (STRIDE > 1) bitonic_merge<E, NP, SIZE, STRIDE / 2>(sk, id, pl);
}

// Bitonic sort of all 64*E entries, blocks of SIZE and up (call with SIZE 2).
template <int E, int NP, int SIZE>
__device__ __forceinline__ void bitonic_regs(uint32_t (&sk)[E], uint32_t (&id)[E], uint32_t (&pl)[NP ? NP : 1][E]) {
    bitonic_merge<E, NP, SIZE, SIZE / 2>(sk, id, pl);
    if constexpr (SIZE < kWave * E) bitonic_regs<E, NP, SIZE * 2>(sk, id, pl);
}

// Sorts list[0, m) (m <= 64 * E, E entries per lane, lane l holding entries
// l*E .. l*E+E-1, in registers) best first, ties by ascending index, and
// writes the first k_i to the row: the sort is both the selection and the
// output order.  With prefer_larger_index the entries equal to the k_i-th key
// keep their largest-index members instead, still written in index order.
// The network carries the ordered key and the index only: the raw key is the
// inverse of the ordered bits, unless a -0.0 is among the entries (then the
// raw bits ride along), and the values are gathered after the sort.
template <int KT, bool LARGEST, int E>
__device__ __forceinline__ void sort_select(const uint2 *list, uint32_t m, const Params &p,
                                            const Seg &sg) {
    constexpr uint32_t kNegZero = Key<KT>::kBits == 32 ? 0x80000000u : 0x8000u;
    const uint32_t ln = lane_id();
    uint32_t sk[E], id[E], pl[1][E];
    bool negzero = false;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const uint32_t j = ln * E + e;
        sk[e] = kNone;
        id[e] = kNone;
        pl[0][e] = 0;
        if (j < m) {
            const uint2 x = list[j];
            const uint32_t o = Key<KT>::ord(x.x);
            sk[e] = LARGEST ? ~o : o;
            id[e] = x.y;
            pl[0][e] = x.x;
            negzero = negzero || (Key<KT>::kSignMag && x.x == kNegZero);
        }
    }
    const bool carry_raw = Key<KT>::kSignMag && __any(negzero);
    if (p.sorted || m > sg.k_i) {
        if (carry_raw)
            bitonic_regs<E, 1, 2>(sk, id, pl);
        else
            bitonic_regs<E, 0, 2>(sk, id, pl);
    }
    // Output position of sorted position j: j itself, except that with
    // prefer_larger_index the group [a, b) of entries equal to the k_i-th
    // keeps its last k_i - a members, moved down to [a, k_i).
    uint32_t shift = 0, a = sg.k_i;
    if (p.prefer_larger && m > sg.k_i) {
        const uint32_t kj = sg.k_i - 1;
        uint32_t mine = 0;
#pragma unroll
        for (int e = 0; e < E; ++e)
            if ((uint32_t)e == kj % E) mine = sk[e];
        const uint32_t ks = wave_bcast(mine, kj / E);
        uint32_t lt = 0, le = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const bool real = ln * E + (uint32_t)e < m;  // padding sorts last
            lt += (uint32_t)__popcll(__ballot(real && sk[e] < ks));
            le += (uint32_t)__popcll(__ballot(real && sk[e] <= ks));
        }
        a = lt;
        shift = le - sg.k_i;  // b - (k_i - a) - a
    }
    uint32_t pos[E], vv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const uint32_t j = ln * E + e;
        pos[e] = j;
        if (j >= a) pos[e] = (j >= a + shift) ? j - shift : kNone;
        if (j >= m) pos[e] = kNone;
        vv[e] = (p.vals_in && pos[e] < sg.k_i && id[e] < sg.n) ? val_load(p, sg, id[e]) : kNone;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (pos[e] < sg.k_i) {
            const size_t o = (size_t)sg.row * p.k + pos[e];
            const uint32_t rw = carry_raw ? pl[0][e] : Key<KT>::inv_ord(LARGEST ? ~sk[e] : sk[e]);
            if (Key<KT>::kBytes == 4)
                static_cast<uint32_t *>(p.keys_out)[o] = rw;
            else
                static_cast<uint16_t *>(p.keys_out)[o] = (uint16_t)rw;
            if (p.vals_in) val_store(p, o, vv[e]);
        }
    }
}

// The staged results outbuf[0, k_i): registers for small k, else an LDS sort.
template <int KT, bool LARGEST>
__device__ __forceinline__ void write_staged(uint2 *outbuf, const Params &p, const Seg &sg) {
    if (sg.k_i <= 64) {
        sort_select<KT, LARGEST, 1>(outbuf, sg.k_i, p, sg);
    } else if (sg.k_i <= 128) {
        sort_select<KT, LARGEST, 2>(outbuf, sg.k_i, p, sg);
    } else if (sg.k_i <= 256) {
        sort_select<KT, LARGEST, 4>(outbuf, sg.k_i, p, sg);
    } else {
        if (p.sorted) wave_bitonic<KT, LARGEST>(outbuf, sg.k_i);
        constexpr int kB = 8;
        for (uint32_t base = 0; base < sg.k_i; base += kB * kWave) {
            uint32_t pos[kB];
            uint2 e[kB];
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                pos[u] = base + (uint32_t)u * kWave + lane_id();
                e[u] = pos[u] < sg.k_i ? outbuf[pos[u]] : make_uint2(0u, kNone);
            }
            write_batch<KT, kB>(p, sg, pos, e);
        }
    }
}

// k >= n: every key of the segment is selected (one wave).
template <int KT, bool LARGEST>
__device__ __forceinline__ void wave_select_all(uint2 *outbuf, const Params &p, const Seg &sg) {
    const uint32_t ln = lane_id();
    WaveRange<KT> L;
    L.init(p.keys_in, sg.begin, 0u, sg.n);
    if (p.sorted) {  // n <= k <= out_cap
        L.for_each(ln, [&](uint32_t raw, uint32_t idx, bool act) {
            if (act) outbuf[idx] = make_uint2(raw, idx);
        });
        wave_sync();
        write_staged<KT, LARGEST>(outbuf, p, sg);
    } else {
        L.for_each(ln, [&](uint32_t raw, uint32_t idx, bool act) {
            if (act) write_out<KT>(p, sg, idx, raw, idx);
        });
    }
}

// ---------------------------------------------------------------------------
// Passes 1.., the tie selection and the output, by one wave, given the
// pass-0 result (bucket k0.b holds the k-th key, k0.before keys precede it,
// k0.count keys are in it).  hist is scratch.
// ---------------------------------------------------------------------------
template <int KT, bool LARGEST>
__device__ __forceinline__ void wave_finish(uint32_t *hist, uint2 *outbuf, const Params &p,
                                            const Seg &sg, const Cands<KT> &cand, Kth k0,
                                            uint32_t placed = 0) {
    constexpr int KB = Key<KT>::kBits;
    const uint32_t ln = lane_id();
    const bool pl = p.prefer_larger != 0;

    int hi = KB - kDigit;
    uint32_t kmask = (uint32_t)(kBuckets - 1) << hi;
    uint32_t kpref = (LARGEST ? (uint32_t)(kBuckets - 1) - k0.b : k0.b) << hi;
    uint32_t krem = sg.k_i - k0.before;
    uint32_t front = k0.before;
    bool done = (k0.count == krem);

    // Key digits.  The first pass also takes the OR and AND of the keys at
    // the prefix: digits on which they all agree (heavy ties) are then taken
    // without a pass.
    bool first = true;
    while (!done && hi > 0) {
        const int w = hi < kLaterDigit ? hi : kLaterDigit;
        const int sh = hi - w;
        const uint32_t nb = 1u << w;
        wave_clear(hist, nb);
        wave_sync();
        uint32_t co = 0, ca = ~0u;
        cand.visit([&](uint32_t r, uint32_t idx, bool act) {
            const uint32_t o = Key<KT>::ord(r);
            if (act && (o & kmask) == kpref) {
                const uint32_t d = (o >> sh) & (nb - 1);
                atomicAdd(&hist[LARGEST ? nb - 1 - d : d], 1u);
                co |= o;
                ca &= o;
            }
        });
        wave_sync();
        const Kth f = wave_find(hist, nb, krem);
        krem -= f.before;
        front += f.before;
        kpref |= (LARGEST ? nb - 1 - f.b : f.b) << sh;
        kmask |= (nb - 1) << sh;
        done = (f.count == krem);
        hi = sh;
        if (first && !done) {
            wave_or_and(co, ca);
            skip_common_bits(co, ca, hi, kmask, kpref);
        }
        first = false;
        wave_sync();
    }

    // Deterministic modes: narrow the splitter-equal keys by source index.
    // The `ties` winners are the best of them by index; `front` stays.
    const uint32_t ties = krem;
    bool by_index = false;
    uint32_t imask = 0, ipref = 0;
    if (!done && p.det) {
        by_index = true;
        hi = 32 - __clz((int)(sg.n - 1u));
        while (!done && hi > 0) {
            const int w = hi < kLaterDigit ? hi : kLaterDigit;
            const int sh = hi - w;
            const uint32_t nb = 1u << w;
            wave_clear(hist, nb);
            wave_sync();
            cand.visit([&](uint32_t r, uint32_t idx, bool act) {
                if (act && (Key<KT>::ord(r) & kmask) == kpref && (idx & imask) == ipref) {
                    const uint32_t d = (idx >> sh) & (nb - 1);
                    atomicAdd(&hist[pl ? nb - 1 - d : d], 1u);
                }
            });
            wave_sync();
            const Kth f = wave_find(hist, nb, krem);
            krem -= f.before;
            ipref |= (pl ? nb - 1 - f.b : f.b) << sh;
            imask |= (nb - 1) << sh;
            done = (f.count == krem);
            hi = sh;
            wave_sync();
        }
    }

    // Final filter: keys better than the splitter to [placed, front) (the
    // caller has written [0, placed) already), the chosen ties to
    // [front, k_i).
    uint32_t nf = placed, nt = 0;
    if (!outbuf && cand.lds) {
        // Written straight to the output: classify 8 entries per lane, then
        // write them with their value loads in flight together.
        constexpr int kB = 8;
        for (uint32_t base = 0; base < cand.count; base += kB * kWave) {
            uint32_t pos[kB];
            uint2 e[kB];
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                const uint32_t i = base + (uint32_t)u * kWave + ln;
                const bool act = i < cand.count;
                e[u] = act ? cand.list[i] : make_uint2(0u, kNone);
                const uint32_t km = Key<KT>::ord(e[u].x) & kmask;
                const bool better = act && (LARGEST ? km > kpref : km < kpref);
                bool tie = act && km == kpref;
                if (by_index) {
                    const uint32_t im = e[u].y & imask;
                    tie = tie && (pl ? im >= ipref : im <= ipref);
                }
                const uint64_t mb = __ballot(better);
                const uint64_t mt = __ballot(tie);
                const uint32_t pb = nf + lanes_below(mb);
                const uint32_t pt = nt + lanes_below(mt);
                nf += (uint32_t)__popcll(mb);
                nt += (uint32_t)__popcll(mt);
                pos[u] = kNone;
                if (better && pb < front) pos[u] = pb;
                if (tie && pt < ties) pos[u] = front + pt;
            }
            write_batch<KT, kB>(p, sg, pos, e);
        }
        return;
    }
    cand.visit([&](uint32_t r, uint32_t idx, bool act) {
        const uint32_t km = Key<KT>::ord(r) & kmask;
        const bool better = act && (LARGEST ? km > kpref : km < kpref);
        bool tie = act && km == kpref;
        if (by_index) {
            const uint32_t im = idx & imask;
            tie = tie && (pl ? im >= ipref : im <= ipref);
        }
        const uint64_t mb = __ballot(better);
        const uint64_t mt = __ballot(tie);
        const uint32_t pb = nf + lanes_below(mb);
        const uint32_t pt = nt + lanes_below(mt);
        nf += (uint32_t)__popcll(mb);
        nt += (uint32_t)__popcll(mt);
        uint32_t pos = kNone;
        if (better && pb < front) pos = pb;
        if (tie && pt < ties) pos = front + pt;
        if (pos != kNone) {
            if (outbuf)
                outbuf[pos] = make_uint2(r, idx);
            else
                write_out<KT>(p, sg, pos, r, idx);
        }
    });
    if (outbuf) {
        wave_sync();
        write_staged<KT, LARGEST>(outbuf, p, sg);
    }
}

// ---------------------------------------------------------------------------
// The kernel.  Grid: ceil(S / 8) * 8 * P workgroups of four waves.
// Workgroup b serves segment (b / 8 / P) * 8 + b % 8, slice (b / 8) % P, so all
// workgroups of one segment share b % 8 -- the XCD they are dispatched to --
// and their atomics and slots stay in one L2.
// ---------------------------------------------------------------------------
struct alignas(16) Shared {
    uint32_t hist[kBuckets];
    uint32_t wcount[kWaves];
    uint32_t wbad[kWaves];
    uint32_t wdefer[kWaves];
    uint32_t wkept[kWaves];  // entries of each wave's region within the workgroup's bound
    uint32_t rg;
    uint32_t last, total, any_bad, nfront, ntie, nstage;  // the last arriver's state
    uint32_t ncand;                               // candidates listed (one-chunk segments)
    uint32_t kb, kbefore, kcount, pad;            // the k-th bucket found by wave 0 (same)
};

// The splitter bits resolved before a finish starts: `hi` low bits are still
// open; the resolved high bits of the k-th key are kpref under kmask.
struct Prefix {
    int hi;
    uint32_t kmask, kpref;
};

// The prefix after pass 0 (the k-th key's pass-0 bucket b).
template <int KT, bool LARGEST> __device__ __forceinline__ Prefix pass0_prefix(uint32_t b) {
    constexpr int hi = Key<KT>::kBits - kDigit;
    Prefix f;
    f.hi = hi;
    f.kmask = (uint32_t)(kBuckets - 1) << hi;
    f.kpref = (LARGEST ? (uint32_t)(kBuckets - 1) - b : b) << hi;
    return f;
}

// Passes 1.., the tie selection and the output by the four waves of the
// workgroup together, over the LDS list list[0, count) of keys that match the
// resolved prefix pf0 (k0.before keys better than it come first in the
// output; `placed` of them are written already): in every visit each wave
// takes a quarter of the list; the histograms and the output positions are
// shared through LDS, with a workgroup barrier between the steps, and every
// wave finds the same bucket in the shared histogram.  The result is
// wave_finish's: in the deterministic modes exactly the required ties pass
// the final test, so arrival order decides only positions, which sorted
// output fixes afterwards.  Called by all four waves.
template <int KT, bool LARGEST>
__device__ __forceinline__ void block_finish(Shared &sh, uint2 *outbuf, const Params &p,
                                             const Seg &sg, const uint2 *list, uint32_t count,
                                             Kth k0, uint32_t placed, Prefix pf0) {
    const uint32_t t = threadIdx.x;
    const uint32_t w = t / kWave;
    const uint32_t ln = lane_id();
    const bool pl = p.prefer_larger != 0;
    uint32_t *hist = sh.hist;
    const uint32_t chunks = (count + kWave - 1) / kWave;
    const uint32_t c0 = chunks * w / kWaves, c1 = chunks * (w + 1) / kWaves;
    auto visit = [&](auto &&f) {
        for (uint32_t c = c0; c < c1; ++c) {
            const uint32_t i = c * kWave + ln;
            const bool act = i < count;
            const uint2 e = act ? list[i] : make_uint2(0u, 0u);
            f(e.x, e.y, act);
        }
    };

    int hi = pf0.hi;
    uint32_t kmask = pf0.kmask;
    uint32_t kpref = pf0.kpref;
    uint32_t krem = sg.k_i - k0.before;
    uint32_t front = k0.before;
    bool done = (k0.count == krem);

    // Key digits.  The first pass also takes the OR and AND of the keys at
    // the prefix (in the histogram's last two words): digits on which they
    // all agree (heavy ties) are then taken without a pass.
    bool first = true;
    while (!done && hi > 0) {
        const int wd = hi < kLaterDigit ? hi : kLaterDigit;
        const int sh_ = hi - wd;
        const uint32_t nb = 1u << wd;
        for (uint32_t i = t; i < nb; i += kThreads) hist[i] = 0u;
        if (t == 0) {
            hist[kBuckets - 2] = 0u;
            hist[kBuckets - 1] = ~0u;
        }
        __syncthreads();
        uint32_t co = 0, ca = ~0u;
        visit([&](uint32_t r, uint32_t idx, bool act) {
            const uint32_t o = Key<KT>::ord(r);
            if (act && (o & kmask) == kpref) {
                const uint32_t d = (o >> sh_) & (nb - 1);
                atomicAdd(&hist[LARGEST ? nb - 1 - d : d], 1u);
                co |= o;
                ca &= o;
            }
        });
        if (first) {
            wave_or_and(co, ca);
            if (ln == 0) {
                atomicOr(&hist[kBuckets - 2], co);
                atomicAnd(&hist[kBuckets - 1], ca);
            }
        }
        __syncthreads();
        const Kth f = wave_find(hist, nb, krem);
        krem -= f.before;
        front += f.before;
        kpref |= (LARGEST ? nb - 1 - f.b : f.b) << sh_;
        kmask |= (nb - 1) << sh_;
        done = (f.count == krem);
        hi = sh_;
        if (first && !done) skip_common_bits(hist[kBuckets - 2], hist[kBuckets - 1], hi, kmask, kpref);
        first = false;
        __syncthreads();
    }

    // Deterministic modes: narrow the splitter-equal keys by source index.
    const uint32_t ties = krem;
    bool by_index = false;
    uint32_t imask = 0, ipref = 0;
    if (!done && p.det) {
        by_index = true;
        hi = 32 - __clz((int)(sg.n - 1u));
        while (!done && hi > 0) {
            const int wd = hi < kLaterDigit ? hi : kLaterDigit;
            const int sh_ = hi - wd;
            const uint32_t nb = 1u << wd;
            for (uint32_t i = t; i < nb; i += kThreads) hist[i] = 0u;
            __syncthreads();
            visit([&](uint32_t r, uint32_t idx, bool act) {
                if (act && (Key<KT>::ord(r) & kmask) == kpref && (idx & imask) == ipref) {
                    const uint32_t d = (idx >> sh_) & (nb - 1);
                    atomicAdd(&hist[pl ? nb - 1 - d : d], 1u);
                }
            });
            __syncthreads();
            const Kth f = wave_find(hist, nb, krem);
            krem -= f.before;
            ipref |= (pl ? nb - 1 - f.b : f.b) << sh_;
            imask |= (nb - 1) << sh_;
            done = (f.count == krem);
            hi = sh_;
            __syncthreads();
        }
    }

    // Final filter: keys better than the splitter to [placed, front), the
    // chosen ties to [front, k_i); each wave reserves its positions per 64
    // entries with one LDS atomic per kind.
    if (t == 0) {
        sh.nfront = placed;
        sh.ntie = 0;
    }
    __syncthreads();
    visit([&](uint32_t r, uint32_t idx, bool act) {
        const uint32_t km = Key<KT>::ord(r) & kmask;
        const bool better = act && (LARGEST ? km > kpref : km < kpref);
        bool tie = act && km == kpref;
        if (by_index) {
            const uint32_t im = idx & imask;
            tie = tie && (pl ? im >= ipref : im <= ipref);
        }
        const uint64_t mb = __ballot(better);
        const uint64_t mt = __ballot(tie);
        uint32_t fb = 0, tb = 0;
        if (ln == 0) {
            fb = mb ? atomicAdd(&sh.nfront, (uint32_t)__popcll(mb)) : 0u;
            tb = mt ? atomicAdd(&sh.ntie, (uint32_t)__popcll(mt)) : 0u;
        }
        const uint32_t pb = wave_bcast(fb, 0) + lanes_below(mb);
        const uint32_t pt = wave_bcast(tb, 0) + lanes_below(mt);
        uint32_t pos = kNone;
        if (better && pb < front) pos = pb;
        if (tie && pt < ties) pos = front + pt;
        if (pos != kNone) {
            if (outbuf)
                outbuf[pos] = make_uint2(r, idx);
            else
                write_out<KT>(p, sg, pos, r, idx);
        }
    });
    if (outbuf) {
        __syncthreads();
        if (w == 0) write_staged<KT, LARGEST>(outbuf, p, sg);
    }
}

// block_finish right after pass 0.
template <int KT, bool LARGEST>
__device__ __forceinline__ void block_finish(Shared &sh, uint2 *outbuf, const Params &p,
                                             const Seg &sg, const uint2 *list, uint32_t count,
                                             Kth k0, uint32_t placed) {
    block_finish<KT, LARGEST>(sh, outbuf, p, sg, list, count, k0, placed,
                              pass0_prefix<KT, LARGEST>(k0.b));
}

// The last workgroup of a segment to finish pass 0, all four waves: the
// segment's exact k-th bucket b* from the merged histogram, then every slot's
// entries up to b* (a prefix, as the slots are sorted by bucket): those of
// better buckets are winners and are written at once, those of b* go to the
// LDS list for the remaining passes (wave 0).
// CLEAN: once the merged histogram is in LDS, the segment's scratch words
// that a call expects zero (merged and shared histograms, ticket) are cleared
// again, so that the next call on the same scratch needs no clearing pass.
template <int KT, bool LARGEST, bool CLEAN>
__device__ __forceinline__ void slice_last(Shared &sh, uint2 *stash, uint2 *outbuf,
                                           const Params &p, const Seg &sg, int64_t s, uint32_t P,
                                           uint32_t ps, uint32_t slice) {
    const uint32_t w = threadIdx.x / kWave;
    const uint32_t ln = lane_id();
    const uint32_t *gh = p.ws_hist + (size_t)s * kBuckets;
    const uint32_t *info = p.ws_slot_info + (size_t)s * P * 4;
    const uint32_t *slot_cum = p.ws_slot_cum + (size_t)s * P * kBuckets;
    const uint2 *slot_data = p.ws_slot_data + (size_t)s * P * p.stash_cap;

    // Merged histogram into LDS (plain loads: the ticket's acquire fence
    // made every slice's additions visible).
    {
        const uint4 *g4 = reinterpret_cast<const uint4 *>(gh);
        uint4 *h4 = reinterpret_cast<uint4 *>(sh.hist);
        for (uint32_t i = threadIdx.x; i < (uint32_t)kBuckets / 4; i += kThreads) h4[i] = g4[i];
    }
    __syncthreads();
    if constexpr (CLEAN) {
        // Every other slice has taken its ticket: none reads these any more.
        uint4 *m4 = reinterpret_cast<uint4 *>(p.ws_hist + (size_t)s * kBuckets);
        const uint32_t ne = p.spread ? 8u : 1u;  // shared histograms of the segment
        uint4 *e4 = reinterpret_cast<uint4 *>(p.ws_early + (size_t)s * ne * kBuckets);
        for (uint32_t i = threadIdx.x; i < (uint32_t)kBuckets / 4; i += kThreads)
            m4[i] = make_uint4(0u, 0u, 0u, 0u);
        for (uint32_t i = threadIdx.x; i < ne * (uint32_t)kBuckets / 4; i += kThreads)
            e4[i] = make_uint4(0u, 0u, 0u, 0u);
        if (threadIdx.x == 0) p.ws_ticket[s] = 0u;
    }
    const Kth ks = wave_find(sh.hist, kBuckets, sg.k_i);  // alike in every wave
    __syncthreads();

    // Per slot, the prefix up to b*, laid end to end (exclusive prefix).  The
    // slots' counts are read by every thread at once (one round of loads),
    // then scanned by wave 0.
    uint32_t *pre = sh.hist;
    for (uint32_t qi = threadIdx.x; qi < ps; qi += kThreads) {
        uint32_t c = kNone;  // a slice that lost candidates
        if (info[4 * qi + 1] == 0) {
            c = slot_cum[(size_t)qi * kBuckets + ks.b];
            c = c < p.stash_cap ? c : p.stash_cap;
        }
        pre[qi] = c;
    }
    __syncthreads();
    if (w == 0) {
        uint32_t total = 0;
        bool any_bad = false;
        for (uint32_t base = 0; base < ps; base += kWave) {
            const uint32_t qi = base + ln;
            uint32_t c = qi < ps ? pre[qi] : 0u;
            const bool bd = c == kNone;
            if (bd) c = 0;
            any_bad = any_bad || __any(bd);
            const uint32_t incl = wave_incl_sum(c);
            if (qi < ps) pre[qi] = total + incl - c;
            total += wave_bcast(incl, kWave - 1);
        }
        if (ln == 0) {
            pre[ps] = total;
            sh.total = total;
            sh.any_bad = any_bad ? 1u : 0u;
            sh.nfront = 0;
            sh.ntie = 0;
            sh.nstage = 0;
        }
    }
    __syncthreads();
    const uint32_t total = sh.total;
    bool fast = sh.any_bad == 0 && ks.count <= p.stash_cap;
    // Bucket b* too large for the LDS list, with room to stage it in a row.
    const bool stage = !fast && sh.any_bad == 0 && p.ws_stage != nullptr && ks.count <= kStageCap;

    // The slot of every prefix entry, when the table fits: in the words that
    // kept this workgroup's shared-histogram contributions (free after the
    // stream; 2 * kBuckets entries), or in the stash when bucket b* is staged
    // (the pass that reads the slots then writes no LDS list).  Else each
    // entry's slot is found by binary search over the prefixes.
    uint16_t *owner = nullptr;
    if (total <= 2u * kBuckets)
        owner = reinterpret_cast<uint16_t *>(stash + p.stash_cap + p.out_cap);
    else if (stage && total <= 4u * p.stash_cap)
        owner = reinterpret_cast<uint16_t *>(stash);
    if (owner) {
        for (uint32_t a = threadIdx.x; a < ps; a += kThreads)
            for (uint32_t j = pre[a]; j < pre[a + 1]; ++j) owner[j] = (uint16_t)a;
        __syncthreads();
    }

    // Entries [base + u * 64 + lane] of the slots' prefixes laid end to end,
    // 8 per lane, spread over the waves by the caller.
    constexpr int kB = 8;
    // The slot of entry j is the last a with pre[a] <= j; the eight searches
    // of a lane step together (eight LDS reads in flight per step).
    uint32_t top = 1;
    while (top * 2u <= ps) top *= 2u;  // the largest power of two <= ps
    auto load_batch = [&](uint32_t base, uint2 (&e)[kB]) {
        if (owner) {
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                const uint32_t j = base + (uint32_t)u * kWave + ln;
                e[u] = make_uint2(0u, kNone);
                if (j < total) {
                    const uint32_t a = owner[j];
                    e[u] = slot_data[(size_t)a * p.stash_cap + (j - pre[a])];
                }
            }
            return;
        }
        uint32_t a[kB], pa[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            a[u] = 0;
            pa[u] = 0;  // pre[0]
        }
        for (uint32_t h = top; h != 0; h >>= 1) {
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                const uint32_t j = base + (uint32_t)u * kWave + ln;
                const uint32_t m = a[u] + h;
                const uint32_t v = m < ps ? pre[m] : kNone;
                if (v <= j) {
                    a[u] = m;
                    pa[u] = v;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const uint32_t j = base + (uint32_t)u * kWave + ln;
            e[u] = make_uint2(0u, kNone);
            if (j < total) e[u] = slot_data[(size_t)a[u] * p.stash_cap + (j - pa[u])];
        }
    };
    // Rank of the key's next digit below the pass-0 digit (best first).
    constexpr int kSubW = (Key<KT>::kBits - kDigit) < kLaterDigit ? (Key<KT>::kBits - kDigit)
                                                                    : kLaterDigit;
    constexpr int kSubSh = Key<KT>::kBits - kDigit - kSubW;
    constexpr uint32_t kSubN = 1u << kSubW;
    auto sub_rank = [](uint32_t raw) {
        const uint32_t d = (Key<KT>::ord(raw) >> kSubSh) & (kSubN - 1u);
        return LARGEST ? kSubN - 1u - d : d;
    };

    // Bucket b* holds more keys than the LDS list: one more digit of its keys,
    // counted from the slots by the four waves, narrows it (the better
    // sub-buckets' keys become winners).  The count lives above the slot
    // prefix table, which takes at most kMaxWgPerSeg + 1 words.
    // With room for them in the staging area (a segment spread over every
    // XCD), the same pass also writes the keys of better buckets, which win
    // whatever the narrowing gives, and copies bucket b*'s entries in a row,
    // so that the pass after the narrowing reads them from there instead of
    // searching the slots again.
    bool refine = false;
    uint32_t dstar = 0, front = ks.before;
    Kth kf = ks;
    Prefix pf0 = pass0_prefix<KT, LARGEST>(ks.b);
    // Unsorted 4-byte values: the passes write each winner's source index in
    // its value slot, and one gather at the end replaces the indices by the
    // values, so that no batch waits for its values' loads.
    Params q = p;
    const bool late_vals = p.vals_in != nullptr && p.vindex == 0u && outbuf == nullptr;
    if (late_vals) q.vindex = 1u;
    uint2 *stg = stage ? p.ws_stage + (size_t)s * kStageCap : nullptr;
    if (!fast && sh.any_bad == 0) {
        uint32_t *sub = sh.hist + kBuckets - kSubN;
        for (uint32_t i = threadIdx.x; i < kSubN; i += kThreads) sub[i] = 0u;
        __syncthreads();
        // Software-pipelined: the next batch's loads are issued before this
        // batch's stores, so the wait for them does not also wait for the
        // stores (the memory counter retires in order).
        uint2 e[kB];
        if (w * kB * kWave < total) load_batch(w * kB * kWave, e);
        for (uint32_t base = w * kB * kWave; base < total; base += kWaves * kB * kWave) {
            uint2 en[kB];
            const bool more = base + kWaves * kB * kWave < total;
            if (more) load_batch(base + kWaves * kB * kWave, en);
            bool bet[kB], tie[kB];
            uint32_t nb = 0, nt = 0;
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                const uint32_t rk =
                    e[u].y != kNone ? rank0<KT, LARGEST>(Key<KT>::ord(e[u].x)) : kNone;
                bet[u] = rk < ks.b;
                tie[u] = rk == ks.b;
                if (tie[u]) atomicAdd(&sub[sub_rank(e[u].x)], 1u);
                if (stage) {
                    nb += (uint32_t)__popcll(__ballot(bet[u]));
                    nt += (uint32_t)__popcll(__ballot(tie[u]));
                }
            }
            if (!stage) {
                if (more)
#pragma unroll
                    for (int u = 0; u < kB; ++u) e[u] = en[u];
                continue;
            }
            uint32_t fb = 0, tb = 0;
            if (ln == 0) {
                fb = nb ? atomicAdd(&sh.nfront, nb) : 0u;
                tb = nt ? atomicAdd(&sh.nstage, nt) : 0u;
            }
            fb = wave_bcast(fb, 0);
            tb = wave_bcast(tb, 0);
            uint32_t fpos[kB];
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                const uint64_t mb = __ballot(bet[u]);
                const uint64_t mt = __ballot(tie[u]);
                const uint32_t pb = fb + lanes_below(mb);
                const uint32_t pt = tb + lanes_below(mt);
                fb += (uint32_t)__popcll(mb);
                tb += (uint32_t)__popcll(mt);
                fpos[u] = (bet[u] && pb < ks.before) ? pb : kNone;
                if (outbuf && fpos[u] != kNone) outbuf[pb] = e[u];
                if (tie[u] && pt < kStageCap) stg[pt] = e[u];
            }
            if (!outbuf) write_batch<KT, kB>(q, sg, fpos, e);
            if (more)
#pragma unroll
                for (int u = 0; u < kB; ++u) e[u] = en[u];
        }
        __syncthreads();
        const Kth f2 = wave_find(sub, kSubN, sg.k_i - ks.before);  // alike in every wave
        if (f2.found && f2.count <= p.stash_cap) {
            refine = true;
            dstar = f2.b;
            front = ks.before + f2.before;
            kf.before = front;
            kf.count = f2.count;
            pf0.hi = kSubSh;
            pf0.kmask |= (kSubN - 1u) << kSubSh;
            pf0.kpref |= (LARGEST ? kSubN - 1u - dstar : dstar) << kSubSh;
        }
        __syncthreads();
    }
    // Staged and narrowed: bucket b*'s entries in a row, the better buckets'
    // keys written already.
    const bool staged = refine && stage;
    const uint32_t nread = staged ? (sh.nstage < kStageCap ? sh.nstage : kStageCap) : total;
    if (fast || refine) {
        // Batches of 8 entries per lane, spread over the waves; positions
        // come from LDS counters, one reservation per batch and kind.
        auto fetch = [&](uint32_t base, uint2 (&e)[kB]) {
            if (staged) {
#pragma unroll
                for (int u = 0; u < kB; ++u) {
                    const uint32_t j = base + (uint32_t)u * kWave + ln;
                    e[u] = j < nread ? stg[j] : make_uint2(0u, kNone);
                }
            } else {
                load_batch(base, e);
            }
        };
        uint2 e[kB];
        if (w * kB * kWave < nread) fetch(w * kB * kWave, e);
        for (uint32_t base = w * kB * kWave; base < nread; base += kWaves * kB * kWave) {
            uint2 en[kB];
            const bool more = base + kWaves * kB * kWave < nread;
            if (more) fetch(base + kWaves * kB * kWave, en);
            uint32_t nb = 0, nt = 0;
            bool bet[kB], tie[kB];
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                const uint32_t rk =
                    e[u].y != kNone ? rank0<KT, LARGEST>(Key<KT>::ord(e[u].x)) : kNone;
                const uint32_t sr = refine ? sub_rank(e[u].x) : 0u;
                bet[u] = rk < ks.b || (refine && rk == ks.b && sr < dstar);
                tie[u] = rk == ks.b && (!refine || sr == dstar);
                nb += (uint32_t)__popcll(__ballot(bet[u]));
                nt += (uint32_t)__popcll(__ballot(tie[u]));
            }
            uint32_t fb = 0, tb = 0;
            if (ln == 0) {
                fb = nb ? atomicAdd(&sh.nfront, nb) : 0u;
                tb = nt ? atomicAdd(&sh.ntie, nt) : 0u;
            }
            fb = wave_bcast(fb, 0);
            tb = wave_bcast(tb, 0);
            uint32_t fpos[kB];
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                const uint64_t mb = __ballot(bet[u]);
                const uint64_t mt = __ballot(tie[u]);
                const uint32_t pb = fb + lanes_below(mb);
                const uint32_t pt = tb + lanes_below(mt);
                fb += (uint32_t)__popcll(mb);
                tb += (uint32_t)__popcll(mt);
                fpos[u] = (bet[u] && pb < front) ? pb : kNone;
                if (outbuf && fpos[u] != kNone) outbuf[pb] = e[u];
                if (tie[u] && pt < p.stash_cap) stash[pt] = e[u];
            }
            if (!outbuf) write_batch<KT, kB>(q, sg, fpos, e);
            if (more)
#pragma unroll
                for (int u = 0; u < kB; ++u) e[u] = en[u];
        }
    }
    __syncthreads();
    if (fast || refine) {
        // The four waves finish together on the list of keys at the prefix.
        block_finish<KT, LARGEST>(sh, outbuf, q, sg, stash,
                                  sh.ntie < p.stash_cap ? sh.ntie : p.stash_cap, kf, front, pf0);
        if (late_vals) {
            // Every winner is written: replace the indices by the values, 8
            // per thread in flight.
            __syncthreads();
            const size_t row = (size_t)sg.row * p.k;
            for (uint32_t o0 = threadIdx.x; o0 < sg.k_i; o0 += 8u * kThreads) {
                uint32_t v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const uint32_t o = o0 + (uint32_t)u * kThreads;
                    v[u] = o < sg.k_i ? p.vals_out[row + o] : kNone;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = v[u] < sg.n ? p.vals_in[sg.begin + v[u]] : kNone;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const uint32_t o = o0 + (uint32_t)u * kThreads;
                    if (o < sg.k_i) p.vals_out[row + o] = v[u];
                }
            }
        }
        return;
    }
    if (w != 0) return;

    Cands<KT> cand;
    cand.list = stash;
    cand.keys_in = p.keys_in;
    cand.begin = sg.begin;
    cand.n = sg.n;
    cand.nslices = ps;
    cand.slice = slice;
    cand.slot_info = info;
    cand.slot_cum = slot_cum;
    cand.slot_data = slot_data;
    cand.slot_cap = p.stash_cap;
    cand.bstar = ks.b;
    cand.lds = false;
    cand.count = 0;
    {
        // Rare: a slice lost candidates, or bucket b* does not fit in LDS
        // even narrowed by one more digit (heavy ties).  Pull what fits into
        // LDS, else leave the candidates in place.
        const Prefilter pf = prefilter<KT, LARGEST>(ks.b);
        const uint32_t cap = p.stash_cap;
        uint32_t got = 0;
        cand.visit([&](uint32_t r, uint32_t idx, bool act) {
            const bool keep = act && pf_key(pf, r);
            const uint64_t m = __ballot(keep);
            const uint32_t pos = got + lanes_below(m);
            if (keep && pos < cap) stash[pos] = make_uint2(r, idx);
            got += (uint32_t)__popcll(m);
        });
        wave_sync();
        if (got <= cap) {
            cand.lds = true;
            cand.count = got;
        }
    }
    wave_finish<KT, LARGEST>(sh.hist, outbuf, p, sg, cand, ks, 0u);
}

// A segment of one chunk per wave (each wave's quarter [wlo, whi) fits one
// chunk of U loads per lane): the keys stay in registers; every key is
// counted, every wave finds the exact k-th bucket in the finished histogram,
// and pushes its keys in or before that bucket straight into one candidate
// list (their number is known from the histogram); wave 0 finishes.  Waves
// 1..3 return after the last workgroup barrier.
template <int KT, bool LARGEST, int U>
__device__ __forceinline__ void small_block(Shared &sh, uint2 *stash, uint2 *outbuf, const Params &p,
                                            const Seg &sg, uint32_t wlo, uint32_t whi) {
    using Rg = WaveRange<KT, U>;
    constexpr int V = Rg::kVec;
    const uint32_t t = threadIdx.x;
    const uint32_t w = t / kWave;
    const uint32_t ln = lane_id();
    Rg L;
    L.init(p.keys_in, sg.begin, wlo, whi);
    uint32_t raw[Rg::kDw], vidx[Rg::kU];
    L.template load_chunk<true>(0, ln, raw, vidx);  // in flight during the clear
    const bool sv = ln < L.nscalar;
    const uint32_t si = sv ? L.scalar_idx(ln) : 0u;
    const uint32_t sx = sv ? L.load_scalar(si) : 0u;
    for (uint32_t i = t * 4; i < (uint32_t)kBuckets; i += 4 * kThreads)
        *reinterpret_cast<uint4 *>(&sh.hist[i]) = make_uint4(0u, 0u, 0u, 0u);
    if (t == 0) sh.ncand = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < Rg::kU; ++u)
#pragma unroll
        for (int e = 0; e < V; ++e)
            if (vidx[u] != kNone)
                atomicAdd(&sh.hist[rank0<KT, LARGEST>(Key<KT>::ord(Rg::key_at(raw, u * V + e)))], 1u);
    if (sv) atomicAdd(&sh.hist[rank0<KT, LARGEST>(Key<KT>::ord(sx))], 1u);
    __syncthreads();
    if (w == 0) {  // one scan, for every wave
        const Kth f = wave_find(sh.hist, kBuckets, sg.k_i);
        if (ln == 0) {
            sh.kb = f.b;
            sh.kbefore = f.before;
            sh.kcount = f.count;
        }
    }
    __syncthreads();
    Kth kw;
    kw.found = 1;
    kw.b = sh.kb;
    kw.before = sh.kbefore;
    kw.count = sh.kcount;
    const bool fits = kw.before + kw.count <= p.stash_cap;
    if (fits) {
        // Count this wave's candidates (ballots only), reserve their places
        // with one LDS atomic, then write them: per key one compare whose
        // ballot is masked by the load's validity on the scalar unit.
        const Prefilter pf = prefilter<KT, LARGEST>(kw.b);
        const uint64_t ms = __builtin_amdgcn_ballot_w64(pf_key(pf, sx)) & __ballot(sv);
        uint64_t vm[Rg::kU];
        uint32_t total = (uint32_t)__popcll(ms);
#pragma unroll
        for (int u = 0; u < Rg::kU; ++u) {
            vm[u] = __ballot(vidx[u] != kNone);
#pragma unroll
            for (int e = 0; e < V; ++e)
                total += (uint32_t)__popcll(
                    __builtin_amdgcn_ballot_w64(pf_key(pf, Rg::key_at(raw, u * V + e))) & vm[u]);
        }
        uint32_t base = 0;
        if (ln == 0 && total) base = atomicAdd(&sh.ncand, total);
        uint32_t pos = __builtin_amdgcn_readfirstlane(wave_bcast(base, 0));
        auto put = [&](uint64_t m, uint32_t x, uint32_t idx) {
            if (m == 0) return;
            if (__builtin_amdgcn_inverse_ballot_w64(m))
                stash[__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)m, pos))] =
                    make_uint2(x, idx);
            pos += (uint32_t)__popcll(m);
        };
        put(ms, sx, si);
#pragma unroll
        for (int u = 0; u < Rg::kU; ++u)
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const uint32_t x = Rg::key_at(raw, u * V + e);
                put(__builtin_amdgcn_ballot_w64(pf_key(pf, x)) & vm[u], x, vidx[u] + (uint32_t)e);
            }
    }
    __syncthreads();
    if (fits && sh.ncand > kBlockFinishMin) {
        block_finish<KT, LARGEST>(sh, outbuf, p, sg, stash, sh.ncand, kw, 0u);
        return;
    }
    if (w != 0) return;
    Cands<KT> cand;
    cand.list = stash;
    cand.count = fits ? sh.ncand : 0u;
    cand.lds = fits;  // else the passes read the segment again
    cand.keys_in = p.keys_in;
    cand.begin = sg.begin;
    cand.n = sg.n;
    cand.nslices = 1;
    cand.slice = sg.n;
    cand.slot_info = nullptr;
    cand.slot_cum = nullptr;
    cand.slot_data = nullptr;
    cand.slot_cap = p.stash_cap;
    cand.bstar = 0;
    wave_finish<KT, LARGEST>(sh.hist, outbuf, p, sg, cand, kw);
}

// ---------------------------------------------------------------------------
// Batches whose segments all fit one load of four per lane in each wave (the
// caller's size hint says so): a kernel with only that path, so that its
// register budget is not set by the streaming code.  A segment longer than
// the hint is still answered exactly: every wave counts its share, and wave 0
// finishes with passes that read the segment again.
// ---------------------------------------------------------------------------
template <int KT> constexpr uint32_t small_keys() { return kWaves * WaveRange<KT, 4>::kChunkKeys; }
static_assert(small_keys<SEGTOPK_KEY_F32>() == kSmallKeys32 && small_keys<SEGTOPK_KEY_BF16>() == kSmallKeys16,
              "the host's small-segment limits match one load of four per lane");
template <int KT> constexpr int small_waves() { return Key<KT>::kBytes == 4 ? kSmallWaves32 : kSmallWaves16; }

template <int KT, bool LARGEST>
__global__ __launch_bounds__(kThreads, (small_waves<KT>())) void topk_small_kernel(Params p) {
    __shared__ Shared sh;
    extern __shared__ uint4 dyn[];
    uint2 *stash = reinterpret_cast<uint2 *>(dyn);
    uint2 *outbuf = p.out_cap ? stash + p.stash_cap : nullptr;
    const uint32_t t = threadIdx.x;
    const uint32_t w = t / kWave;
    const uint32_t ln = lane_id();
    const int64_t s = (int64_t)blockIdx.x;
    if (s >= p.num_segments) return;

    Seg sg;
    sg.begin = p.offsets[s];
    const int64_t end = p.offsets[s + 1];
    sg.n = end > sg.begin ? (uint32_t)(end - sg.begin) : 0u;
    sg.k_i = sg.n < p.k ? sg.n : p.k;
    if (p.kseg) {
        const int32_t ks = p.kseg[s];
        const uint32_t ku = ks > 0 ? (uint32_t)ks : 0u;
        sg.k_i = ku < sg.k_i ? ku : sg.k_i;
    }
    sg.row = s;
    if (sg.k_i == 0) return;
    if (sg.n <= sg.k_i) {
        if (w == 0) wave_select_all<KT, LARGEST>(outbuf, p, sg);
        return;
    }
    uint32_t part = (sg.n + kWaves - 1) / kWaves;
    part = (part + 63u) & ~63u;
    const uint32_t wlo = w * part < sg.n ? w * part : sg.n;
    const uint32_t whi = (w + 1) * part < sg.n ? (w + 1) * part : sg.n;
    if (part <= WaveRange<KT, 4>::kChunkKeys) {
        small_block<KT, LARGEST, 4>(sh, stash, outbuf, p, sg, wlo, whi);
        return;
    }
    // Longer than the hint: count every key, then finish from the keys.
    for (uint32_t i = t * 4; i < (uint32_t)kBuckets; i += 4 * kThreads)
        *reinterpret_cast<uint4 *>(&sh.hist[i]) = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    {
        WaveRange<KT> L;
        L.init(p.keys_in, sg.begin, wlo, whi);
        L.for_each(ln, [&](uint32_t r, uint32_t, bool act) {
            if (act) atomicAdd(&sh.hist[rank0<KT, LARGEST>(Key<KT>::ord(r))], 1u);
        });
    }
    __syncthreads();
    if (w != 0) return;
    const Kth kw = wave_find(sh.hist, kBuckets, sg.k_i);
    Cands<KT> cand;
    cand.list = stash;
    cand.count = 0;
    cand.lds = false;
    cand.keys_in = p.keys_in;
    cand.begin = sg.begin;
    cand.n = sg.n;
    cand.nslices = 1;
    cand.slice = sg.n;
    cand.slot_info = nullptr;
    cand.slot_cum = nullptr;
    cand.slot_data = nullptr;
    cand.slot_cap = p.stash_cap;
    cand.bstar = 0;
    wave_finish<KT, LARGEST>(sh.hist, outbuf, p, sg, cand, kw);
}

// Waves per SIMD the kernel is built for.  With 4 loads per lane: 6 for
// 32-bit keys (at most 80 VGPRs; some spill, but the many-small-segment
// batches this serves gain more from the extra resident workgroups than they
// lose: on the 4096 x 4096 workload 6 beat 5, 7 and 8), 4 for 16-bit keys.
// With 8 loads per lane: 3 and 2.
template <int KT, int U> constexpr int topk_waves() {
    return U == 4 ? (Key<KT>::kBytes == 4 ? 6 : 4) : (Key<KT>::kBytes == 4 ? 3 : 2);
}

template <int KT, bool LARGEST, int U, bool SLICED>
__global__ __launch_bounds__(kThreads, (topk_waves<KT, U>())) void topk_kernel(Params p) {
    __shared__ Shared sh;
    extern __shared__ uint4 dyn[];
    uint2 *stash = reinterpret_cast<uint2 *>(dyn);  // kWaves regions of capw entries
    uint2 *outbuf = p.out_cap ? stash + p.stash_cap : nullptr;
    const uint32_t t = threadIdx.x;
    const uint32_t w = t / kWave;
    const uint32_t ln = lane_id();

    const uint32_t P = p.wg_per_seg;
    const uint32_t b = blockIdx.x;
    int64_t s;
    uint32_t q;
    if (p.spread) {
        // A batch of few segments: each segment's workgroups are consecutive,
        // so the dispatcher deals them over every XCD.
        s = (int64_t)(b / P);
        q = b % P;
    } else {
        // Workgroups of one segment share b % 8, the XCD they run on.
        const uint32_t qq = b >> 3;
        s = (int64_t)(qq / P) * 8 + (b & 7u);
        q = qq % P;
    }
    if (p.order) {  // one workgroup per segment, largest segments first
        if ((int64_t)b >= p.num_segments) return;
        s = p.order[b];
    }
    if (s >= p.num_segments) return;

    Seg sg;
    sg.begin = p.offsets[s];
    const int64_t end = p.offsets[s + 1];
    sg.n = end > sg.begin ? (uint32_t)(end - sg.begin) : 0u;
    sg.k_i = sg.n < p.k ? sg.n : p.k;
    if (p.kseg) {  // per-segment k, clamped to [0, k]
        const int32_t ks = p.kseg[s];
        const uint32_t ku = ks > 0 ? (uint32_t)ks : 0u;
        sg.k_i = ku < sg.k_i ? ku : sg.k_i;
    }
    sg.row = s;
    if (sg.k_i == 0) return;

    // Workgroups that share this segment.
    uint32_t ps = 1, slice = sg.n;
    if (P > 1 && sg.n > sg.k_i) {
        uint32_t sl = (uint32_t)(((uint64_t)sg.n + P - 1) / P);
        if (sl < p.min_slice) sl = p.min_slice;
        sl = (sl + 255u) & ~255u;
        ps = (uint32_t)(((uint64_t)sg.n + sl - 1) / sl);
        slice = sl;
    }
    if (q >= ps) return;

    if (sg.n <= sg.k_i) {  // select-all: one wave does it
        if (w == 0) wave_select_all<KT, LARGEST>(outbuf, p, sg);
        return;
    }

    // ---- pass 0: each wave streams a quarter of this workgroup's keys ----
    const uint32_t lo = q * slice;
    const uint32_t hi = (sg.n - lo) > slice ? lo + slice : sg.n;
    const uint32_t len = hi - lo;
    uint32_t part = (len + kWaves - 1) / kWaves;
    part = (part + 63u) & ~63u;
    const uint32_t wlo = lo + (w * part < len ? w * part : len);
    const uint32_t whi = lo + ((w + 1) * part < len ? (w + 1) * part : len);
    const uint32_t capw = p.stash_cap / kWaves;
    if (ps == 1 && part <= WaveRange<KT, U>::kChunkKeys) {
        small_block<KT, LARGEST, U>(sh, stash, outbuf, p, sg, wlo, whi);
        return;
    }
    for (uint32_t i = t * 4; i < (uint32_t)kBuckets; i += 4 * kThreads)
        *reinterpret_cast<uint4 *>(&sh.hist[i]) = make_uint4(0u, 0u, 0u, 0u);
    if (t == 0) {
        sh.rg = kBuckets - 1;
    }
    __syncthreads();
    Share share;
    share.rg = &sh.rg;
    // A segment spread over every XCD has one shared histogram per XCD (the
    // dispatcher deals workgroups to XCDs in turn): eight times fewer
    // workgroups add to and read each one.  Any of them gives a valid bound,
    // since each undercounts the segment.
    share.gearly = ps > 1 ? p.ws_early + ((size_t)s * (p.spread ? 8u : 1u) + (p.spread ? (b & 7u) : 0u)) *
                                             kBuckets
                          : nullptr;
    // The sliced variant keeps the workgroup's contributions in dynamic LDS
    // after the stash and the output staging.
    share.glast = (SLICED && ps > 1)
                      ? reinterpret_cast<uint32_t *>(stash + p.stash_cap + p.out_cap)
                      : nullptr;
    share.wave = w;
    share.spread = p.spread;
    if constexpr (Key<KT>::kBytes == 2 && !SLICED) {
        // After the stash and the output staging: four rings of loads, then
        // their element indices.
        uint4 *rb = reinterpret_cast<uint4 *>(stash + p.stash_cap + p.out_cap);
        share.ring = rb + w * kRingLoads;
        share.ring_idx = reinterpret_cast<uint32_t *>(rb + kWaves * kRingLoads) + w * kRingLoads;
    } else {
        share.ring = nullptr;
        share.ring_idx = nullptr;
    }
    const Pass0 r0 = wave_pass0_stash<KT, LARGEST, U, SLICED>(sh.hist, stash + w * capw, capw, p.keys_in,
                                                   sg.begin, wlo, whi, sg.k_i, share);
    if (ln == 0) {
        sh.wcount[w] = r0.count;
        sh.wbad[w] = 0;
        sh.wdefer[w] = r0.defer;
    }
    __syncthreads();
    bool anydefer = false;
    for (uint32_t v = 0; v < (uint32_t)kWaves; ++v) anydefer = anydefer || sh.wdefer[v] != 0;
    if (anydefer) {
        // Every key of the workgroup is counted now: stash the deferred
        // chunks under the workgroup's bound (computed alike by every wave).
        uint32_t Rf = wave_find(sh.hist, kBuckets, sg.k_i).b;
        if (ps > 1 && sh.rg < Rf) Rf = sh.rg;
        if (r0.defer != 0) {
            uint32_t cnt = r0.count;
            const bool ok = wave_reread<KT, LARGEST, U>(stash + w * capw, capw, cnt, p.keys_in,
                                                     sg.begin, wlo, whi, r0.defer, Rf);
            if (ln == 0) {
                sh.wcount[w] = cnt;
                sh.wbad[w] = ok ? 0u : 1u;
            }
        }
        __syncthreads();
    }
    // One workgroup per segment: every wave finds the workgroup's k-th bucket
    // itself (alike in every wave) and keeps, in place, the entries of its
    // own stash region within it; wave 0 then only closes the gaps between
    // the regions.  32-bit keys only: the 16-bit kernels measured slower with
    // it (their register budget is tighter).
    bool pgather = false;
    Kth kw1;
    kw1.found = 0;
    kw1.b = kBuckets - 1;
    kw1.before = 0;
    kw1.count = 0;
    if (Key<KT>::kBytes == 4 && ps == 1) {
        bool anybad = false;
        for (uint32_t v = 0; v < (uint32_t)kWaves; ++v) anybad = anybad || sh.wbad[v] != 0;
        if (!anybad) {
            pgather = true;
            kw1 = wave_find(sh.hist, kBuckets, sg.k_i);
            const Prefilter pf = prefilter<KT, LARGEST>(kw1.b);
            const uint32_t cnt = sh.wcount[w];
            uint2 *reg = stash + w * capw;
            uint32_t n = 0;
            for (uint32_t base = 0; base < cnt; base += kWave) {
                const uint32_t i = base + ln;
                const bool act = i < cnt;
                const uint2 e = act ? reg[i] : make_uint2(0u, 0u);
                const bool keep = act && pf_key(pf, e.x);
                const uint64_t m = __ballot(keep);
                wave_sync();
                if (keep) reg[n + lanes_below(m)] = e;
                n += (uint32_t)__popcll(m);
                wave_sync();
            }
            if (ln == 0) sh.wkept[w] = n;
        }
        __syncthreads();
    }
    if (w != 0) {
        // Wave 0 gathers the workgroup's candidates; with one workgroup per
        // segment a long list is finished by the four waves together, with
        // several workgroups per segment the others wait for the ticket and
        // help the last one.
        __syncthreads();
        if (ps == 1) {
            if (sh.ncand != kNone && sh.ncand > kBlockFinishMin) {
                Kth kb;
                kb.found = 1;
                kb.b = sh.kb;
                kb.before = sh.kbefore;
                kb.count = sh.kcount;
                block_finish<KT, LARGEST>(sh, outbuf, p, sg, stash, sh.ncand, kb, 0u);
            }
            return;
        }
        if (!sh.last) return;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        if constexpr (SLICED) slice_last<KT, LARGEST, SLICED>(sh, stash, outbuf, p, sg, s, P, ps, slice);
        return;
    }

    // ---- wave 0: this workgroup's k-th bucket, then its candidates ----
    const Kth kw = pgather ? kw1 : wave_find(sh.hist, kBuckets, sg.k_i);
    uint32_t R = kw.b;  // the last bucket when the range holds fewer keys
    // A bound shared by the segment's workgroups is valid for this slice too.
    if (ps > 1 && sh.rg < R) R = sh.rg;
    bool bad = false;
    for (uint32_t v = 0; v < (uint32_t)kWaves; ++v) bad = bad || sh.wbad[v] != 0;
    // Gather, in place, every stash entry with rank <= R (wave regions are
    // visited in order, so writes never pass reads).
    uint32_t ncand = 0;
    if (pgather) {
        // The regions hold only entries within the bound: move regions 1..3
        // down behind region 0 (each destination starts before its source).
        ncand = sh.wkept[0];
        for (uint32_t v = 1; v < (uint32_t)kWaves; ++v) {
            const uint32_t cnt = sh.wkept[v];
            const uint2 *src = stash + v * capw;
            for (uint32_t base = 0; base < cnt; base += kWave) {
                const uint32_t i = base + ln;
                const uint2 e = i < cnt ? src[i] : make_uint2(0u, 0u);
                wave_sync();
                if (i < cnt) stash[ncand + i] = e;
                wave_sync();
            }
            ncand += cnt;
        }
    } else if (!bad) {
        const Prefilter pf = prefilter<KT, LARGEST>(R);
        for (uint32_t v = 0; v < (uint32_t)kWaves; ++v) {
            const uint32_t cnt = sh.wcount[v];
            const uint2 *src = stash + v * capw;
            for (uint32_t base = 0; base < cnt; base += kWave) {
                const uint32_t i = base + ln;
                const bool act = i < cnt;
                const uint2 e = act ? src[i] : make_uint2(0u, 0u);
                const bool keep = act && pf_key(pf, e.x);
                const uint64_t m = __ballot(keep);
                wave_sync();
                if (keep) stash[ncand + lanes_below(m)] = e;
                ncand += (uint32_t)__popcll(m);
                wave_sync();
            }
        }
    }

    Cands<KT> cand;
    cand.list = stash;
    cand.count = ncand;
    cand.lds = !bad;
    cand.keys_in = p.keys_in;
    cand.begin = sg.begin;
    cand.n = sg.n;
    cand.nslices = 1;
    cand.slice = sg.n;
    cand.slot_info = nullptr;
    cand.slot_cum = nullptr;
    cand.slot_data = nullptr;
    cand.slot_cap = p.stash_cap;
    cand.bstar = 0;

    if (ps == 1) {
        // Publish the list; a long one is finished by the four waves.
        const bool blk = !bad && ncand > kBlockFinishMin;
        if (ln == 0) {
            sh.ncand = bad ? kNone : ncand;
            sh.kb = kw.b;
            sh.kbefore = kw.before;
            sh.kcount = kw.count;
        }
        __syncthreads();
        if (blk) {
            block_finish<KT, LARGEST>(sh, outbuf, p, sg, stash, ncand, kw, 0u);
            return;
        }
        wave_finish<KT, LARGEST>(sh.hist, outbuf, p, sg, cand, kw);
        return;
    }

    // ---- several workgroups per segment: publish this slice ----
    uint32_t *gh = p.ws_hist + (size_t)s * kBuckets;
    uint32_t *info = p.ws_slot_info + (size_t)s * P * 4;
    uint32_t *cum = p.ws_slot_cum + ((size_t)s * P + q) * kBuckets;
    uint2 *slot = p.ws_slot_data + ((size_t)s * P + q) * p.stash_cap;
    for (uint32_t i = ln; i <= R; i += kWave) {
        const uint32_t h = sh.hist[i];
        if (h) atomicAdd(&gh[i], h);
    }
    if (!bad) {
        // Counting sort of the candidates by rank into the slot: hist becomes
        // the exclusive prefix (a cursor per rank); after the scatter each
        // cursor holds the number of entries with rank <= r.
        uint32_t carry = 0;
        for (uint32_t base = 0; base <= R; base += kWave) {
            const uint32_t i = base + ln;
            const uint32_t h = i <= R ? sh.hist[i] : 0u;
            const uint32_t incl = wave_incl_sum(h);
            if (i <= R) sh.hist[i] = carry + incl - h;
            carry += wave_bcast(incl, kWave - 1);
        }
        wave_sync();
        for (uint32_t base = 0; base < ncand; base += kWave) {
            const uint32_t i = base + ln;
            if (i < ncand) {
                const uint2 e = stash[i];
                const uint32_t pos = atomicAdd(&sh.hist[rank0<KT, LARGEST>(Key<KT>::ord(e.x))], 1u);
                if (pos < p.stash_cap) slot[pos] = e;
            }
        }
        wave_sync();
        for (uint32_t i = ln; i <= R; i += kWave) cum[i] = sh.hist[i];
    }
    if (ln == 0) {
        info[4 * q + 0] = bad ? 0u : ncand;
        info[4 * q + 1] = bad ? 1u : 0u;
        info[4 * q + 2] = R;
    }
    // Release this slice's slot, histogram and info before taking a ticket;
    // the last arriver acquires all of them.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    uint32_t last = 0;
    if (ln == 0) last = (atomicAdd(&p.ws_ticket[s], 1u) == ps - 1) ? 1u : 0u;
    last = wave_bcast(last, 0);

    if (ln == 0) sh.last = last;
    __syncthreads();  // pairs with the one the other waves wait in
    if (!last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if constexpr (SLICED) slice_last<KT, LARGEST, SLICED>(sh, stash, outbuf, p, sg, s, P, ps, slice);
}

// Dynamic LDS above 64 KiB has to be allowed per kernel, once per device.
// Once per kernel and device (the flag is per template instance, that is
// per kernel).
template <auto Kernel> hipError_t allow_lds(size_t lds) {
    static std::atomic<uint64_t> done{0};
    if (lds <= 64 * 1024) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev < 64 ? (1ull << dev) : 0ull;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(Kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxDynLds);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

template <int KT, bool LARGEST, int U, bool SLICED>
hipError_t launch_u(const Params &p, uint32_t grid, size_t lds, hipStream_t st) {
    hipError_t e;
    if ((e = allow_lds<topk_kernel<KT, LARGEST, U, SLICED>>(lds)) != hipSuccess) return e;
    hipLaunchKernelGGL((topk_kernel<KT, LARGEST, U, SLICED>), dim3(grid), dim3(kThreads), lds, st, p);
    return hipGetLastError();
}

template <int KT, bool LARGEST>
hipError_t launch_small(const Params &p, uint32_t grid, size_t lds, hipStream_t st) {
    hipError_t e;
    if ((e = allow_lds<topk_small_kernel<KT, LARGEST>>(lds)) != hipSuccess) return e;
    hipLaunchKernelGGL((topk_small_kernel<KT, LARGEST>), dim3(grid), dim3(kThreads), lds, st, p);
    return hipGetLastError();
}

}  // namespace

template <int KT>
hipError_t launch_topk(const Params &p, bool largest, int variant, uint32_t grid, size_t lds,
                       hipStream_t st) {
    if (variant == kVariantSmall)
        return largest ? launch_small<KT, true>(p, grid, lds, st) : launch_small<KT, false>(p, grid, lds, st);
    if (largest) {
        if (variant == kVariantSliced) return launch_u<KT, true, kSplitU, true>(p, grid, lds, st);
        return variant == kVariantSplit ? launch_u<KT, true, kSplitU, false>(p, grid, lds, st)
                                        : launch_u<KT, true, 4, false>(p, grid, lds, st);
    }
    if (variant == kVariantSliced) return launch_u<KT, false, kSplitU, true>(p, grid, lds, st);
    return variant == kVariantSplit ? launch_u<KT, false, kSplitU, false>(p, grid, lds, st)
                                    : launch_u<KT, false, 4, false>(p, grid, lds, st);
}

template <int KT> int topk_per_cu(bool largest, size_t lds) {
    const void *fn = largest ? reinterpret_cast<const void *>(topk_kernel<KT, true, kSplitU, true>)
                             : reinterpret_cast<const void *>(topk_kernel<KT, false, kSplitU, true>);
    if (lds > 64 * 1024)
        (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxDynLds);
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, lds) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    return per_cu;
}

}  // namespace segtopk_impl
