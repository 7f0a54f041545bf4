// topk_plain_kernel.h -- segmented top-k for the key widths the streaming
// kernels do not serve: 64-bit keys (uint64, int64, binary64) and 8-bit keys
// (uint8, int8).
//
// The same method as the 32- and 16-bit kernels -- most-significant-digit radix
// selection with early stop, then a final filter that writes every key beyond
// the splitter plus exactly enough splitter-equal keys, ties narrowed by
// source index in the deterministic modes --
//   [PR "Implement Segmented TopK using Thread-Block-Clusters", §1.2 Radix
//    (digit) top-k, §1.4 Early stop, §1.5 Final filter and output placement,
//    §1.6 Determinism / tie-breaking]
// laid out more plainly:
//  * one workgroup of four wave64 per segment;
//  * 11-bit digits (64 = 5 x 11 + 9 bits; an 8-bit key is one digit of 8
//    bits), every pass a histogram of the next
//    digit of the keys that match the splitter so far, scanned best-first;
//    buckets are reversed for MAX after the order-preserving transform, which
//    folds -0.0 onto +0.0   [PR "Fix BlockTopK +/-0.0 handling", Fix];
//  * while the keys that match the prefix are more than the LDS candidate list
//    holds, each pass streams the segment from HBM; once they fit, one more
//    pass gathers them into LDS (and writes at once the keys already known to
//    win), and the remaining passes, the index passes and the final filter run
//    on that list;
//  * sorted output is staged in LDS and sorted by (ordered key best-first,
//    index ascending) with a bitonic network over the whole workgroup.
#pragma once

#include "topk_kernel.h"

namespace segtopk_impl {
namespace {

constexpr uint32_t kCand64 = 2048;  // LDS candidate list entries (16 bytes each)

// Order-preserving bits, widened to 64: ord(a) < ord(b) exactly when a < b,
// ord(-0.0) == ord(+0.0).  Raw is the key's storage type.
template <int KT> struct KeyW;
template <> struct KeyW<SEGTOPK_KEY_U64> {
    typedef uint64_t Raw;
    static constexpr int kBits = 64;
    __host__ __device__ __forceinline__ static uint64_t ord(Raw r) { return r; }
};
template <> struct KeyW<SEGTOPK_KEY_I64> {
    typedef uint64_t Raw;
    static constexpr int kBits = 64;
    __host__ __device__ __forceinline__ static uint64_t ord(Raw r) {
        return r ^ 0x8000000000000000ull;
    }
};
template <> struct KeyW<SEGTOPK_KEY_F64> {
    typedef uint64_t Raw;
    static constexpr int kBits = 64;
    __host__ __device__ __forceinline__ static uint64_t ord(Raw r) {
        r = (r == 0x8000000000000000ull) ? 0ull : r;  // -0.0 joins +0.0
        return r ^ ((uint64_t)((int64_t)r >> 63) | 0x8000000000000000ull);
    }
};
template <> struct KeyW<SEGTOPK_KEY_U8> {
    typedef uint8_t Raw;
    static constexpr int kBits = 8;
    __host__ __device__ __forceinline__ static uint64_t ord(Raw r) { return r; }
};
template <> struct KeyW<SEGTOPK_KEY_I8> {
    typedef uint8_t Raw;
    static constexpr int kBits = 8;
    __host__ __device__ __forceinline__ static uint64_t ord(Raw r) { return (uint64_t)(r ^ 0x80u); }
};

struct Shared64 {
    uint32_t hist[kBuckets];
    uint32_t b, before, count, ncand, nfront, ntie, pad0, pad1;
};

// "better than" on masked ordered keys.
template <bool LARGEST> __device__ __forceinline__ bool better64(uint64_t a, uint64_t b) {
    return LARGEST ? a > b : a < b;
}

// Output order: better ordered key first, then smaller index; padding last.
template <bool LARGEST> __device__ __forceinline__ bool out_before64(uint4 a, uint4 b) {
    if (a.z == kNone) return false;
    if (b.z == kNone) return true;
    const uint64_t oa = ((uint64_t)a.y << 32) | a.x, ob = ((uint64_t)b.y << 32) | b.x;
    if (oa != ob) return better64<LARGEST>(oa, ob);
    return a.z < b.z;
}

template <int KT, bool LARGEST>
__global__ __launch_bounds__(kThreads) void topk_plain_kernel(Params p) {
    typedef typename KeyW<KT>::Raw Raw;
    __shared__ Shared64 sh;
    extern __shared__ uint4 dyn64[];
    uint4 *cand = dyn64;                                    // kCand64 entries
    uint4 *stage = p.out_cap ? dyn64 + kCand64 : nullptr;   // sorted/staged output
    const uint32_t t = threadIdx.x;
    const uint32_t w = t / kWave;
    const uint32_t ln = lane_id();
    const int64_t s = blockIdx.x;
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
    const Raw *keys = static_cast<const Raw *>(p.keys_in) + sg.begin;

    // Places one winner: staged for sorting, or written out.
    auto emit = [&](uint32_t pos, Raw raw, uint32_t idx) {
        if (pos >= sg.k_i) return;
        if (stage) {
            const uint64_t o = KeyW<KT>::ord(raw);
            stage[pos] = make_uint4((uint32_t)o, (uint32_t)(o >> 32), idx, 0u);
            return;
        }
        const size_t oi = (size_t)sg.row * p.k + pos;
        static_cast<Raw *>(p.keys_out)[oi] = raw;
        if (p.vals_in) val_store(p, oi, val_load(p, sg, idx));
    };

    // Visits every key whose ordered bits match pref under mask: from the LDS
    // list (which holds the keys that matched when it was gathered; later
    // passes narrow the prefix further), or from the whole segment in HBM.
    bool in_lds = false;
    uint32_t ncand = 0;
    uint64_t mask = 0, pref = 0;
    auto visit = [&](auto &&f) {
        if (in_lds) {
            for (uint32_t i = t; i < ncand; i += kThreads) {
                const uint4 e = cand[i];
                const uint64_t o = ((uint64_t)e.y << 32) | e.x;
                if ((o & mask) == pref) f(o, e.z);
            }
        } else {
            for (uint32_t i = t; i < sg.n; i += kThreads) {
                const uint64_t o = KeyW<KT>::ord(keys[i]);
                if ((o & mask) == pref) f(o, i);
            }
        }
    };

    if (sg.n <= sg.k_i) {
        // Select-all: every key wins.
        for (uint32_t i = t; i < sg.n; i += kThreads) emit(i, keys[i], i);
    } else {
        // ---- key digits ----
        uint32_t krem = sg.k_i, front = 0, placed = 0;
        bool done = false;
        int shift = KeyW<KT>::kBits;
        while (!done && shift > 0) {
            const int wd = shift < kDigit ? shift : kDigit;
            const int sh_ = shift - wd;
            const uint32_t nb = 1u << wd;
            for (uint32_t i = t; i < nb; i += kThreads) sh.hist[i] = 0u;
            __syncthreads();
            visit([&](uint64_t o, uint32_t) {
                const uint32_t d = (uint32_t)(o >> sh_) & (nb - 1u);
                atomicAdd(&sh.hist[LARGEST ? nb - 1u - d : d], 1u);
            });
            __syncthreads();
            if (w == 0) {
                const Kth f = wave_find(sh.hist, nb, krem);
                if (ln == 0) {
                    sh.b = f.b;
                    sh.before = f.before;
                    sh.count = f.count;
                }
            }
            __syncthreads();
            const uint32_t fb = sh.b, fbefore = sh.before, fcount = sh.count;
            krem -= fbefore;
            front += fbefore;
            pref |= (uint64_t)(LARGEST ? nb - 1u - fb : fb) << sh_;
            mask |= (uint64_t)(nb - 1u) << sh_;
            done = fcount == krem;
            shift = sh_;
            if (!in_lds && !done && fcount <= kCand64) {
                // Gather the keys at the prefix into LDS; the keys better than
                // it (front of them, all winners) go out now.
                if (t == 0) {
                    sh.ncand = 0;
                    sh.nfront = 0;
                }
                __syncthreads();
                const uint64_t pmask = mask, ppref = pref;
                for (uint32_t i = t; i < sg.n; i += kThreads) {
                    const Raw raw = keys[i];
                    const uint64_t o = KeyW<KT>::ord(raw);
                    const uint64_t m = o & pmask;
                    if (m == ppref) {
                        const uint32_t at = atomicAdd(&sh.ncand, 1u);
                        if (at < kCand64) cand[at] = make_uint4((uint32_t)o, (uint32_t)(o >> 32), i, 0u);
                    } else if (better64<LARGEST>(m, ppref)) {
                        emit(atomicAdd(&sh.nfront, 1u), raw, i);
                    }
                }
                __syncthreads();
                ncand = sh.ncand < kCand64 ? sh.ncand : kCand64;
                in_lds = true;
                placed = front;
                __syncthreads();
            }
        }

        // ---- deterministic modes: the splitter-equal keys by source index ----
        const uint32_t ties = krem;
        bool by_index = false;
        uint32_t imask = 0, ipref = 0;
        const bool pl = p.prefer_larger != 0;
        if (!done && p.det) {
            by_index = true;
            int hi = 32 - __clz((int)(sg.n - 1u));
            while (!done && hi > 0) {
                const int wd = hi < kLaterDigit ? hi : kLaterDigit;
                const int sh_ = hi - wd;
                const uint32_t nb = 1u << wd;
                for (uint32_t i = t; i < nb; i += kThreads) sh.hist[i] = 0u;
                __syncthreads();
                visit([&](uint64_t o, uint32_t idx) {
                    if ((o & mask) == pref && (idx & imask) == ipref) {
                        const uint32_t d = (idx >> sh_) & (nb - 1u);
                        atomicAdd(&sh.hist[pl ? nb - 1u - d : d], 1u);
                    }
                });
                __syncthreads();
                if (w == 0) {
                    const Kth f = wave_find(sh.hist, nb, krem);
                    if (ln == 0) {
                        sh.b = f.b;
                        sh.before = f.before;
                        sh.count = f.count;
                    }
                }
                __syncthreads();
                krem -= sh.before;
                ipref |= (pl ? nb - 1u - sh.b : sh.b) << sh_;
                imask |= (nb - 1u) << sh_;
                done = sh.count == krem;
                hi = sh_;
                __syncthreads();
            }
        }

        // ---- final filter: better keys to [placed, front), ties to [front, k_i) ----
        if (t == 0) {
            sh.nfront = placed;
            sh.ntie = 0;
        }
        __syncthreads();
        auto classify = [&](uint64_t o, uint32_t idx, Raw raw) {
            const uint64_t m = o & mask;
            if (better64<LARGEST>(m, pref)) {
                const uint32_t at = atomicAdd(&sh.nfront, 1u);
                if (at < front) emit(at, raw, idx);
            } else if (m == pref) {
                bool take = true;
                if (by_index) {
                    const uint32_t im = idx & imask;
                    take = pl ? im >= ipref : im <= ipref;
                }
                if (take) {
                    const uint32_t at = atomicAdd(&sh.ntie, 1u);
                    if (at < ties) emit(front + at, raw, idx);
                }
            }
        };
        if (in_lds) {
            for (uint32_t i = t; i < ncand; i += kThreads) {
                const uint4 e = cand[i];
                classify(((uint64_t)e.y << 32) | e.x, e.z, keys[e.z]);
            }
        } else {
            for (uint32_t i = t; i < sg.n; i += kThreads) {
                const Raw raw = keys[i];
                classify(KeyW<KT>::ord(raw), i, raw);
            }
        }
    }

    if (!stage) return;
    // ---- staged output: sort (sorted orderings), then write ----
    __syncthreads();
    const uint32_t cnt = sg.k_i;
    uint32_t P = 1;
    while (P < cnt) P <<= 1;
    for (uint32_t i = cnt + t; i < P; i += kThreads) stage[i] = make_uint4(0u, 0u, kNone, 0u);
    __syncthreads();
    if (p.sorted) {
        for (uint32_t size = 2; size <= P; size <<= 1) {
            for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
                for (uint32_t i = t; i < (P >> 1); i += kThreads) {
                    const uint32_t lo = 2 * i - (i & (stride - 1));
                    const uint32_t hi = lo + stride;
                    const bool asc = (lo & size) == 0;
                    const uint4 a = stage[lo], b = stage[hi];
                    if (out_before64<LARGEST>(b, a) == asc) {
                        stage[lo] = b;
                        stage[hi] = a;
                    }
                }
                __syncthreads();
            }
        }
    }
    for (uint32_t i = t; i < cnt; i += kThreads) {
        const uint4 e = stage[i];
        if (e.z == kNone) continue;
        const size_t oi = (size_t)sg.row * p.k + i;
        static_cast<Raw *>(p.keys_out)[oi] = keys[e.z];
        if (p.vals_in) val_store(p, oi, val_load(p, sg, e.z));
    }
}

// Once per kernel and device (the flag is per template instance).
template <auto Kernel> hipError_t allow_lds_plain(size_t lds) {
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

}  // namespace

template <int KT>
hipError_t launch_topk_plain(const Params &p, bool largest, uint32_t grid, size_t lds,
                             hipStream_t st) {
    hipError_t e;
    if (largest) {
        if ((e = allow_lds_plain<topk_plain_kernel<KT, true>>(lds)) != hipSuccess) return e;
        hipLaunchKernelGGL((topk_plain_kernel<KT, true>), dim3(grid), dim3(kThreads), lds, st, p);
    } else {
        if ((e = allow_lds_plain<topk_plain_kernel<KT, false>>(lds)) != hipSuccess) return e;
        hipLaunchKernelGGL((topk_plain_kernel<KT, false>), dim3(grid), dim3(kThreads), lds, st, p);
    }
    return hipGetLastError();
}

}  // namespace segtopk_impl
