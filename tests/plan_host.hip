// Host check of the launch plan (no GPU needed): the host source of the
// library is compiled host-only, with the per-key-type kernel entry points
// stubbed (3 resident workgroups per CU), and make_plan is driven over
// extreme requests -- k up to 2^31 - 1, one to 2^31 - 1 segments, every
// ordering, with and without a segment-size hint.  Each plan must come back
// (an alarm ends a hang), with LDS, grid and scratch sizes inside their limits.
#include "../segmented_top_selection_amd/csrc/segtopk.hip"

#include <csignal>
#include <cstdio>
#include <unistd.h>

namespace segtopk_impl {
template <int KT>
hipError_t launch_topk(const Params &, bool, int, uint32_t, size_t, hipStream_t) {
    return hipSuccess;
}
template <int KT> int topk_per_cu(bool, size_t) { return 3; }
template <int KT>
hipError_t launch_topk_plain(const Params &, bool, uint32_t, size_t, hipStream_t) {
    return hipSuccess;
}
}  // namespace segtopk_impl

static long g_bad = 0, g_plans = 0;

static void fail(const char *what, int64_t S, int64_t k, int ord, int64_t hint) {
    if (g_bad < 10)
        std::printf("  bad plan (%s): S=%lld k=%lld ordering=%d hint=%lld\n", what, (long long)S,
                    (long long)k, ord, (long long)hint);
    ++g_bad;
}

int main() {
    std::signal(SIGALRM, SIG_DFL);
    alarm(60);
    segtopk_keys keys{reinterpret_cast<const void *>(0x10000), reinterpret_cast<void *>(0x20000),
                      SEGTOPK_KEY_F32};
    segtopk_values vals{reinterpret_cast<const void *>(0x30000), reinterpret_cast<void *>(0x40000)};
    const int64_t Ss[] = {1, 2, 3, 7, 8, 9, 100, 255, 256, 1000, 2047, 2048, 100000, INT32_MAX};
    const int64_t ks[] = {1, 2, 63, 64, 256, 4096, 4097, 65536, (1ll << 30) + 1, INT32_MAX};
    const int64_t hints[] = {0, 1, 1000, 4096, 4097, 8192, 8193, 16384, 1ll << 20, 1ll << 40};
    for (int kt : {SEGTOPK_KEY_F32, SEGTOPK_KEY_BF16, SEGTOPK_KEY_U64})
        for (int64_t S : Ss)
            for (int64_t k : ks)
                for (int ord : {SEGTOPK_UNSORTED, SEGTOPK_STABLE_SORTED})
                    for (int64_t hint : hints) {
                        keys.type = kt;
                        const Request r{&keys, &vals, 4, reinterpret_cast<const int64_t *>(0x50000),
                                        S, k, nullptr, hint, SEGTOPK_MAX, SEGTOPK_GPU_TO_GPU,
                                        SEGTOPK_PREFER_SMALLER_INDEX, ord, nullptr};
                        const int v = validate(r);
                        if (v >= 0) {
                            if (ord != SEGTOPK_UNSORTED && k > SEGTOPK_MAX_SORTED_K &&
                                v != SEGTOPK_NOT_SUPPORTED)
                                fail("sorted k limit", S, k, ord, hint);
                            continue;
                        }
                        Plan pl;
                        const int st = make_plan(r, 0, pl);
                        ++g_plans;
                        if (st != SEGTOPK_OK) {
                            fail("status", S, k, ord, hint);
                            continue;
                        }
                        const Params &p = pl.p;
                        if (kt == SEGTOPK_KEY_U64) {
                            // 64-bit keys: one workgroup per segment, no scratch
                            if (pl.grid != (uint64_t)S || pl.scratch_bytes || pl.lds > kMaxDynLds ||
                                (ord != SEGTOPK_UNSORTED && p.out_cap < (uint64_t)k))
                                fail("64-bit plan", S, k, ord, hint);
                            continue;
                        }
                        if (p.stash_cap < 1024 || p.stash_cap > 8192 ||
                            (p.stash_cap & (p.stash_cap - 1)))
                            fail("stash size", S, k, ord, hint);
                        if (8 * ((size_t)p.stash_cap + p.out_cap) > kMaxDynLds || pl.lds > kMaxDynLds)
                            fail("LDS", S, k, ord, hint);
                        if (ord != SEGTOPK_UNSORTED && p.out_cap < (uint64_t)k)
                            fail("sorted staging smaller than k", S, k, ord, hint);
                        if (p.wg_per_seg < 1 || p.wg_per_seg > kMaxWgPerSeg)
                            fail("workgroups per segment", S, k, ord, hint);
                        if (pl.grid == 0 || pl.grid > 0x7FFFFFFFu) fail("grid", S, k, ord, hint);
                        const uint64_t need = p.wg_per_seg == 1 ? (uint64_t)S
                                              : p.spread ? (uint64_t)S * p.wg_per_seg
                                                         : (uint64_t)(S + 7) / 8 * 8 * p.wg_per_seg;
                        if (pl.grid != need) fail("grid shape", S, k, ord, hint);
                        if (p.spread && (S >= 8 || pl.grid > 768)) fail("spread", S, k, ord, hint);
                        if (p.wg_per_seg > 1 && pl.scratch_bytes <
                                (uint64_t)S * p.wg_per_seg * p.stash_cap * 8)
                            fail("scratch", S, k, ord, hint);
                        if (S >= 2048 && (pl.scratch_bytes != 0 || p.wg_per_seg != 1))
                            fail("many segments need no scratch", S, k, ord, hint);
                        // The small-segment kernel: whenever the hint keeps every
                        // segment within one load of four per lane in each wave.
                        const uint64_t small = kt == SEGTOPK_KEY_BF16 ? kSmallKeys16 : kSmallKeys32;
                        const bool want_small = hint > 0 && (uint64_t)hint <= small;
                        if ((pl.variant == kVariantSmall) != want_small)
                            fail("small-segment kernel choice", S, k, ord, hint);
                        if (pl.variant == kVariantSmall &&
                            (pl.grid != (uint64_t)S || pl.scratch_bytes || pl.order || pl.sliced ||
                             p.wg_per_seg != 1 || pl.lds != 8 * ((size_t)p.stash_cap + p.out_cap)))
                            fail("small-segment plan", S, k, ord, hint);
                        if (pl.sliced) {
                            // Zeroed words: merged histograms, shared histograms
                            // (one per XCD when spread), tickets; a spread plan
                            // ends with the staging area of bucket b*.
                            const uint64_t ne = (p.spread ? 8u : 1u) * (uint64_t)S * kBuckets;
                            if (pl.n_hist != (uint64_t)S * kBuckets || pl.n_early != ne ||
                                pl.zero_words != pl.n_hist + ne + (uint64_t)S)
                                fail("zeroed words", S, k, ord, hint);
                            const uint64_t slots = pl.data_off +
                                                   (uint64_t)S * p.wg_per_seg * p.stash_cap * 8;
                            if (p.spread ? (pl.stage_off != slots ||
                                            pl.scratch_bytes != slots + (uint64_t)S * kStageCap * 8)
                                         : (pl.stage_off != 0 || pl.scratch_bytes != slots))
                                fail("slots and staging", S, k, ord, hint);
                            if (pl.data_off < 4 * (pl.zero_words + pl.info_words) || (pl.data_off & 255))
                                fail("layout order", S, k, ord, hint);
                        }
                    }
    std::printf("plans checked: %ld, bad: %ld\n", g_plans, g_bad);
    return g_bad != 0;
}
