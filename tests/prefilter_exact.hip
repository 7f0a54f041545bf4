// Host check of the key transforms used by the top-k kernels: for every key
// type and direction, the raw-bit test built for a bucket bound passes exactly
// the keys whose order-preserving bits are within the bound (-0.0 counted as
// +0.0), the per-lane chunk reduction passes exactly when one of the chunk's
// keys does, and the inverse of the order-preserving bits gives back every
// key's raw bits (-0.0 comes back as +0.0, which the sort never relies on:
// it carries the raw bits whenever a -0.0 is present).  16-bit keys: every bit pattern against every pass-0
// bound; 32-bit keys: boundary patterns plus seeded random ones.  Built
// host-only; prints the number of mismatches and exits non-zero on any.
#include "../segmented_top_selection_amd/csrc/topk_kernel.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <random>
#include <string>
#include <vector>

using namespace segtopk_impl;

static long g_bad = 0;

template <int KT, bool LARGEST>
static void check(const std::vector<uint32_t> &keys, const std::vector<uint32_t> &thrs,
                  const char *name) {
    long bad = 0, pass = 0;
    for (uint32_t thr : thrs) {
        const Prefilter f = prefilter_thr<KT, LARGEST>(thr);
        for (uint32_t x : keys) {
            const uint32_t o = Key<KT>::ord(x);
            const bool want = LARGEST ? o >= thr : o <= thr;
            const bool got = pf_key(f, x);
            pass += want;
            if (got != want) {
                if (bad < 5)
                    std::printf("  %s %s thr=%08x key=%08x want=%d got=%d\n", name,
                                LARGEST ? "max" : "min", thr, x, want, got);
                ++bad;
            }
        }
    }
    // Chunk reduction: 16 dwords (32 16-bit keys or 16 32-bit keys), random
    // draws from the key set; it passes exactly when some key passes.
    std::mt19937 rng(7);
    std::uniform_int_distribution<size_t> pick(0, keys.size() - 1);
    for (uint32_t thr : thrs) {
        const Prefilter f = prefilter_thr<KT, LARGEST>(thr);
        for (int rep = 0; rep < 8; ++rep) {
            uint32_t d[16];
            bool any = false;
            for (int j = 0; j < 16; ++j) {
                uint32_t a = keys[pick(rng)], b = keys[pick(rng)];
                if (Key<KT>::kBytes == 2) {
                    d[j] = (a & 0xFFFFu) | (b << 16);
                    any = any || pf_key(f, a & 0xFFFFu) || pf_key(f, b & 0xFFFFu);
                } else {
                    d[j] = a;
                    any = any || pf_key(f, a);
                }
            }
            if (pf_chunk<KT>(f, d) != any) {
                if (bad < 5)
                    std::printf("  %s %s thr=%08x chunk reduction mismatch\n", name,
                                LARGEST ? "max" : "min", thr);
                ++bad;
            }
        }
    }
    std::printf("%-4s %s: %zu thresholds x %zu keys, %ld passing, %ld mismatches\n", name,
                LARGEST ? "max" : "min", thrs.size(), keys.size(), pass, bad);
    g_bad += bad;
}

template <int KT> static void run(const std::vector<uint32_t> &keys, const char *name) {
    constexpr uint32_t H = 1u << (Key<KT>::kBits - 1);
    long inv_bad = 0;
    for (uint32_t x : keys) {
        const uint32_t want = (Key<KT>::kSignMag && x == H) ? 0u : x;
        if (Key<KT>::inv_ord(Key<KT>::ord(x)) != want) {
            if (inv_bad < 5) std::printf("  %s inv_ord(ord(%08x)) = %08x\n", name, x, Key<KT>::inv_ord(Key<KT>::ord(x)));
            ++inv_bad;
        }
    }
    std::printf("%-4s inverse of the ordered bits: %zu keys, %ld mismatches\n", name, keys.size(), inv_bad);
    g_bad += inv_bad;
    std::vector<uint32_t> tmax, tmin;
    for (uint32_t R = 0; R < (uint32_t)kBuckets; ++R) {
        tmax.push_back(rank_thr<KT, true>(R));
        tmin.push_back(rank_thr<KT, false>(R));
    }
    // Thresholds next to zero, whatever the digit width.
    for (uint32_t t : {H - 2u, H - 1u, H, H + 1u, H + 2u, 0u, 1u, 2u * H - 1u}) {
        tmax.push_back(t);
        tmin.push_back(t);
    }
    check<KT, true>(keys, tmax, name);
    check<KT, false>(keys, tmin, name);
}

// ---------------------------------------------------------------------------
// The order-preserving transform itself, against IEEE / integer comparison of
// the decoded keys (decoded here by the compiler's own conversions, not by
// the kernel header): a < b exactly when ord(a) < ord(b), and a == b exactly
// when ord(a) == ord(b), so that -0.0 and +0.0 share one ordered value.  NaN
// patterns are left out (outside the contract).  Checked by sorting the keys
// by value and walking neighbours: ord must rise strictly across every rise of
// the value and stay equal within every run of equal values, which gives both
// equivalences for every pair.
//   [PR "Fix BlockTopK +/-0.0 handling", Description: Cause / Fix]
// ---------------------------------------------------------------------------
template <int KT> static double decode(uint32_t x) {
    if constexpr (KT == SEGTOPK_KEY_F32) {
        float f;
        std::memcpy(&f, &x, 4);
        return (double)f;
    } else if constexpr (KT == SEGTOPK_KEY_BF16) {
        const uint32_t w = x << 16;
        float f;
        std::memcpy(&f, &w, 4);
        return (double)f;
    } else if constexpr (KT == SEGTOPK_KEY_F16) {
        const uint16_t h16 = (uint16_t)x;
        _Float16 h;
        std::memcpy(&h, &h16, 2);
        return (double)h;
    } else if constexpr (KT == SEGTOPK_KEY_U32 || KT == SEGTOPK_KEY_U16) {
        return (double)x;
    } else if constexpr (KT == SEGTOPK_KEY_I16) {
        return (double)(int16_t)(uint16_t)x;
    } else {
        return (double)(int32_t)x;
    }
}

// A transform with a planted mistake (the -0.0 fold dropped), to show that
// the check below catches one.
template <int KT> static uint32_t ord_perturbed(uint32_t r) {
    if constexpr (Key<KT>::kSignMag) {
        constexpr uint32_t H = 1u << (Key<KT>::kBits - 1);
        constexpr uint32_t M = Key<KT>::kBits == 32 ? 0xFFFFFFFFu : 0xFFFFu;
        return (r & H) ? (~r & M) : (r | H);
    } else {
        return Key<KT>::ord(r) ^ 1u;
    }
}

static bool g_perturbed = false;

template <int KT> static void check_order(const std::vector<uint32_t> &in, const char *name) {
    std::vector<std::pair<double, uint32_t>> v;
    for (uint32_t x : in) {
        const double d = decode<KT>(x);
        if (!std::isnan(d)) v.push_back({d, x});
    }
    std::sort(v.begin(), v.end());
    auto ord = [](uint32_t x) { return g_perturbed ? ord_perturbed<KT>(x) : Key<KT>::ord(x); };
    long bad = 0;
    for (size_t i = 1; i < v.size(); ++i) {
        const uint32_t oa = ord(v[i - 1].second), ob = ord(v[i].second);
        const bool ok = v[i - 1].first < v[i].first ? oa < ob : oa == ob;
        if (!ok) {
            if (bad < 5)
                std::printf("  %s ord not monotone: %08x (%g) -> %08x, %08x (%g) -> %08x\n", name,
                            v[i - 1].second, v[i - 1].first, oa, v[i].second, v[i].first, ob);
            ++bad;
        }
    }
    std::printf("%-4s ordered bits vs numeric order: %zu keys, %ld mismatches\n", name, v.size(),
                bad);
    g_bad += bad;
}

int main(int argc, char **argv) {
    if (argc > 1 && std::string(argv[1]) == "--perturbed") {
        // Only the transform check, with the planted mistake: must report
        // mismatches for every key type.
        g_perturbed = true;
        std::vector<uint32_t> k16;
        for (uint32_t x = 0; x < 65536u; ++x) k16.push_back(x);
        std::vector<uint32_t> k32 = {0x00000000u, 0x80000000u, 0x3F800000u, 0xBF800000u, 1u, 2u, 3u};
        long types_caught = 0;
        long before = g_bad;
        check_order<SEGTOPK_KEY_BF16>(k16, "bf16"); types_caught += g_bad > before; before = g_bad;
        check_order<SEGTOPK_KEY_F16>(k16, "f16"); types_caught += g_bad > before; before = g_bad;
        check_order<SEGTOPK_KEY_F32>(k32, "f32"); types_caught += g_bad > before; before = g_bad;
        check_order<SEGTOPK_KEY_U32>(k32, "u32"); types_caught += g_bad > before; before = g_bad;
        check_order<SEGTOPK_KEY_I32>(k32, "i32"); types_caught += g_bad > before; before = g_bad;
        check_order<SEGTOPK_KEY_U16>(k16, "u16"); types_caught += g_bad > before; before = g_bad;
        check_order<SEGTOPK_KEY_I16>(k16, "i16"); types_caught += g_bad > before;
        std::printf("perturbed transform caught for %ld of 7 key types\n", types_caught);
        return types_caught == 7 ? 0 : 1;
    }
    std::vector<uint32_t> k16;
    for (uint32_t x = 0; x < 65536u; ++x) k16.push_back(x);
    std::vector<uint32_t> k32 = {0x00000000u, 0x80000000u, 0x00000001u, 0x80000001u, 0x007FFFFFu,
                                 0x807FFFFFu, 0x00800000u, 0x80800000u, 0x3F800000u, 0xBF800000u,
                                 0x7F7FFFFFu, 0xFF7FFFFFu, 0x7F800000u, 0xFF800000u, 0x7FFFFFFFu,
                                 0xFFFFFFFFu, 0x7FC00000u, 0xFFC00000u, 0x40000000u, 0xC0000000u};
    std::mt19937 rng(1234);
    for (int i = 0; i < 4000; ++i) k32.push_back((uint32_t)rng());
    // Patterns on and next to every 11-bit bucket boundary.
    for (uint32_t b = 0; b < 2048u; ++b) {
        const uint32_t base = b << 21;
        for (uint32_t d : {0u, 1u, (1u << 21) - 1u}) k32.push_back(base + d);
        k32.push_back(base - 1u);
    }
    check_order<SEGTOPK_KEY_BF16>(k16, "bf16");
    check_order<SEGTOPK_KEY_F16>(k16, "f16");
    check_order<SEGTOPK_KEY_U16>(k16, "u16");
    check_order<SEGTOPK_KEY_I16>(k16, "i16");
    {
        // 32-bit keys: the boundary patterns, every pattern next to a power of
        // two, and a million seeded random ones.
        std::vector<uint32_t> w = k32;
        for (int e = 0; e < 32; ++e)
            for (uint32_t d : {0u, 1u, 0xFFFFFFFFu})
                for (uint32_t sgn : {0u, 0x80000000u}) w.push_back(((1u << e) + d) ^ sgn);
        std::mt19937 r2(99);
        for (int i = 0; i < 1000000; ++i) w.push_back((uint32_t)r2());
        check_order<SEGTOPK_KEY_F32>(w, "f32");
        check_order<SEGTOPK_KEY_U32>(w, "u32");
        check_order<SEGTOPK_KEY_I32>(w, "i32");
    }
    run<SEGTOPK_KEY_BF16>(k16, "bf16");
    run<SEGTOPK_KEY_F16>(k16, "f16");
    run<SEGTOPK_KEY_F32>(k32, "f32");
    run<SEGTOPK_KEY_U32>(k32, "u32");
    run<SEGTOPK_KEY_I32>(k32, "i32");
    run<SEGTOPK_KEY_U16>(k16, "u16");
    run<SEGTOPK_KEY_I16>(k16, "i16");
    std::printf("total mismatches: %ld\n", g_bad);
    return g_bad != 0;
}
