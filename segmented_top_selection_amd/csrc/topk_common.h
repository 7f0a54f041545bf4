// topk_common.h -- what the host code of libsegtopk and its per-key-type
// kernel translation units share: launch constants, the kernel argument block
// and the two entry points every key type provides.
#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "segtopk.h"

namespace segtopk_impl {

constexpr int kWave = 64;               // wave64
constexpr int kWaves = 4;               // waves per workgroup
constexpr int kThreads = kWave * kWaves;
constexpr int kDigit = 11;              // digit width of pass 0 over the keys
constexpr int kBuckets = 1 << kDigit;   // 2048 histogram buckets
constexpr int kLaterDigit = 8;          // digit width of the passes over the candidates
constexpr uint32_t kBlockFinishMin = 512;  // longer candidate lists are finished by all four waves
constexpr uint32_t kNone = 0xFFFFFFFFu; // "no element" / sort padding
constexpr int kSplitU = 8;               // loads per lane per chunk when segments are split
constexpr int kSmallWaves32 = 8;        // waves per SIMD of the small-segment kernel, 32-bit keys
constexpr int kSmallWaves16 = 6;        // and 16-bit keys
// Longest segment of the small-segment kernel: one load of four per lane in
// each of the four waves (16 bytes a load).
constexpr uint32_t kSmallKeys32 = 4096;
constexpr uint32_t kSmallKeys16 = 8192;
constexpr size_t kMaxDynLds = 120 * 1024;
constexpr uint32_t kMaxWgPerSeg = 1024;  // slices of one segment (the last arriver's prefix table fits LDS)
// 16-bit keys with one workgroup per segment: per wave, a ring of this many
// 16-byte loads (and their element indices) waiting to be tested key by key.
constexpr uint32_t kRingLoads = 128;
constexpr size_t kRingBytes = 4 * kRingLoads * (16 + 4);  // four waves
// A segment spread over every XCD: room for this many entries of its k-th
// bucket, copied in a row by the last workgroup when it narrows the bucket.
constexpr uint32_t kStageCap = 32768;

// ---------------------------------------------------------------------------
// Kernel arguments.
// ---------------------------------------------------------------------------
struct Params {
    const void *keys_in;
    void *keys_out;
    const uint32_t *vals_in;  // nullptr: keys only
    uint32_t *vals_out;
    const int64_t *offsets;
    int64_t num_segments;
    const int32_t *kseg;     // [segments] per-segment k (clamped to [0, k]), or nullptr
    uint32_t k;              // output row stride and largest k
    uint32_t det;            // deterministic tie-break requested
    uint32_t prefer_larger;  // ties toward larger source indices
    uint32_t sorted;         // sorted or stable_sorted output
    uint32_t stash_cap;      // LDS stash entries per workgroup (four equal wave regions)
    uint32_t out_cap;        // LDS output staging entries (power of two), 0 = none
    uint32_t wg_per_seg;     // workgroups per segment (1: one workgroup each)
    uint32_t min_slice;      // smallest slice a segment is split into
    uint32_t *ws_hist;       // [segments][kBuckets]    merged pass-0 histograms
    uint32_t *ws_early;      // [segments][1 or 8][kBuckets] shared histograms (bound sharing)
    uint32_t *ws_ticket;     // [segments]              arrival tickets
    uint32_t *ws_slot_info;  // [segments][P][4]        (count, overflowed, bound, -)
    uint32_t *ws_slot_cum;   // [segments][P][kBuckets] entries with rank <= r
    uint2 *ws_slot_data;     // [segments][P][stash_cap] candidates sorted by rank
    uint2 *ws_stage;         // [segments][kStageCap] bucket b*'s entries in a row (spread plans), or nullptr
    const uint32_t *order;   // [segments] processing order (one workgroup each), or nullptr
    uint32_t spread;         // workgroup b serves segment b / P, slice b % P (small batches)
    uint32_t vindex;         // write the source index as the value (no gather)
    uint32_t vshift;         // value slot o is vals_out[o << vshift] (1: 8-byte slots)
    uint32_t pad_;
};

// Kernel variants: one workgroup per segment for many segments (4 loads per
// lane); the plan for fewer segments (8 loads per lane) with one workgroup
// per segment; and the same with several workgroups per segment (slices).
constexpr int kVariantOne = 0;
constexpr int kVariantSplit = 1;
constexpr int kVariantSliced = 2;
constexpr int kVariantSmall = 3;

// Launches the top-k kernel for key type KT on `st`: grid workgroups of
// kThreads threads with `lds` bytes of dynamic LDS, in the given variant.
template <int KT>
hipError_t launch_topk(const Params &p, bool largest, int variant, uint32_t grid, size_t lds,
                       hipStream_t st);

// Workgroups of the split variant of that kernel that fit on one CU of the
// current device with `lds` bytes of dynamic LDS (at least 1).
template <int KT> int topk_per_cu(bool largest, size_t lds);

// Launches the plain kernel (64-bit and 8-bit keys) for key type KT: one
// workgroup per segment, grid workgroups, `lds` bytes of dynamic LDS.
template <int KT>
hipError_t launch_topk_plain(const Params &p, bool largest, uint32_t grid, size_t lds,
                             hipStream_t st);

}  // namespace segtopk_impl
