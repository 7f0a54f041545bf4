/*
 * segtopk.h -- segmented (batched) top-k on AMD Instinct MI355X (gfx950).
 *
 * One call, batched_topk(), selects for every segment of a batch the k
 * largest (or smallest) keys, optionally carrying a 32-bit value payload.
 * Selection is multi-pass most-significant-digit radix selection: each pass
 * builds a digit histogram over the surviving candidates, scans it to find the
 * bucket that holds the k-th key, narrows k and the candidate set to that
 * bucket and folds the digit into a running splitter; a final filter writes
 * every key beyond the splitter plus exactly enough splitter-equal keys.
 *   [PR "Implement Segmented TopK using Thread-Block-Clusters", §1.2 Radix
 *    (digit) top-k, §1.4 Early stop, §1.5 Final filter and output placement]
 *
 * The request model (determinism x tie-break x output ordering, their valid
 * pairings and defaults) follows the CCCL page "Top-K: Determinism,
 * Tie-Breaking, and Output Ordering".
 *
 * All pointers passed to batched_topk() are DEVICE pointers except the two
 * descriptor structs themselves, which live in host memory and are read
 * during the call only.  The library never frees or retains caller memory.
 */
#ifndef SEGTOPK_H
#define SEGTOPK_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define SEGTOPK_OK 0
#define SEGTOPK_INVALID_ARGUMENT 1 /* bad pointer, enum, pairing or size      */
#define SEGTOPK_NOT_SUPPORTED 2    /* valid request this build does not serve */
#define SEGTOPK_HIP_ERROR 3        /* a HIP runtime call or launch failed     */
#define SEGTOPK_SCRATCH_TOO_SMALL 4 /* batched_topk_ex_noalloc: the request's
                                       plan needs more scratch than
                                       SEGTOPK_STATIC_SCRATCH_BYTES          */

/* ---- key types ------------------------------------------------------- */
/* Keys are compared by numeric value.  Floating-point keys: -0.0 and +0.0
 * compare equal (either may be selected; the selected key is written with its
 * own original bit pattern, so a selected -0.0 comes back as -0.0); +inf and
 * -inf are the largest and smallest values.  NaN keys are outside the
 * contract (they are ordered above +inf / below -inf by sign, but no result is
 * promised for them).
 *   [PR "Fix BlockTopK +/-0.0 handling", Description: Cause / Fix] */
typedef enum segtopk_key_type {
    SEGTOPK_KEY_F32 = 0,  /* IEEE binary32                          */
    SEGTOPK_KEY_BF16 = 1, /* bfloat16 (upper half of a binary32)    */
    SEGTOPK_KEY_U32 = 2,  /* unsigned 32-bit integer                */
    SEGTOPK_KEY_I32 = 3,  /* signed 32-bit integer                  */
    SEGTOPK_KEY_F16 = 4,  /* IEEE binary16                          */
    SEGTOPK_KEY_U16 = 5,  /* unsigned 16-bit integer                */
    SEGTOPK_KEY_I16 = 6,  /* signed 16-bit integer                  */
    SEGTOPK_KEY_U64 = 7,  /* unsigned 64-bit integer                */
    SEGTOPK_KEY_I64 = 8,  /* signed 64-bit integer                  */
    SEGTOPK_KEY_F64 = 9,  /* IEEE binary64                          */
    SEGTOPK_KEY_U8 = 10,  /* unsigned 8-bit integer                 */
    SEGTOPK_KEY_I8 = 11   /* signed 8-bit integer                   */
} segtopk_key_type;

/* ---- request --------------------------------------------------------- */
/* Which end: the MaxKeys/MaxPairs vs MinKeys/MinPairs entry points. */
typedef enum segtopk_direction { SEGTOPK_MAX = 0, SEGTOPK_MIN = 1 } segtopk_direction;

/* Determinism of the result SET (not of positions).
 *   [docs "Top-K: Determinism ...", "Determinism (cuda::execution::determinism)"] */
typedef enum segtopk_determinism {
    SEGTOPK_NOT_GUARANTEED = 0, /* ties at the boundary: any valid subset      */
    SEGTOPK_RUN_TO_RUN = 1,     /* same set on every run on this GPU          */
    SEGTOPK_GPU_TO_GPU = 2      /* same set on every GPU of this architecture */
} segtopk_determinism;

/* Which tied boundary keys win.  prefer_smaller_index / prefer_larger_index
 * are valid only together with SEGTOPK_GPU_TO_GPU; unspecified is valid with
 * every determinism level.  With a deterministic level and unspecified, this
 * library resolves ties toward the smaller index.
 *   [docs "Top-K: Determinism ...", "Tie-break" and "Which items are
 *    selected?" tables] */
typedef enum segtopk_tie_break {
    SEGTOPK_TIE_UNSPECIFIED = 0,
    SEGTOPK_PREFER_SMALLER_INDEX = 1,
    SEGTOPK_PREFER_LARGER_INDEX = 2
} segtopk_tie_break;

/* How the selected set is laid out in each output row.
 *   unsorted       any permutation of the set
 *   sorted         by key, best first (descending for MAX, ascending for MIN);
 *                  this library writes the stable order
 *   stable_sorted  by key, best first; equal keys by source index ascending
 *   [docs "Top-K: Determinism ...", "Output ordering" table] */
typedef enum segtopk_ordering {
    SEGTOPK_UNSORTED = 0,
    SEGTOPK_SORTED = 1,
    SEGTOPK_STABLE_SORTED = 2
} segtopk_ordering;

/* Largest k served with SEGTOPK_SORTED / SEGTOPK_STABLE_SORTED (the sort runs
 * on-chip); larger k with a sorted ordering returns SEGTOPK_NOT_SUPPORTED.
 * Unsorted output has no such limit. */
#define SEGTOPK_MAX_SORTED_K 4096

/* ---- buffers ---------------------------------------------------------- */
/* Keys: `in` holds offsets[num_segments] elements of `type` (device memory,
 * aligned to the element size); `out` receives num_segments * k elements,
 * row-major with a fixed row stride of k. */
typedef struct segtopk_keys {
    const void *in;
    void *out;
    int32_t type; /* a segtopk_key_type */
} segtopk_keys;

/* Values: any 32-bit payload aligned with keys.in (batched_topk_ex also takes
 * 64-bit payloads), copied bit for bit; `out` has the same num_segments x k
 * shape as the key output.  Pass NULL (or in == NULL) for a keys-only
 * request. */
typedef struct segtopk_values {
    const void *in;
    void *out;
} segtopk_values;

/*
 * batched_topk -- top-k of every segment.
 *
 *   keys             key descriptor (host struct, device buffers), required
 *   values           value descriptor or NULL for keys only
 *   segment_offsets  device array of num_segments + 1 int64 offsets; segment
 *                    i is keys.in[segment_offsets[i] .. segment_offsets[i+1]).
 *                    A negative size (end < begin) is an empty segment.  Each
 *                    segment must hold fewer than 2^31 keys; the total may
 *                    exceed 2^31.
 *   num_segments     number of segments, >= 0
 *   k                keys kept per segment and the output row stride,
 *                    0 <= k <= 2^31 - 1.  Segment i writes k_i = min(k, n_i)
 *                    items to row i; slots k_i .. k-1 are left untouched.
 *                    k at or above the segment size selects the whole segment.
 *   direction        segtopk_direction
 *   determinism      segtopk_determinism
 *   tie_break        segtopk_tie_break (see the pairing rule above)
 *   ordering         segtopk_ordering
 *   stream           HIP stream the work is queued on (NULL: default stream)
 *
 * The call is asynchronous: it validates the request, queues kernels on
 * `stream` and returns without waiting.  It never copies data to the host.
 * Internal scratch (only for batches of fewer than 2048 segments) is one
 * buffer per (device, stream), taken from a memory pool the library creates
 * for the device (the device's default pool is not touched) on `stream` the
 * first time a call on that stream needs it, and grown (the old buffer freed
 * on `stream`) when a later call needs more.  Calls on one stream reuse it in
 * stream order.  The library keeps such buffers for at most 16 (device,
 * stream) pairs; the least recently used one is freed, in stream order, when
 * a seventeenth pair needs one.  A stream handle that is destroyed and
 * created again may inherit the buffer of its predecessor, which is safe
 * because every call first waits for the buffer's previous use.
 * Outputs must not overlap the inputs.  Calls on different streams are
 * independent.
 *
 * Returns SEGTOPK_OK, or SEGTOPK_INVALID_ARGUMENT for a NULL required pointer,
 * an out-of-range enum, k or num_segments, values.in without values.out, or a
 * (determinism, tie_break) pair outside the five valid ones; no work is queued
 * then.  k == 0 or num_segments == 0 returns SEGTOPK_OK with no work.
 * Offsets that decrease other than as empty segments, or a segment of 2^31 or
 * more keys, are precondition violations with undefined results.
 */
int batched_topk(const segtopk_keys *keys, const segtopk_values *values,
                 const int64_t *segment_offsets, int64_t num_segments, int64_t k,
                 int direction, int determinism, int tie_break, int ordering,
                 hipStream_t stream);

/*
 * batched_topk_ex -- batched_topk with per-segment k, a segment-size hint and
 * 64-bit payloads.   [PR "Implement Segmented TopK using
 * Thread-Block-Clusters", the review comment asking for deferred (per-segment)
 * k and for k and num_segments to be validated beyond their wrapper form;
 * §3.4 Single-CTA path and the runtime collapse; the static segment-size
 * bounds of the tuning discussion]
 *
 *   value_bytes       size of one payload item: 4 or 8 (ignored for a
 *                     keys-only request).  values.in / values.out must be
 *                     aligned to it.
 *   k                 output row stride and the largest k of any segment,
 *                     0 <= k <= 2^31 - 1
 *   k_per_segment     NULL (every segment uses k), or a DEVICE array of
 *                     num_segments int32 counts, aligned to 4 bytes: segment i
 *                     keeps k_i = min(max(k_per_segment[i], 0), k, n_i) items.
 *                     Slots k_i .. k-1 of row i are left untouched.  Read on
 *                     the device, in stream order, so it may be written by
 *                     earlier work on `stream`.
 *   max_segment_size  host-side hint: no segment holds more keys than this;
 *                     <= 0 means unknown.  It only steers the launch plan
 *                     (whether segments are split over several workgroups,
 *                     scratch and stash sizes, and, at 4096 keys or fewer for
 *                     4-byte keys and 8192 or fewer for 2-byte keys, a kernel
 *                     built only for segments that fit one load per lane);
 *                     a segment larger than the hint is still served
 *                     correctly, at the cost of a less suited plan.
 *   the other arguments are batched_topk's.
 *
 * With value_bytes == 8 the selection writes each winner's source index into
 * its output slot and a second kernel on `stream` replaces it with the
 * payload; no scratch is taken for that.
 * Returns what batched_topk returns; value_bytes other than 4 or 8, or a
 * misaligned k_per_segment, is SEGTOPK_INVALID_ARGUMENT.
 *
 * batched_topk(keys, values, off, S, k, ...) is
 * batched_topk_ex(keys, values, 4, off, S, k, NULL, 0, ...).
 *
 * Graph capture: a request whose plan needs internal scratch (fewer than
 * 2048 segments, unless max_segment_size shows that no segment needs more
 * than one workgroup) returns SEGTOPK_NOT_SUPPORTED while `stream` is being
 * captured; the other plans queue only kernel launches and may be captured.
 */
int batched_topk_ex(const segtopk_keys *keys, const segtopk_values *values, int32_t value_bytes,
                    const int64_t *segment_offsets, int64_t num_segments, int64_t k,
                    const int32_t *k_per_segment, int64_t max_segment_size, int direction,
                    int determinism, int tie_break, int ordering, hipStream_t stream);

/*
 * batched_topk_ex_noalloc -- batched_topk_ex that allocates nothing.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * arguments, results and errors are batched_topk_ex's.  Instead of a
 * per-stream buffer from a memory pool, the scratch that plans for fewer than
 * 2048 segments use (the segment processing order; the per-segment histograms,
 * tickets and candidate slots when segments are split over workgroups) lives
 * in one file-scope device array of SEGTOPK_STATIC_SCRATCH_BYTES, which every
 * GPU the library runs on holds until the process ends.  The call makes no
 * hipMalloc / hipFree / pool call and no allocating library call; it queues
 * only kernels (a small fill kernel clears the words that must start at zero,
 * on every call that uses the array), so it may be captured into a graph.
 *
 * All calls on one device share that device's array and it keeps the last
 * call's contents: calls that can overlap on one device (on different
 * streams, or replays of graphs holding such calls) race and must be ordered
 * by the caller.  A request whose plan needs more than
 * SEGTOPK_STATIC_SCRATCH_BYTES returns SEGTOPK_SCRATCH_TOO_SMALL and queues
 * nothing (for instance 500 segments with k = 2048 of unknown sizes, split
 * two ways: about 41 MB of per-workgroup candidate slots; a max_segment_size
 * hint that rules out splitting avoids that scratch).  32 x 4 Mi keys with
 * k = 2048 (30.5 MiB) or one segment with k = 2048 (30.3 MiB) fit.
 */
#define SEGTOPK_STATIC_SCRATCH_BYTES (32u << 20)
int batched_topk_ex_noalloc(const segtopk_keys *keys, const segtopk_values *values,
                            int32_t value_bytes, const int64_t *segment_offsets,
                            int64_t num_segments, int64_t k, const int32_t *k_per_segment,
                            int64_t max_segment_size, int direction, int determinism,
                            int tie_break, int ordering, hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char *segtopk_status_string(int status);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int segtopk_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SEGTOPK_H */
