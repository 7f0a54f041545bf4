/*
 * oracle.c -- plain, slow, obviously correct CPU reference for segmented
 * (batched) top-k.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * cpu_baseline leg of the benchmark may load this library.  The GPU library
 * shares no code, header, table or helper with it and never calls it.
 *
 * What it computes is the plain definition of the result; the radix digit
 * selection the GPU path runs reaches exactly this result:
 *
 *   For segment i let n_i = max(0, off[i+1] - off[i]) and k_i = min(k, n_i)
 *   (a negative size is an empty segment; k at or above the segment size
 *   selects the whole segment).
 *     [PR "Implement Segmented TopK using Thread-Block-Clusters", the request
 *      checklist (k == 0 / empty / negative sizes) and §6 "select-all"]
 *
 *   Order the items of the segment by
 *     1. the numeric key value, better first: larger for a MAX request,
 *        smaller for a MIN request.  IEEE comparison, so -0.0 == +0.0 and the
 *        infinities sit at the two ends;
 *          [PR "Fix BlockTopK +/-0.0 handling", Description / Cause]
 *     2. the source index inside the segment: ascending for
 *        prefer_smaller_index, descending for prefer_larger_index;
 *          [docs "Top-K: Determinism, Tie-Breaking, and Output Ordering",
 *           "Tie-break (cuda::execution::tie_break)" table;
 *           PR "Implement Segmented TopK ...", §1.6 Determinism / tie-breaking]
 *   and keep the first k_i items.  That is the result set: every key strictly
 *   better than the k_i-th key plus exactly enough keys equal to it, taken by
 *   the tie-break.
 *     [PR "Implement Segmented TopK ...", §1.2 Radix (digit) top-k and
 *      §1.5 Final filter and output placement]
 *
 *   The kept items are written in stable order: key better first, equal keys
 *   by source index ascending, whatever the tie-break.
 *     [docs "Top-K: Determinism ...", "Output ordering" table, stable_sorted,
 *      and the worked example, prefer_larger_index x stable_sorted row]
 *
 *   Row i of the outputs (fixed stride k) receives the k_i kept keys, with
 *   their original bit patterns (so -0.0 stays -0.0), and, when a value array
 *   is given, values[off[i] + index] for each kept item.  Slots k_i .. k-1 of
 *   the row are not written.
 *
 * NaN keys are outside the contract (the pages are silent on them); results
 * for NaN input are unspecified here and the tests never generate NaN.
 *
 * Key types (the caller's raw bit patterns):
 *   0 = binary32 float, 1 = bfloat16 (16 bits), 2 = uint32, 3 = int32,
 *   4 = binary16 float (16 bits), 5 = uint16, 6 = int16, 7 = uint64,
 *   8 = int64, 9 = binary64 float, 10 = uint8, 11 = int8.
 * Floating-point keys are compared as C doubles (every binary16, bfloat16,
 * binary32 and binary64 value is one exactly); integer keys are compared as
 * integers (int64_t, and uint64_t for uint64 keys, which a double cannot
 * hold exactly), so every comparison below is exact.
 *
 * Per-segment k (the extended entry point): when a k_per_segment array is
 * given, segment i keeps min(max(k_per_segment[i], 0), k, n_i) items, where k
 * stays the fixed row stride of the outputs.
 *   [PR "Implement Segmented TopK ...", the review comment on deferred /
 *    per-segment k, and §3.4 Single-CTA path and the runtime collapse]
 * Values are an opaque payload of 4 or 8 bytes per item, copied bit for bit.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_U32 = 2, OR_I32 = 3, OR_F16 = 4, OR_U16 = 5, OR_I16 = 6,
       OR_U64 = 7, OR_I64 = 8, OR_F64 = 9, OR_U8 = 10, OR_I8 = 11 };

/* One item of a segment.  The key is held exactly in one of three fields
 * (the other two are zero): f for floating-point keys, s for signed and
 * narrow unsigned integers, u for uint64.  dir is +1 for a MIN request and -1
 * for a MAX request, so that "ascending under dir" means "better first". */
typedef struct {
    double f;
    int64_t s;
    uint64_t u;
    int dir;
    int64_t tie;  /* index, negated for prefer_larger_index */
    int64_t idx;  /* source index inside the segment */
} item_t;

/* Decode one key to a double (exact for every supported type). */
static double decode_key(const void *keys, int type, int64_t pos)
{
    switch (type) {
    case OR_F32: {
        float f;
        memcpy(&f, (const char *)keys + 4 * pos, 4);
        return (double)f;
    }
    case OR_BF16: {
        /* bfloat16 is the upper half of a binary32 pattern. */
        uint16_t h;
        uint32_t w;
        float f;
        memcpy(&h, (const char *)keys + 2 * pos, 2);
        w = (uint32_t)h << 16;
        memcpy(&f, &w, 4);
        return (double)f;
    }
    case OR_U32: {
        uint32_t u;
        memcpy(&u, (const char *)keys + 4 * pos, 4);
        return (double)u;
    }
    case OR_I32: {
        int32_t s;
        memcpy(&s, (const char *)keys + 4 * pos, 4);
        return (double)s;
    }
    case OR_F16: {
        /* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
        uint16_t h;
        int sign, e, m;
        double mag;
        memcpy(&h, (const char *)keys + 2 * pos, 2);
        sign = h >> 15;
        e = (h >> 10) & 0x1f;
        m = h & 0x3ff;
        if (e == 0x1f)
            mag = m ? NAN : INFINITY;
        else if (e == 0)
            mag = ldexp((double)m, -24); /* subnormal: m * 2^-14 * 2^-10 */
        else
            mag = ldexp((double)(m | 0x400), e - 25); /* 1.m * 2^(e-15) */
        return sign ? -mag : mag;
    }
    case OR_F64: {
        double d;
        memcpy(&d, (const char *)keys + 8 * pos, 8);
        return d;
    }
    default:
        return NAN;
    }
}

static int is_float_type(int type)
{
    return type == OR_F32 || type == OR_BF16 || type == OR_F16 || type == OR_F64;
}

/* Integer keys other than uint64, widened exactly to int64_t. */
static int64_t decode_int(const void *keys, int type, int64_t pos)
{
    switch (type) {
    case OR_U32: {
        uint32_t u;
        memcpy(&u, (const char *)keys + 4 * pos, 4);
        return (int64_t)u;
    }
    case OR_I32: {
        int32_t v;
        memcpy(&v, (const char *)keys + 4 * pos, 4);
        return (int64_t)v;
    }
    case OR_U16: {
        uint16_t v;
        memcpy(&v, (const char *)keys + 2 * pos, 2);
        return (int64_t)v;
    }
    case OR_I16: {
        int16_t v;
        memcpy(&v, (const char *)keys + 2 * pos, 2);
        return (int64_t)v;
    }
    case OR_I64: {
        int64_t v;
        memcpy(&v, (const char *)keys + 8 * pos, 8);
        return v;
    }
    case OR_U8:
        return (int64_t)((const uint8_t *)keys)[pos];
    case OR_I8:
        return (int64_t)((const int8_t *)keys)[pos];
    default:
        return 0;
    }
}

static int key_bytes(int type)
{
    switch (type) {
    case OR_U8: case OR_I8: return 1;
    case OR_BF16: case OR_F16: case OR_U16: case OR_I16: return 2;
    case OR_U64: case OR_I64: case OR_F64: return 8;
    default: return 4;
    }
}

/* Key order under the request's direction: <0 when a is better than b. */
static int cmp_key(const item_t *a, const item_t *b)
{
    if (a->f != b->f) return (a->f < b->f ? -1 : 1) * a->dir;
    if (a->s != b->s) return (a->s < b->s ? -1 : 1) * a->dir;
    if (a->u != b->u) return (a->u < b->u ? -1 : 1) * a->dir;
    return 0;
}

/* Selection order: better key first, then the tie-break order of indices. */
static int cmp_select(const void *pa, const void *pb)
{
    const item_t *a = (const item_t *)pa, *b = (const item_t *)pb;
    int c = cmp_key(a, b);
    if (c) return c;
    if (a->tie < b->tie) return -1;
    if (a->tie > b->tie) return 1;
    return 0;
}

/* Output order (stable_sorted): better key first, then index ascending. */
static int cmp_output(const void *pa, const void *pb)
{
    const item_t *a = (const item_t *)pa, *b = (const item_t *)pb;
    int c = cmp_key(a, b);
    if (c) return c;
    if (a->idx < b->idx) return -1;
    if (a->idx > b->idx) return 1;
    return 0;
}

/* One segment: sort-and-take.  Returns 0, or -1 when memory runs out. */
static int one_segment(const void *keys_in, int type, const void *values_in, int value_bytes,
                       int64_t begin, int64_t n, int64_t k_i, int64_t stride, int largest,
                       int prefer_larger, void *keys_out, void *values_out, int64_t row)
{
    int64_t j;
    int kb = key_bytes(type);
    item_t *items;

    if (n <= 0 || k_i <= 0)
        return 0;
    if (k_i > n)
        k_i = n;
    items = (item_t *)malloc((size_t)n * sizeof(item_t));
    if (!items)
        return -1;
    for (j = 0; j < n; ++j) {
        items[j].f = 0.0;
        items[j].s = 0;
        items[j].u = 0;
        if (is_float_type(type))
            items[j].f = decode_key(keys_in, type, begin + j);
        else if (type == OR_U64)
            memcpy(&items[j].u, (const char *)keys_in + 8 * (begin + j), 8);
        else
            items[j].s = decode_int(keys_in, type, begin + j);
        items[j].dir = largest ? -1 : 1;
        items[j].tie = prefer_larger ? -j : j;
        items[j].idx = j;
    }
    /* The comparators are total orders (indices are unique), so the
     * instability of qsort cannot change the outcome. */
    qsort(items, (size_t)n, sizeof(item_t), cmp_select);
    qsort(items, (size_t)k_i, sizeof(item_t), cmp_output);
    for (j = 0; j < k_i; ++j) {
        int64_t src = begin + items[j].idx;
        int64_t dst = row * stride + j;
        memcpy((char *)keys_out + kb * dst, (const char *)keys_in + kb * src, (size_t)kb);
        if (values_in)
            memcpy((char *)values_out + (int64_t)value_bytes * dst,
                   (const char *)values_in + (int64_t)value_bytes * src, (size_t)value_bytes);
    }
    free(items);
    return 0;
}

/*
 * Batched top-k over num_segments segments.
 *   keys_in       raw key patterns, type `key_type` (see the list above)
 *   values_in     payload of value_bytes (4 or 8) per key, aligned with
 *                 keys_in, or NULL (keys only)
 *   offsets       num_segments + 1 int64 offsets into keys_in / values_in
 *   k             largest number of items kept per segment, and the fixed
 *                 row stride of the outputs
 *   k_per_segment NULL (every segment keeps up to k), or num_segments int32
 *                 counts, each clamped to [0, k]
 *   largest       1 = MAX request, 0 = MIN request
 *   prefer_larger 1 = ties at the boundary resolved toward larger indices
 *   keys_out      num_segments * k keys; values_out likewise (when values_in)
 *   num_threads   worker threads over segments (<= 0: the runtime default)
 * Returns 0 on success, 1 on a bad argument, 2 when memory runs out.
 */
int oracle_batched_topk_ex(const void *keys_in, int key_type, const void *values_in,
                           int value_bytes, const int64_t *offsets, int64_t num_segments,
                           int64_t k, const int32_t *k_per_segment, int largest,
                           int prefer_larger, void *keys_out, void *values_out,
                           int num_threads)
{
    int64_t i;
    int failed = 0;

    if (num_segments < 0 || k < 0 || key_type < OR_F32 || key_type > OR_I8)
        return 1;
    if (values_in && value_bytes != 4 && value_bytes != 8)
        return 1;
    if (num_segments == 0 || k == 0)
        return 0;
    if (!keys_in || !keys_out || !offsets || (values_in && !values_out))
        return 1;

#ifdef _OPENMP
    if (num_threads <= 0)
        num_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads) reduction(|| : failed)
#endif
    for (i = 0; i < num_segments; ++i) {
        int64_t begin = offsets[i];
        int64_t n = offsets[i + 1] - offsets[i];
        int64_t k_i = k;
        if (k_per_segment) {
            k_i = k_per_segment[i] < 0 ? 0 : (int64_t)k_per_segment[i];
            if (k_i > k)
                k_i = k;
        }
        if (one_segment(keys_in, key_type, values_in, value_bytes, begin, n, k_i, k, largest,
                        prefer_larger, keys_out, values_out, i) != 0)
            failed = 1;
    }
    (void)num_threads;
    return failed ? 2 : 0;
}

/* The same with one k for every segment and 32-bit values. */
int oracle_batched_topk(const void *keys_in, int key_type, const uint32_t *values_in,
                        const int64_t *offsets, int64_t num_segments, int64_t k,
                        int largest, int prefer_larger, void *keys_out, uint32_t *values_out,
                        int num_threads)
{
    return oracle_batched_topk_ex(keys_in, key_type, values_in, 4, offsets, num_segments, k,
                                  NULL, largest, prefer_larger, keys_out, values_out,
                                  num_threads);
}

/* Threads the runtime would use by default (reported next to timings). */
int oracle_default_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
