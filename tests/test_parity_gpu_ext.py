"""GPU-vs-oracle parity for the extended call (batched_topk_ex): per-segment k,
the segment-size hint, 8-byte payloads, 16-bit integer keys, and batches of
fewer than eight segments, whose workgroups spread over the whole device.

Rows are compared as in tests/parity.py (bitwise in the deterministic modes,
key multiset plus validity in not_guaranteed, untouched slots past k_i).
"""
import sys

import numpy as np
import pytest
import torch

from parity import check, check_all_rows

pytestmark = pytest.mark.gpu

DEV = "cuda"
MODES = [("not_guaranteed", "unspecified"), ("run_to_run", "unspecified"),
         ("gpu_to_gpu", "unspecified"), ("gpu_to_gpu", "prefer_smaller_index"),
         ("gpu_to_gpu", "prefer_larger_index")]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rand_keys(total, key_type, gen, levels=None):
    if key_type in ("f32", "bf16", "f16"):
        if levels:
            x = torch.randint(-levels, levels, (total,), generator=gen, device=DEV).float() / 4
        else:
            x = torch.randn(total, generator=gen, device=DEV) * 3
        return x.to({"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[key_type])
    if key_type in ("u16", "i16"):
        lo, hi = (-(2 ** 15), 2 ** 15) if not levels else (-levels, levels)
        return torch.randint(lo, hi, (total,), generator=gen, device=DEV,
                             dtype=torch.int32).to(torch.int16)
    lo, hi = (-(2 ** 31), 2 ** 31) if not levels else (-levels, levels)
    return torch.randint(lo, hi, (total,), generator=gen, device=DEV,
                         dtype=torch.int64).to(torch.int32)


def offsets_from(sizes, start=0):
    off = [start]
    for s_ in sizes:
        off.append(off[-1] + int(s_))
    return torch.tensor(off, dtype=torch.int64, device=DEV), max(off) + 3


# Plans: many segments (one workgroup each), a few hundred (one workgroup each,
# largest first), a few dozen long ones (several workgroups each).
PLANS = {
    "many": lambda rng: rng.choice([0, 1, 5, 64, 300, 1000, 4096, 5000, 20000], size=2100),
    "ordered": lambda rng: rng.integers(0, 30000, 300),
    "sliced": lambda rng: np.concatenate([rng.integers(100000, 400000, 12), [0, 7, 50, 2000]]),
}


@pytest.mark.parametrize("plan", list(PLANS))
@pytest.mark.parametrize("key_type", ["f32", "bf16"])
def test_per_segment_k(plan, key_type):
    rng = np.random.default_rng(101)
    sizes = PLANS[plan](rng)
    off, total = offsets_from(sizes, 3)
    S = len(sizes)
    g = torch.Generator(device=DEV)
    g.manual_seed(202)
    vals = torch.arange(total, dtype=torch.int32, device=DEV)
    k = 300
    kseg = rng.integers(-5, k + 50, S).astype(np.int32)
    kseg[:6] = [0, 1, k, k + 7, 2 ** 31 - 1, -2 ** 31]
    kseg_t = torch.from_numpy(kseg).to(DEV)
    say(f"[per-segment k {plan} {key_type}] segments={S} keys={total}")
    for levels in (None, 6):
        keys = rand_keys(total, key_type, g, levels)
        for largest in (True, False):
            for det, tb in (MODES if levels else [MODES[0], MODES[3]]):
                for ordering in ("unsorted", "stable_sorted"):
                    check(keys, vals, off, k, key_type, largest, det, tb, ordering,
                          values_are="position", k_per_segment=kseg_t)


@pytest.mark.parametrize("key_type", ["bf16", "f32"])
def test_slice_mode_repeated_calls_per_segment_k(key_type):
    """Back-to-back slice-mode calls on one stream reuse the scratch that each
    call leaves cleared (merged and shared histograms, tickets): repeated
    calls with per-segment k (including k_i = 0 and 1) must each match the
    oracle."""
    rng = np.random.default_rng(111)
    sizes = PLANS["sliced"](rng)
    off, total = offsets_from(sizes, 3)
    S = len(sizes)
    g = torch.Generator(device=DEV)
    g.manual_seed(212)
    vals = torch.arange(total, dtype=torch.int32, device=DEV)
    k = 300
    kseg = rng.integers(-5, k + 50, S).astype(np.int32)
    kseg[:6] = [0, 1, k, k + 7, 1, 2]
    kseg_t = torch.from_numpy(kseg).to(DEV)
    for rep in range(4):
        keys = rand_keys(total, key_type, g, None if rep % 2 == 0 else 6)
        say(f"[slice mode repeated {key_type}] call group {rep}")
        for largest in (True, False):
            for det, tb in (MODES[0], MODES[3], MODES[4]):
                check(keys, vals, off, k, key_type, largest, det, tb,
                      "stable_sorted" if rep < 2 else "unsorted", values_are="position",
                      k_per_segment=kseg_t)


@pytest.mark.parametrize("hint_kind", ["exact", "too_small", "huge"])
def test_max_segment_size_hint(hint_kind):
    """The hint only steers the plan: results are the same when it is exact,
    when a segment exceeds it, and when it is far too large."""
    rng = np.random.default_rng(7)
    cases = [
        (rng.integers(100, 4000, 64), 33),        # small segments, few
        (rng.integers(1000, 8000, 700), 100),     # small segments, a few hundred
        (rng.integers(50000, 300000, 10), 500),   # long segments, few
    ]
    g = torch.Generator(device=DEV)
    g.manual_seed(8)
    for sizes, k in cases:
        off, total = offsets_from(sizes)
        keys = rand_keys(total, "f32", g, 40)
        vals = torch.arange(total, dtype=torch.int32, device=DEV)
        mx = int(sizes.max())
        hint = {"exact": mx, "too_small": max(1, mx // 5), "huge": 2 ** 40}[hint_kind]
        say(f"[hint {hint_kind}] segments={len(sizes)} max={mx} hint={hint} k={k}")
        for largest in (True, False):
            for det, tb in (MODES[0], MODES[4]):
                check(keys, vals, off, k, "f32", largest, det, tb, "stable_sorted",
                      values_are="position", max_segment_size=hint)
                check(keys, vals, off, k, "f32", largest, det, tb, "unsorted",
                      values_are="position", max_segment_size=hint)


# Longest segment of the small-segment kernel (one load of four per lane in
# each of four waves), per key type.
SMALL = {"f32": 4096, "u32": 4096, "i32": 4096, "bf16": 8192, "f16": 8192, "u16": 8192,
         "i16": 8192}


@pytest.mark.parametrize("key_type", list(SMALL))
def test_small_segment_kernel(key_type):
    """A size hint within the small-segment limit selects the kernel with only
    the one-load path: ragged sizes up to the hint in every mode and ordering,
    tied levels (candidate lists past the stash), per-segment k, then
    segments longer than the hint (counted and re-read by the same kernel)."""
    lim = SMALL[key_type]
    k = 50
    sizes = [0, 1, 2, k - 1, k, k + 1, 3, 100, 257, 1000, lim // 2 + 1, lim - 1, lim, -5, 0,
             33, 5, lim - 64, 4000]
    off, total = offsets_from(sizes, 3)
    g = torch.Generator(device=DEV)
    g.manual_seed(303)
    vals = torch.arange(total, dtype=torch.int32, device=DEV)
    say(f"[small kernel {key_type}] segments={len(sizes)} hint={lim}")
    # levels=1: two values, so the k-th bucket overflows the stash and the
    # finish reads the segment again.
    for levels in (None, 3, 1):
        keys = rand_keys(total, key_type, g, levels)
        for largest in (True, False):
            for det, tb in MODES:
                for ordering in ("unsorted", "sorted", "stable_sorted"):
                    check(keys, vals, off, k, key_type, largest, det, tb, ordering,
                          values_are="position", max_segment_size=lim)
    rng = np.random.default_rng(304)
    kseg = torch.from_numpy(rng.integers(-2, k + 9, len(sizes)).astype(np.int32)).to(DEV)
    keys = rand_keys(total, key_type, g, 6)
    for det, tb in (MODES[0], MODES[3], MODES[4]):
        check(keys, vals, off, k, key_type, True, det, tb, "stable_sorted", values_are="position",
              k_per_segment=kseg, max_segment_size=lim)
    say(f"[small kernel {key_type}] segments longer than the hint")
    sizes = [lim + 1, 3 * lim + 17, 70000, 10, lim, 2 * lim]
    off, total = offsets_from(sizes, 1)
    vals = torch.arange(total, dtype=torch.int32, device=DEV)
    for levels in (None, 5):
        keys = rand_keys(total, key_type, g, levels)
        for det, tb in (MODES[0], MODES[1], MODES[3], MODES[4]):
            for ordering in ("unsorted", "stable_sorted"):
                check(keys, vals, off, k, key_type, levels is None, det, tb, ordering,
                      values_are="position", max_segment_size=lim)


@pytest.mark.parametrize("key_type", ["f32", "bf16"])
def test_small_segment_kernel_many_segments(key_type):
    """Thousands of segments under the small-segment hint, several k."""
    lim = SMALL[key_type]
    rng = np.random.default_rng(305)
    sizes = rng.choice([0, 1, 9, 64, 65, 300, 1000, lim // 2, lim - 1, lim, -2], size=3000)
    off, total = offsets_from(sizes, 7)
    g = torch.Generator(device=DEV)
    g.manual_seed(306)
    vals = torch.arange(total, dtype=torch.int32, device=DEV)
    for k in (1, 64, 256, 1000, 3000):
        for levels in (None, 8):
            keys = rand_keys(total, key_type, g, levels)
            say(f"[small kernel many {key_type}] k={k} levels={levels}")
            for det, tb in (MODES[0], MODES[3], MODES[4]):
                check(keys, vals, off, k, key_type, True, det, tb, "stable_sorted",
                      values_are="position", max_segment_size=lim)
                check(keys, vals, off, k, key_type, False, det, tb, "unsorted",
                      values_are="position", max_segment_size=lim)


@pytest.mark.parametrize("plan", list(PLANS))
def test_eight_byte_values(plan):
    rng = np.random.default_rng(55)
    sizes = PLANS[plan](rng)
    off, total = offsets_from(sizes, 1)
    g = torch.Generator(device=DEV)
    g.manual_seed(56)
    keys = rand_keys(total, "f32", g, 9)
    pos = torch.arange(total, dtype=torch.int64, device=DEV)
    tagged = pos | (torch.randint(1, 2 ** 31, (total,), generator=g, device=DEV,
                                  dtype=torch.int64) << 32)
    kseg = torch.from_numpy(rng.integers(0, 80, len(sizes)).astype(np.int32)).to(DEV)
    say(f"[8-byte values {plan}] segments={len(sizes)} keys={total}")
    for largest in (True, False):
        for det, tb in MODES[1:]:
            for ordering in ("unsorted", "stable_sorted"):
                check(keys, tagged, off, 64, "f32", largest, det, tb, ordering)
                check(keys, tagged, off, 64, "f32", largest, det, tb, ordering,
                      k_per_segment=kseg)
        # not_guaranteed checks each value against the key at that position.
        check(keys, pos, off, 64, "f32", largest, "not_guaranteed", "unspecified", "unsorted",
              values_are="position")


@pytest.mark.parametrize("key_type", ["u16", "i16"])
def test_sixteen_bit_integer_keys(key_type):
    rng = np.random.default_rng(71)
    sizes = [0, 1, 7, 33, 34, 100, 4095, 8192, 9000, 40000, -3, 70000, 5]
    off, total = offsets_from(sizes, 5)
    vals = torch.arange(total, dtype=torch.int32, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(72)
    pool = np.array([0, 1, 2, 0x7FFF, 0x8000, 0x8001, 0xFFFE, 0xFFFF], dtype=np.uint16)
    extreme = torch.from_numpy(rng.choice(pool, total).view(np.int16).copy()).to(DEV)
    for keys in (rand_keys(total, key_type, g), rand_keys(total, key_type, g, 5), extreme):
        for largest in (True, False):
            for det, tb in MODES:
                for ordering in ("unsorted", "stable_sorted"):
                    check(keys, vals, off, 33, key_type, largest, det, tb, ordering,
                          values_are="position")
    # many segments (one workgroup each) and a few long ones (several each)
    for sizes in (rng.integers(0, 9000, 2500), rng.integers(100000, 300000, 5)):
        off, total = offsets_from(sizes)
        keys = rand_keys(total, key_type, g, 300)
        vals = torch.arange(total, dtype=torch.int32, device=DEV)
        for det, tb in (MODES[0], MODES[4]):
            check(keys, vals, off, 200, key_type, True, det, tb, "unsorted",
                  values_are="position")


@pytest.mark.parametrize("S", [1, 2, 5, 7])
def test_few_segments_spread_over_the_device(S):
    """Fewer than eight segments: each segment's workgroups are dealt over
    every XCD and merge through device-wide atomics."""
    g = torch.Generator(device=DEV)
    g.manual_seed(300 + S)
    n = (1 << 24) // S
    keys = torch.randn(S * n, generator=g, device=DEV) * 10
    off = torch.arange(S + 1, dtype=torch.int64, device=DEV) * n
    vals = torch.arange(n, dtype=torch.int32, device=DEV).repeat(S)
    for det, tb in (MODES[0], MODES[3], MODES[4]):
        say(f"[spread S={S}] n={n} {det}/{tb}")
        check_all_rows(keys, vals, off, 2048, "f32", True, det, tb, "unsorted", chunk_rows=8)
    # heavy ties: quantised keys
    q = (torch.randint(0, 50, (S * n,), generator=g, device=DEV).float())
    for det, tb in (MODES[0], MODES[4]):
        check_all_rows(q, vals, off, 1000, "f32", False, det, tb, "unsorted", chunk_rows=8)


def _closed_form_check(keys_np, got_idx, got_bits, k, largest, det, tb):
    """One segment: the result set against the definition, computed with
    numpy instead of a sort of the whole segment.  s = the k-th best value;
    every key strictly better than s is selected, and k - #better keys equal
    to s, the smallest (prefer_smaller / unspecified deterministic) or largest
    (prefer_larger) indices among them; not_guaranteed: any of them."""
    n = keys_np.shape[0]
    vals = keys_np.astype(np.float64)
    kth = np.partition(-vals if largest else vals, k - 1)[k - 1]
    s = -kth if largest else kth
    better = np.nonzero(vals > s if largest else vals < s)[0]
    ties = np.nonzero(vals == s)[0]
    m = k - better.size
    assert 0 < m <= ties.size
    assert got_idx.size == k and np.unique(got_idx).size == k
    assert np.all(got_idx < n)
    assert np.array_equal(got_bits, keys_np.view(np.uint32)[got_idx])
    got = np.sort(got_idx)
    chosen_ties = np.setdiff1d(got, better, assume_unique=True)
    assert np.all(np.isin(better, got)), "a strictly better key is missing"
    assert chosen_ties.size == m and np.all(vals[chosen_ties] == s)
    if det != "not_guaranteed":
        want = ties[:m] if tb != "prefer_larger_index" else ties[-m:]
        assert np.array_equal(chosen_ties, want), "wrong ties chosen"


@pytest.mark.parametrize("det,tb", [MODES[0], MODES[3], MODES[4]])
def test_one_segment_of_2_28_keys(det, tb):
    """One segment of 2^28 float32 keys over the whole device, k = 2048."""
    n, k = 1 << 28, 2048
    g = torch.Generator(device=DEV)
    g.manual_seed(2028)
    keys = torch.randn(n, generator=g, device=DEV) * 10
    off = torch.tensor([0, n], dtype=torch.int64, device=DEV)
    vals = torch.arange(n, dtype=torch.int32, device=DEV)
    say(f"[one segment 2^28] {det}/{tb}")
    out_k = torch.empty((1, k), dtype=torch.float32, device=DEV)
    out_v = torch.empty((1, k), dtype=torch.int32, device=DEV)
    import segmented_top_selection_amd as st
    st.batched_topk(keys, off, k, values=vals, largest=True, determinism=det, tie_break=tb,
                    ordering="unsorted", out_keys=out_k, out_values=out_v)
    torch.cuda.synchronize()
    kn = keys.cpu().numpy()
    _closed_form_check(kn, out_v.cpu().numpy()[0].astype(np.int64),
                       out_k.cpu().numpy()[0].view(np.uint32), k, True, det, tb)
    # coarse keys: thousands of copies of the k-th value
    q = torch.randint(0, 1 << 16, (n,), generator=g, device=DEV).float()
    st.batched_topk(q, off, k, values=vals, largest=False, determinism=det, tie_break=tb,
                    ordering="unsorted", out_keys=out_k, out_values=out_v)
    torch.cuda.synchronize()
    _closed_form_check(q.cpu().numpy(), out_v.cpu().numpy()[0].astype(np.int64),
                       out_k.cpu().numpy()[0].view(np.uint32), k, False, det, tb)
    del keys, vals, q
    torch.cuda.empty_cache()


@pytest.mark.parametrize("det,tb", [MODES[0], MODES[4]])
def test_one_segment_wide_kth_bucket(det, tb):
    """One segment of 2^27 uniform uint32 keys, k = 2048: the k-th pass-0
    bucket holds about 65,536 keys, more than the staging area of a spread
    segment, so the last workgroup narrows it by reading the slots twice."""
    n, k = 1 << 27, 2048
    g = torch.Generator(device=DEV)
    g.manual_seed(2027)
    keys = torch.randint(-(2 ** 31), 2 ** 31, (n,), generator=g, device=DEV,
                         dtype=torch.int64).to(torch.int32)
    off = torch.tensor([0, n], dtype=torch.int64, device=DEV)
    vals = torch.arange(n, dtype=torch.int32, device=DEV)
    say(f"[one segment 2^27 u32] {det}/{tb}")
    out_k = torch.empty((1, k), dtype=torch.int32, device=DEV)
    out_v = torch.empty((1, k), dtype=torch.int32, device=DEV)
    import segmented_top_selection_amd as st
    st.batched_topk(keys, off, k, values=vals, largest=True, determinism=det, tie_break=tb,
                    ordering="unsorted", key_type="u32", out_keys=out_k, out_values=out_v)
    torch.cuda.synchronize()
    kn = keys.cpu().numpy().view(np.uint32)
    _closed_form_check(kn, out_v.cpu().numpy()[0].astype(np.int64),
                       out_k.cpu().numpy()[0].view(np.uint32), k, True, det, tb)
    del keys, vals
    torch.cuda.empty_cache()


def _keys64(total, key_type, gen, rng, kind):
    """64-bit keys: random full-width bits, a few tied levels, or extremes."""
    if kind == "random":
        if key_type == "f64":
            return torch.randn(total, generator=gen, device=DEV, dtype=torch.float64) * 1e3
        hi = torch.randint(-(2 ** 31), 2 ** 31, (total,), generator=gen, device=DEV, dtype=torch.int64)
        lo = torch.randint(0, 2 ** 32, (total,), generator=gen, device=DEV, dtype=torch.int64)
        return (hi << 32) | lo
    if kind == "levels":
        lv = torch.randint(-6, 7, (total,), generator=gen, device=DEV, dtype=torch.int64)
        return lv.double() / 4 if key_type == "f64" else lv * 3
    if key_type == "f64":
        pool = np.array([0.0, -0.0, 5e-324, -5e-324, 1.0, -1.0, np.inf, -np.inf,
                         1.7976931348623157e308, -1.7976931348623157e308])
        return torch.from_numpy(rng.choice(pool, total)).to(DEV)
    pool = np.array([0, 1, 2, 2 ** 62, 2 ** 63 - 1, -(2 ** 63), -(2 ** 63) + 1, -1, -2],
                    dtype=np.int64)
    return torch.from_numpy(rng.choice(pool, total)).to(DEV)


@pytest.mark.parametrize("key_type", ["u64", "i64", "f64"])
def test_sixty_four_bit_keys(key_type):
    rng = np.random.default_rng(91)
    g = torch.Generator(device=DEV)
    g.manual_seed(92)
    sizes = [0, 1, 7, 33, 34, 100, 2047, 2048, 2049, 5000, -3, 40000, 70000, 5]
    off, total = offsets_from(sizes, 5)
    vals = torch.arange(total, dtype=torch.int32, device=DEV)
    wide = torch.arange(total, dtype=torch.int64, device=DEV) | (7 << 40)
    for kind in ("random", "levels", "extreme"):
        keys = _keys64(total, key_type, g, rng, kind)
        say(f"[64-bit {key_type} {kind}] keys={total}")
        for largest in (True, False):
            for det, tb in MODES:
                for ordering in ("unsorted", "stable_sorted"):
                    check(keys, vals, off, 33, key_type, largest, det, tb, ordering,
                          values_are="position")
            check(keys, wide, off, 300, key_type, largest, "gpu_to_gpu", "prefer_larger_index",
                  "stable_sorted")
            check(keys, None, off, 40, key_type, largest, "gpu_to_gpu", "prefer_smaller_index",
                  "unsorted")
    # many segments; a few long ones (passes streamed from HBM until the
    # k-th bucket fits the candidate list); all-equal keys (index passes)
    for sizes, kind, k in ((rng.integers(0, 9000, 2100), "random", 64),
                           (rng.integers(200000, 500000, 4), "random", 1000),
                           ([300000, 5000, 70000], "levels", 2500)):
        off, total = offsets_from(sizes)
        keys = _keys64(total, key_type, g, rng, kind)
        vals = torch.arange(total, dtype=torch.int32, device=DEV)
        kseg = torch.from_numpy(rng.integers(0, k + 10, len(sizes)).astype(np.int32)).to(DEV)
        for det, tb in (MODES[0], MODES[3], MODES[4]):
            check(keys, vals, off, k, key_type, True, det, tb, "unsorted", values_are="position")
            check(keys, vals, off, k, key_type, False, det, tb, "unsorted",
                  values_are="position", k_per_segment=kseg)
        check(keys, vals, off, min(k, 4096), key_type, True, "gpu_to_gpu", "prefer_smaller_index",
              "stable_sorted", values_are="position")
    same = torch.full((100000,), 3, dtype=torch.int64, device=DEV)
    if key_type == "f64":
        same = same.double()
    off = torch.tensor([0, 100000], dtype=torch.int64, device=DEV)
    vals = torch.arange(100000, dtype=torch.int32, device=DEV)
    for tb in ("prefer_smaller_index", "prefer_larger_index"):
        check(same, vals, off, 3000, key_type, True, "gpu_to_gpu", tb, "stable_sorted")


@pytest.mark.parametrize("key_type", ["u8", "i8"])
def test_eight_bit_keys(key_type):
    """8-bit keys: every value repeats, so the index passes decide most rows."""
    rng = np.random.default_rng(81)
    g = torch.Generator(device=DEV)
    g.manual_seed(82)
    dt = torch.uint8 if key_type == "u8" else torch.int8

    def keys_of(total, kind):
        if kind == "random":
            return torch.randint(0, 256, (total,), generator=g, device=DEV).to(torch.uint8).view(dt)
        if kind == "few":
            return torch.randint(0, 3, (total,), generator=g, device=DEV).to(torch.uint8).view(dt)
        pool = np.array([0, 1, 127, 128, 254, 255], dtype=np.uint8)
        return torch.from_numpy(rng.choice(pool, total)).to(DEV).view(dt)

    sizes = [0, 1, 7, 33, 34, 100, 2047, 2048, 2049, 5000, -3, 40000, 70000, 5]
    off, total = offsets_from(sizes, 5)
    vals = torch.arange(total, dtype=torch.int32, device=DEV)
    for kind in ("random", "few", "extreme"):
        keys = keys_of(total, kind)
        say(f"[8-bit {key_type} {kind}] keys={total}")
        for largest in (True, False):
            for det, tb in MODES:
                for ordering in ("unsorted", "stable_sorted"):
                    check(keys, vals, off, 33, key_type, largest, det, tb, ordering,
                          values_are="position")
            check(keys, None, off, 500, key_type, largest, "gpu_to_gpu", "prefer_larger_index",
                  "stable_sorted")
    for sizes, k in ((rng.integers(0, 5000, 2100), 64), (rng.integers(100000, 300000, 3), 3000)):
        off, total = offsets_from(sizes)
        keys = keys_of(total, "random")
        vals = torch.arange(total, dtype=torch.int32, device=DEV)
        wide = torch.arange(total, dtype=torch.int64, device=DEV) | (5 << 33)
        kseg = torch.from_numpy(rng.integers(-1, k + 5, len(sizes)).astype(np.int32)).to(DEV)
        for det, tb in (MODES[0], MODES[3], MODES[4]):
            check(keys, vals, off, k, key_type, True, det, tb, "unsorted", values_are="position",
                  k_per_segment=kseg)
        check(keys, wide, off, k, key_type, False, "gpu_to_gpu", "prefer_smaller_index",
              "stable_sorted")
