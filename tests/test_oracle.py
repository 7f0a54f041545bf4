"""Pins for the CPU oracle.  None of these checks reuses the oracle's own code
path: they compare it with values printed on the pages, with a brute-force
search over subsets (a different algorithm), with library sorts, and with
invariants that the definition of top-k fixes.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def as_keys(vals, key_type):
    """Numeric values -> raw key array of the given type (exact for the inputs used)."""
    v = np.asarray(vals, dtype=np.float64)
    if key_type == "f32":
        return v.astype(np.float32)
    if key_type == "bf16":
        return (torch.tensor(v, dtype=torch.float64).to(torch.bfloat16)
                .view(torch.int16).numpy().view(np.uint16))
    if key_type == "f16":
        return v.astype(np.float16).view(np.uint16)
    if key_type == "u32":
        return v.astype(np.uint64).astype(np.uint32)
    if key_type == "i32":
        return v.astype(np.int64).astype(np.int32)
    raise ValueError(key_type)


def numeric(keys, key_type):
    """Raw key array -> float64 values, decoded by numpy / torch (not by the oracle)."""
    if key_type == "f32":
        return np.asarray(keys).view(np.float32).astype(np.float64)
    if key_type == "bf16":
        return torch.from_numpy(np.asarray(keys).view(np.int16).copy()).view(
            torch.bfloat16).to(torch.float64).numpy()
    if key_type == "f16":
        return np.asarray(keys).view(np.float16).astype(np.float64)
    if key_type == "u32":
        return np.asarray(keys).view(np.uint32).astype(np.float64)
    if key_type == "i32":
        return np.asarray(keys).view(np.int32).astype(np.float64)
    raise ValueError(key_type)


ALL_TYPES = ["f32", "bf16", "f16", "u32", "i32"]


# --------------------------------------------------------------------------
# 1. The worked example printed on the requirements page.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("key_type", ALL_TYPES)
def test_worked_example(key_type):
    with open(os.path.join(GOLDEN, "worked_example_max_k3.json")) as f:
        g = json.load(f)
    keys = as_keys(g["keys"], key_type)
    vals = np.arange(len(keys), dtype=np.uint32)
    off = np.array([0, len(keys)], dtype=np.int64)
    k = g["k"]
    for case, larger in (("gpu_to_gpu/prefer_smaller_index", False),
                         ("gpu_to_gpu/prefer_larger_index", True)):
        ok, ov = oracle.batched_topk(keys, off, k, key_type=key_type, values=vals,
                                     largest=True, prefer_larger=larger)
        got = [[float(numeric(ok[0, j:j + 1], key_type)[0]), int(ov[0, j])] for j in range(k)]
        want = g["cases"][case]["stable_sorted"]
        assert got == [[float(a), b] for a, b in want], case
        assert sorted(map(tuple, got)) == sorted((float(a), b) for a, b in g["cases"][case]["set"])
    # not_guaranteed: any valid choice; the oracle's must be one of them.
    ok, ov = oracle.batched_topk(keys, off, k, key_type=key_type, values=vals, largest=True)
    ng = g["cases"]["not_guaranteed/unspecified"]
    got = {(float(numeric(ok[0, j:j + 1], key_type)[0]), int(ov[0, j])) for j in range(k)}
    must = {(float(a), b) for a, b in ng["must_contain"]}
    pool = {(float(a), b) for a, b in ng["choose_from"]}
    assert must <= got and len(got - must) == ng["choose_count"] and (got - must) <= pool


# --------------------------------------------------------------------------
# 2. Brute force over all k-subsets on tiny segments (a different algorithm).
# --------------------------------------------------------------------------
ALPHABET = {
    "f32": [float("-inf"), -1.5, -0.0, 0.0, 1.5, 2.0, float("inf")],
    "bf16": [float("-inf"), -1.5, -0.0, 0.0, 1.5, 2.0, float("inf")],
    "f16": [float("-inf"), -1.5, -0.0, 0.0, 1.5, 2.0, float("inf")],
    "u32": [0, 1, 2, 2 ** 31, 2 ** 32 - 2, 2 ** 32 - 1],
    "i32": [-(2 ** 31), -1, 0, 1, 2 ** 31 - 1],
}


def brute_force(vals, k, largest, prefer_larger):
    """Set of indices chosen by exhaustive search: among all k-subsets whose
    every member is at least as good as every non-member, the one whose
    ascending index tuple is lexicographically smallest (prefer_smaller) or
    largest (prefer_larger)."""
    n = len(vals)
    kk = min(k, n)
    best = None
    for sub in itertools.combinations(range(n), kk):
        inside = [vals[i] for i in sub]
        outside = [vals[i] for i in range(n) if i not in sub]
        if inside and outside:
            if largest and min(inside) < max(outside):
                continue
            if not largest and max(inside) > min(outside):
                continue
        if best is None or (sub > best if prefer_larger else sub < best):
            best = sub
    return best


@pytest.mark.parametrize("key_type", ALL_TYPES)
def test_brute_force_tiny(key_type):
    rng = np.random.default_rng(7)
    alpha = ALPHABET[key_type]
    for trial in range(60):
        n = int(rng.integers(1, 9))
        vals = [alpha[i] for i in rng.integers(0, len(alpha), n)]
        keys = as_keys(vals, key_type)
        num = numeric(keys, key_type)
        payload = rng.permutation(1000)[:n].astype(np.uint32)
        # Put the segment behind a non-zero first offset.
        pad = int(rng.integers(0, 3))
        keys_full = np.concatenate([as_keys([alpha[0]] * pad, key_type), keys])
        pay_full = np.concatenate([np.full(pad, 7777, np.uint32), payload])
        off = np.array([pad, pad + n], dtype=np.int64)
        for k in range(0, n + 2):
            for largest in (True, False):
                for pl in (False, True):
                    canary_k = as_keys([alpha[0]] * max(k, 1), key_type)[None, :k].copy()
                    ok, ov = oracle.batched_topk(keys_full, off, k, key_type=key_type,
                                                 values=pay_full, largest=largest,
                                                 prefer_larger=pl,
                                                 out_keys=canary_k if k else None,
                                                 out_values=np.full((1, k), 0xDEAD, np.uint32))
                    if k == 0:
                        continue
                    want = brute_force(list(num), k, largest, pl)
                    kk = len(want)
                    # Map payload back to indices (payload values are unique).
                    got_idx = sorted(int(np.nonzero(payload == p)[0][0]) for p in ov[0, :kk])
                    assert tuple(got_idx) == want, (vals, k, largest, pl)
                    # Keys written with their own bit patterns.
                    for j in range(kk):
                        i = int(np.nonzero(payload == ov[0, j])[0][0])
                        assert ok[0, j].tobytes() == keys[i].tobytes()
                    # Stable order: better first, equal keys by index ascending.
                    outv = [num[int(np.nonzero(payload == p)[0][0])] for p in ov[0, :kk]]
                    outi = [int(np.nonzero(payload == p)[0][0]) for p in ov[0, :kk]]
                    for j in range(kk - 1):
                        a, b = outv[j], outv[j + 1]
                        assert (a > b or a == b) if largest else (a < b or a == b)
                        if a == b:
                            assert outi[j] < outi[j + 1]
                    # Untouched tail.
                    assert np.all(ov[0, kk:] == 0xDEAD)


# --------------------------------------------------------------------------
# 3. numpy's sort routines on larger random segments.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("key_type", ALL_TYPES)
@pytest.mark.parametrize("largest", [True, False])
@pytest.mark.parametrize("prefer_larger", [False, True])
def test_against_numpy_lexsort(key_type, largest, prefer_larger):
    rng = np.random.default_rng(11)
    sizes = rng.integers(-3, 700, 40)
    sizes[3] = 0
    begin = np.zeros(41, dtype=np.int64)
    ends = np.zeros(41, dtype=np.int64)
    # Offsets with a few negative-size (empty) segments.
    off = [5]
    for s in sizes:
        off.append(off[-1] + int(s))
    off = np.array(off, dtype=np.int64)
    total = int(off.max()) + 10
    if key_type in ("f32", "bf16", "f16"):
        levels = rng.integers(-20, 20, total) / 4.0
        levels[rng.random(total) < 0.05] = -0.0
        levels[rng.random(total) < 0.02] = np.inf
        levels[rng.random(total) < 0.02] = -np.inf
    elif key_type == "u32":
        levels = rng.integers(0, 2 ** 32, total).astype(np.float64)
        levels[rng.random(total) < 0.3] = 12345
    else:
        levels = rng.integers(-(2 ** 31), 2 ** 31, total).astype(np.float64)
        levels[rng.random(total) < 0.3] = -5
    keys = as_keys(levels, key_type)
    num = numeric(keys, key_type)
    payload = rng.integers(0, 2 ** 32, total, dtype=np.uint64).astype(np.uint32)
    k = 37
    ok, ov = oracle.batched_topk(keys, off, k, key_type=key_type, values=payload,
                                 largest=largest, prefer_larger=prefer_larger,
                                 out_values=np.full((40, k), 0xABCD, np.uint32))
    for i in range(40):
        b, e = int(off[i]), int(off[i + 1])
        n = max(0, e - b)
        kk = min(k, n)
        if kk == 0:
            assert np.all(ov[i] == 0xABCD)
            continue
        seg = num[b:b + n]
        idx = np.arange(n)
        primary = -seg if largest else seg
        secondary = -idx if prefer_larger else idx
        order = np.lexsort((secondary, primary))
        chosen = order[:kk]
        # stable output order of the chosen set
        out_order = chosen[np.lexsort((chosen, primary[chosen]))]
        assert np.array_equal(ov[i, :kk], payload[b + out_order])
        assert ok[i, :kk].tobytes() == keys[b + out_order].tobytes()
        assert np.all(ov[i, kk:] == 0xABCD)


# --------------------------------------------------------------------------
# 4. Invariants and special cases fixed by the definition.
# --------------------------------------------------------------------------
def test_select_all_when_k_at_least_n():
    keys = np.array([3, 1, 2, 1], dtype=np.float32)
    off = np.array([0, 4], dtype=np.int64)
    for k in (4, 9):
        ok, ov = oracle.batched_topk(keys, off, k, values=np.arange(4, dtype=np.uint32))
        assert list(ov[0, :4]) == [0, 2, 1, 3]
        ok, ov = oracle.batched_topk(keys, off, k, values=np.arange(4, dtype=np.uint32),
                                     largest=False)
        assert list(ov[0, :4]) == [1, 3, 2, 0]


def test_k_zero_and_empty_segments_write_nothing():
    keys = np.arange(10, dtype=np.float32)
    off = np.array([0, 0, 4, 2, 10], dtype=np.int64)  # empty, 4, negative, 8
    canary = np.full((4, 3), 99, np.uint32)
    ok, ov = oracle.batched_topk(keys, off, 3, values=np.arange(10, dtype=np.uint32),
                                 out_values=canary.copy())
    assert list(ov[0]) == [99, 99, 99]
    assert list(ov[1]) == [3, 2, 1]
    assert list(ov[2]) == [99, 99, 99]
    assert list(ov[3]) == [9, 8, 7]
    ok, ov = oracle.batched_topk(keys, off, 0, values=np.arange(10, dtype=np.uint32))
    assert ov.shape == (4, 0)


@pytest.mark.parametrize("prefer_larger", [False, True])
def test_all_equal_keys_take_index_extremes(prefer_larger):
    n, k = 50, 7
    keys = np.full(n, 0.5, np.float32)
    off = np.array([0, n], dtype=np.int64)
    for largest in (True, False):
        _, ov = oracle.batched_topk(keys, off, k, values=np.arange(n, dtype=np.uint32),
                                    largest=largest, prefer_larger=prefer_larger)
        want = list(range(n - k, n)) if prefer_larger else list(range(k))
        assert list(ov[0]) == want  # stable order: index ascending


def test_negative_zero_kept_bitwise():
    keys = np.array([-0.0, 0.0, -1.0, -0.0], dtype=np.float32)
    off = np.array([0, 4], dtype=np.int64)
    ok, ov = oracle.batched_topk(keys, off, 1, values=np.arange(4, dtype=np.uint32))
    assert ov[0, 0] == 0 and f32_bits(ok[0, 0]) == 0x80000000
    ok, ov = oracle.batched_topk(keys, off, 1, values=np.arange(4, dtype=np.uint32),
                                 prefer_larger=True)
    assert ov[0, 0] == 3 and f32_bits(ok[0, 0]) == 0x80000000
    ok, ov = oracle.batched_topk(keys, off, 3, values=np.arange(4, dtype=np.uint32))
    assert list(ov[0]) == [0, 1, 3]
    assert [int(b) for b in f32_bits(ok[0])] == [0x80000000, 0, 0x80000000]
    ok, ov = oracle.batched_topk(keys, off, 2, values=np.arange(4, dtype=np.uint32),
                                 largest=False)
    assert list(ov[0]) == [2, 0]


def test_infinities_are_the_ends():
    keys = np.array([np.inf, 1e38, -np.inf, -1e38, np.inf], dtype=np.float32)
    off = np.array([0, 5], dtype=np.int64)
    _, ov = oracle.batched_topk(keys, off, 3, values=np.arange(5, dtype=np.uint32))
    assert list(ov[0]) == [0, 4, 1]
    _, ov = oracle.batched_topk(keys, off, 2, values=np.arange(5, dtype=np.uint32),
                                largest=False)
    assert list(ov[0]) == [2, 3]


@pytest.mark.parametrize("key_type", ["bf16", "f16"])
def test_every_16bit_pattern_in_order(key_type):
    """All 2^16 patterns minus NaNs, select-all + stable order, against the
    ordering of numpy / torch decoded values."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    num = numeric(pats, key_type)
    pats = pats[~np.isnan(num)]
    num = num[~np.isnan(num)]
    n = len(pats)
    off = np.array([0, n], dtype=np.int64)
    for largest in (True, False):
        ok, ov = oracle.batched_topk(pats, off, n, key_type=key_type,
                                     values=np.arange(n, dtype=np.uint32), largest=largest)
        primary = -num if largest else num
        want = np.lexsort((np.arange(n), primary))
        assert np.array_equal(ov[0], want.astype(np.uint32))


def test_front_tie_decomposition_random():
    rng = np.random.default_rng(5)
    n, k = 3000, 100
    keys = (rng.integers(0, 40, n) / 8.0).astype(np.float32)
    off = np.array([0, n], dtype=np.int64)
    for largest in (True, False):
        ok, ov = oracle.batched_topk(keys, off, k, values=np.arange(n, dtype=np.uint32),
                                     largest=largest)
        s = ok[0, k - 1]  # k-th best value (stable order: last one)
        front = np.sum(keys > s) if largest else np.sum(keys < s)
        ties = np.sum(keys == s)
        assert front < k <= front + ties
        sel = set(int(v) for v in ov[0])
        rest = [i for i in range(n) if i not in sel]
        worst_in = min(keys[list(sel)]) if largest else max(keys[list(sel)])
        best_out = max(keys[rest]) if largest else min(keys[rest])
        assert (worst_in >= best_out) if largest else (worst_in <= best_out)
        # ties taken toward smaller indices
        tie_sel = sorted(i for i in sel if keys[i] == s)
        tie_all = [i for i in range(n) if keys[i] == s]
        assert tie_sel == tie_all[:len(tie_sel)]


def test_rejects_bad_arguments():
    lib = oracle._load()
    keys = np.zeros(4, np.float32)
    off = np.array([0, 4], dtype=np.int64)
    out = np.zeros(4, np.float32)
    args = lambda k, s, t: (keys.ctypes.data, t, None, off.ctypes.data, s, k, 1, 0,
                            out.ctypes.data, None, 1)
    assert lib.oracle_batched_topk(*args(-1, 1, 0)) == 1
    assert lib.oracle_batched_topk(*args(1, -1, 0)) == 1
    assert lib.oracle_batched_topk(*args(1, 1, 12)) == 1
    assert lib.oracle_batched_topk(*args(1, 1, -1)) == 1
    assert lib.oracle_batched_topk(*args(1, 1, 0)) == 0


# --------------------------------------------------------------------------
# 5. More key types (uint16, int16, uint64, int64, float64), per-segment k and
#    8-byte values.  Integer keys are checked with Python integers (exact at
#    any width), floats with numpy float64; neither goes through the oracle.
# --------------------------------------------------------------------------
WIDE_NUMPY = {"u16": np.uint16, "i16": np.int16, "u64": np.uint64, "i64": np.int64,
              "f64": np.float64, "u8": np.uint8, "i8": np.int8}
WIDE_ALPHABET = {
    "u16": [0, 1, 2, 2 ** 15, 2 ** 16 - 2, 2 ** 16 - 1],
    "i16": [-(2 ** 15), -1, 0, 1, 2 ** 15 - 1],
    # neighbours a double cannot tell apart
    "u64": [0, 1, 2 ** 53 + 1, 2 ** 63, 2 ** 63 + 1, 2 ** 64 - 2, 2 ** 64 - 1],
    "i64": [-(2 ** 63), -(2 ** 63) + 1, -1, 0, 2 ** 53 + 1, 2 ** 63 - 2, 2 ** 63 - 1],
    "f64": [float("-inf"), -1.5, -0.0, 0.0, 5e-324, 1.5, float("inf")],
    "u8": [0, 1, 2, 127, 128, 254, 255],
    "i8": [-128, -127, -1, 0, 1, 126, 127],
}


def wide_keys(vals, key_type):
    if key_type == "f64":
        return np.asarray(vals, dtype=np.float64)
    return np.array([int(v) for v in vals], dtype=WIDE_NUMPY[key_type])


def wide_exact(keys, key_type):
    """Raw keys -> exact Python numbers (ints, or floats for f64)."""
    if key_type == "f64":
        return [float(x) for x in keys]
    return [int(x) for x in keys]


@pytest.mark.parametrize("key_type", list(WIDE_ALPHABET))
def test_brute_force_tiny_wide_types(key_type):
    rng = np.random.default_rng(17)
    alpha = WIDE_ALPHABET[key_type]
    for trial in range(50):
        n = int(rng.integers(1, 9))
        vals = [alpha[i] for i in rng.integers(0, len(alpha), n)]
        keys = wide_keys(vals, key_type)
        exact = wide_exact(keys, key_type)
        payload = (rng.permutation(1000)[:n].astype(np.uint64) << np.uint64(32)) | np.uint64(7)
        off = np.array([0, n], dtype=np.int64)
        for k in range(1, n + 2):
            for largest in (True, False):
                for pl in (False, True):
                    ok, ov = oracle.batched_topk(keys, off, k, key_type=key_type,
                                                 values=payload, largest=largest,
                                                 prefer_larger=pl)
                    want = brute_force(exact, k, largest, pl)
                    kk = len(want)
                    got_idx = sorted(int(np.nonzero(payload == p)[0][0]) for p in ov[0, :kk])
                    assert tuple(got_idx) == want, (vals, k, largest, pl)
                    for j in range(kk):
                        i = int(np.nonzero(payload == ov[0, j])[0][0])
                        assert ok[0, j].tobytes() == keys[i].tobytes()


def test_u64_and_i64_neighbours_are_ordered_exactly():
    # 2^64-1 > 2^64-2 and 2^63+1 > 2^63 although each pair is one double.
    keys = np.array([2 ** 64 - 2, 2 ** 63, 2 ** 64 - 1, 2 ** 63 + 1], dtype=np.uint64)
    off = np.array([0, 4], dtype=np.int64)
    idx = np.arange(4, dtype=np.uint32)
    _, ov = oracle.batched_topk(keys, off, 4, key_type="u64", values=idx, largest=True)
    assert list(ov[0]) == [2, 0, 3, 1]
    _, ov = oracle.batched_topk(keys, off, 1, key_type="u64", values=idx, largest=False)
    assert list(ov[0]) == [1]
    keys = np.array([2 ** 63 - 2, -(2 ** 63) + 1, 2 ** 63 - 1, -(2 ** 63)], dtype=np.int64)
    _, ov = oracle.batched_topk(keys, off, 4, key_type="i64", values=idx, largest=True)
    assert list(ov[0]) == [2, 0, 1, 3]
    _, ov = oracle.batched_topk(keys, off, 2, key_type="i64", values=idx, largest=False,
                                prefer_larger=True)
    assert list(ov[0]) == [3, 1]


def test_f64_signed_zero_denormal_and_infinities():
    keys = np.array([-0.0, 5e-324, 0.0, -5e-324, np.inf, -np.inf], dtype=np.float64)
    off = np.array([0, 6], dtype=np.int64)
    idx = np.arange(6, dtype=np.uint32)
    ok, ov = oracle.batched_topk(keys, off, 6, key_type="f64", values=idx, largest=True)
    assert list(ov[0]) == [4, 1, 0, 2, 3, 5]
    assert ok[0, 2].tobytes() == np.float64(-0.0).tobytes()
    _, ov = oracle.batched_topk(keys, off, 2, key_type="f64", values=idx, largest=True,
                                prefer_larger=True)
    assert list(ov[0]) == [4, 1]


def _python_topk(exact, k, largest, prefer_larger):
    """Indices of the top-k by Python's sort on exact numbers, in stable order."""
    n = len(exact)
    order = sorted(range(n), key=lambda i: ((-exact[i]) if largest else exact[i],
                                            -i if prefer_larger else i))
    chosen = order[:min(k, n)]
    return sorted(chosen, key=lambda i: ((-exact[i]) if largest else exact[i], i))


@pytest.mark.parametrize("key_type", list(WIDE_ALPHABET))
@pytest.mark.parametrize("largest", [True, False])
@pytest.mark.parametrize("prefer_larger", [False, True])
def test_wide_types_against_python_sort_with_per_segment_k(key_type, largest, prefer_larger):
    rng = np.random.default_rng(23)
    S = 30
    sizes = rng.integers(-2, 300, S)
    off = np.concatenate([[3], 3 + np.cumsum(sizes)]).astype(np.int64)
    total = int(off.max()) + 5
    alpha = WIDE_ALPHABET[key_type]
    if key_type == "f64":
        pool = np.array(alpha + list(rng.normal(0, 1e3, 40)), dtype=np.float64)
    elif key_type in ("u64", "i64"):
        lo, hi = (0, 2 ** 64) if key_type == "u64" else (-(2 ** 63), 2 ** 63)
        pool = alpha + [int(x) for x in rng.integers(0, 2 ** 62, 40)] + [hi - 1 - j for j in range(5)]
        pool = [v for v in pool if lo <= v < hi]
    elif key_type in ("u8", "i8"):
        pool = alpha + [int(x) for x in rng.integers(0 if key_type == "u8" else -128, 128, 40)]
    else:
        pool = alpha + [int(x) for x in rng.integers(0 if key_type == "u16" else -(2 ** 15),
                                                      2 ** 15, 40)]
    keys = wide_keys([pool[i] for i in rng.integers(0, len(pool), total)], key_type)
    exact = wide_exact(keys, key_type)
    payload = rng.integers(0, 2 ** 63, total, dtype=np.int64).view(np.uint64) | np.uint64(1 << 63)
    k = 40
    kseg = rng.integers(-3, 60, S).astype(np.int32)
    kseg[0], kseg[1], kseg[2] = 0, 1000, k
    canary = np.full((S, k), 0xFEEDFACECAFEBEEF, np.uint64)
    ok, ov = oracle.batched_topk(keys, off, k, key_type=key_type, values=payload,
                                 largest=largest, prefer_larger=prefer_larger,
                                 out_values=canary, k_per_segment=kseg)
    for i in range(S):
        b, e = int(off[i]), int(off[i + 1])
        n = max(0, e - b)
        kk = min(max(int(kseg[i]), 0), k, n)
        want = _python_topk(exact[b:b + n], kk, largest, prefer_larger) if kk else []
        assert [int(v) for v in ov[i, :kk]] == [int(payload[b + j]) for j in want], i
        assert ok[i, :kk].tobytes() == keys[b + np.array(want, dtype=np.int64)].tobytes()
        assert np.all(ov[i, kk:] == np.uint64(0xFEEDFACECAFEBEEF)), i


@pytest.mark.parametrize("key_type", ALL_TYPES)
def test_per_segment_k_against_brute_force(key_type):
    """Each segment with its own k (0, 1, n, above n, above the row stride)
    against the exhaustive search, every direction and tie-break."""
    rng = np.random.default_rng(29)
    alpha = ALPHABET[key_type]
    S, k = 12, 5
    sizes = rng.integers(0, 8, S)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    total = int(off[-1])
    vals = [alpha[i] for i in rng.integers(0, len(alpha), total)]
    keys = as_keys(vals, key_type)
    num = numeric(keys, key_type)
    payload = np.arange(total, dtype=np.uint32) + 100
    kseg = np.array([0, 1, 2, 3, 4, 5, 6, 9, -1, 5, 2, 100], dtype=np.int32)
    for largest in (True, False):
        for pl in (False, True):
            _, ov = oracle.batched_topk(keys, off, k, key_type=key_type, values=payload,
                                        largest=largest, prefer_larger=pl,
                                        out_values=np.full((S, k), 1, np.uint32),
                                        k_per_segment=kseg)
            for i in range(S):
                b, n = int(off[i]), int(sizes[i])
                kk = min(max(int(kseg[i]), 0), k, n)
                if kk == 0:
                    assert np.all(ov[i] == 1)
                    continue
                want = brute_force(list(num[b:b + n]), kk, largest, pl)
                got = tuple(sorted(int(v) - 100 - b for v in ov[i, :kk]))
                assert got == want, (i, largest, pl)
                assert np.all(ov[i, kk:] == 1)


def test_per_segment_k_equal_to_k_matches_uniform_call():
    rng = np.random.default_rng(31)
    keys = rng.normal(size=5000).astype(np.float32)
    off = np.array([0, 100, 2000, 2001, 5000], dtype=np.int64)
    vals = np.arange(5000, dtype=np.uint32)
    a = oracle.batched_topk(keys, off, 64, values=vals)
    b = oracle.batched_topk(keys, off, 64, values=vals,
                            k_per_segment=np.full(4, 64, np.int32))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("key_type", ["u8", "i8"])
def test_every_8bit_pattern_in_order(key_type):
    """All 256 patterns, select-all + stable order, against Python's ordering
    of the integers they stand for."""
    pats = np.arange(256, dtype=np.uint8).view(WIDE_NUMPY[key_type])
    off = np.array([0, 256], dtype=np.int64)
    for largest in (True, False):
        _, ov = oracle.batched_topk(pats, off, 256, key_type=key_type,
                                    values=np.arange(256, dtype=np.uint32), largest=largest)
        want = sorted(range(256), key=lambda i: (-int(pats[i]) if largest else int(pats[i]), i))
        assert list(ov[0]) == want
