"""batched_topk_ex_noalloc (static scratch, no allocation) against
batched_topk_ex, through the C-ABI.

Two calls in a row on one stream, the second with a smaller input and a
different plan, then every row of both compared with what batched_topk_ex
returns for the same request: positionally and bitwise for stable_sorted
output, as sets of (key, value) pairs per row for unsorted output.  Also: the
plans without scratch, the largest-first plan, and a request whose plan needs
more than the static buffer (refused, nothing written).
"""
import numpy as np
import pytest
import torch

import segmented_top_selection_amd as st
from parity import check_all_rows, key_bits_np

pytestmark = pytest.mark.gpu

DEV = "cuda"
KEY_CANARY = 0x7FC0BEEF
VAL_CANARY = 0x5EEDF00D
ENUM = dict(max=0, min=1, not_guaranteed=0, run_to_run=1, gpu_to_gpu=2, unspecified=0,
            prefer_smaller_index=1, prefer_larger_index=2, unsorted=0, sorted=1, stable_sorted=2)


def problem(S, n, seed, levels=None):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    if isinstance(n, int):
        sizes = [n] * S
    else:
        sizes = list(n)
    off = torch.tensor(np.concatenate([[0], np.cumsum(sizes)]), dtype=torch.int64, device=DEV)
    total = int(off[-1])
    if levels:
        keys = torch.randint(0, levels, (total,), generator=g, device=DEV).float()
    else:
        keys = torch.randn(total, generator=g, device=DEV) * 10
    vals = torch.arange(total, dtype=torch.int32, device=DEV)
    return keys, vals, off


def outputs(S, k):
    ok = torch.full((S, k), KEY_CANARY, dtype=torch.int32, device=DEV)
    ov = torch.full((S, k), VAL_CANARY, dtype=torch.int32, device=DEV)
    return ok, ov


def call(fn, keys, vals, off, k, ok, ov, direction, det, tb, ordering, stream, hint=0):
    S = off.numel() - 1
    return fn(keys.data_ptr(), ok.data_ptr(), 0, vals.data_ptr(), ov.data_ptr(), 4,
              off.data_ptr(), S, k, None, hint, ENUM[direction], ENUM[det], ENUM[tb],
              ENUM[ordering], stream)


def reference(keys, vals, off, k, direction, det, tb, ordering):
    S = off.numel() - 1
    ok, ov = outputs(S, k)
    s = torch.cuda.current_stream().cuda_stream
    assert call(st.raw_call_ex, keys, vals, off, k, ok, ov, direction, det, tb, ordering, s) == 0
    torch.cuda.synchronize()
    return ok, ov


def same(a, b, ordering):
    ak, av = key_bits_np(a[0]), key_bits_np(a[1])
    bk, bv = key_bits_np(b[0]), key_bits_np(b[1])
    if ordering == "unsorted":
        ca = (ak.astype(np.uint64) << np.uint64(32)) | av.astype(np.uint64)
        cb = (bk.astype(np.uint64) << np.uint64(32)) | bv.astype(np.uint64)
        return np.array_equal(np.sort(ca, axis=1), np.sort(cb, axis=1))
    return np.array_equal(ak, bk) and np.array_equal(av, bv)


CASES = [
    # (problem args, k, direction, determinism, tie_break, ordering)
    ((8, 1 << 20, 11), 2048, "max", "gpu_to_gpu", "prefer_larger_index", "unsorted"),  # split
    ((3, 300000, 12), 500, "min", "gpu_to_gpu", "prefer_smaller_index", "stable_sorted"),  # spread
    ((300, np.random.default_rng(3).integers(0, 30000, 300), 13, 40), 256, "min", "gpu_to_gpu",
     "prefer_smaller_index", "stable_sorted"),  # largest first
    ((2100, 3000, 14), 64, "max", "gpu_to_gpu", "prefer_smaller_index", "stable_sorted"),  # none
    ((1, 1 << 22, 15, 100), 2048, "max", "gpu_to_gpu", "prefer_larger_index", "unsorted"),
]


@pytest.mark.parametrize("first,second", [(0, 1), (4, 1), (2, 3), (0, 2)])
def test_noalloc_matches_batched_topk_ex_two_calls(first, second):
    probs = [problem(*CASES[i][0]) for i in (first, second)]
    reqs = [CASES[i][1:] for i in (first, second)]
    refs = [reference(*p, *r) for p, r in zip(probs, reqs)]
    stream = torch.cuda.Stream()
    outs = []
    with torch.cuda.stream(stream):
        for p, r in zip(probs, reqs):
            o = outputs(p[2].numel() - 1, r[0])
            assert call(st.raw_call_ex_noalloc, *p, r[0], *o, *r[1:], stream.cuda_stream) == 0
            outs.append(o)
    torch.cuda.synchronize()
    for o, ref, r in zip(outs, refs, reqs):
        assert same(o, ref, r[-1])


def test_noalloc_first_case_against_the_oracle():
    keys, vals, off = problem(*CASES[1][0])
    k, direction, det, tb, ordering = CASES[1][1:]
    S = off.numel() - 1
    ok, ov = outputs(S, k)
    s = torch.cuda.current_stream().cuda_stream
    assert call(st.raw_call_ex_noalloc, keys, vals, off, k, ok, ov, direction, det, tb,
                ordering, s) == 0
    torch.cuda.synchronize()
    ref = reference(keys, vals, off, k, direction, det, tb, ordering)
    assert same((ok, ov), ref, ordering)
    check_all_rows(keys, vals, off, k, "f32", direction == "max", det, tb, ordering)


def test_noalloc_refuses_a_plan_larger_than_the_buffer():
    # 500 segments with k = 2048, split two ways when their sizes are unknown:
    # about 41 MB of per-workgroup candidate slots, more than the static
    # buffer's 32 MiB.
    keys, vals, off = problem(500, 10000, 16)
    ok, ov = outputs(500, 2048)
    s = torch.cuda.current_stream().cuda_stream
    rc = call(st.raw_call_ex_noalloc, keys, vals, off, 2048, ok, ov, "max", "gpu_to_gpu",
              "prefer_smaller_index", "unsorted", s)
    torch.cuda.synchronize()
    assert rc == 4
    assert st.library().segtopk_status_string(4).startswith(b"request needs more scratch")
    assert bool((ok == KEY_CANARY).all()) and bool((ov == VAL_CANARY).all())
    # The same request with a hint that rules out splitting needs only the
    # segment order (2 KB).
    assert call(st.raw_call_ex_noalloc, keys, vals, off, 2048, ok, ov, "max", "gpu_to_gpu",
                "prefer_smaller_index", "unsorted", s, hint=10000) == 0
    torch.cuda.synchronize()
    ref = reference(keys, vals, off, 2048, "max", "gpu_to_gpu", "prefer_smaller_index",
                    "unsorted")
    assert same((ok, ov), ref, "unsorted")


def test_noalloc_small_segment_kernel_matches_general_kernel():
    # A hint of at most 4096 keys selects the small-segment kernel (no
    # scratch); its rows must equal those of the general kernel, which the
    # same request without a hint takes.
    for args, k, ordering in (((2100, 3000, 17), 64, "stable_sorted"),
                              ((700, np.random.default_rng(5).integers(0, 4097, 700), 18, 9),
                               300, "unsorted")):
        keys, vals, off = problem(*args)
        S = off.numel() - 1
        ok, ov = outputs(S, k)
        s = torch.cuda.current_stream().cuda_stream
        assert call(st.raw_call_ex_noalloc, keys, vals, off, k, ok, ov, "max", "gpu_to_gpu",
                    "prefer_smaller_index", ordering, s, hint=4096) == 0
        torch.cuda.synchronize()
        ref = reference(keys, vals, off, k, "max", "gpu_to_gpu", "prefer_smaller_index", ordering)
        assert same((ok, ov), ref, ordering)
