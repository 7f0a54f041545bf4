"""Comparison of the GPU library's output with the CPU oracle's.

Deterministic modes pin the result SET; stable_sorted also pins positions.
not_guaranteed pins only the multiset of key values.  Rows are compared as:
  * deterministic + (stable_)sorted: positional, bitwise, keys and values
  * deterministic + unsorted: the row's (key bits, value) pairs as a sorted
    multiset, bitwise
  * not_guaranteed: the multiset of numeric key values equals the oracle's;
    every returned value (the source index) points at a key with exactly the
    returned bits; the values of a row are distinct
  * always: slots k_i .. k-1 still hold the canary
"""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import oracle
import segmented_top_selection_amd as st

KEY_CANARY = {"f32": 0x7FC0BEEF, "u32": 0x7FC0BEEF, "i32": 0x7FC0BEEF, "bf16": 0xFFBE,
              "f16": 0xFFBE}
VAL_CANARY = 0x5EEDF00D

TORCH_KEY_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16,
                   "u32": torch.int32, "i32": torch.int32}


def key_bits_np(t: torch.Tensor) -> np.ndarray:
    """Raw key bits of a CPU/GPU tensor as uint32 numpy."""
    t = t.detach().cpu().contiguous()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16).astype(np.uint32)
    return t.view(torch.int32).numpy().view(np.uint32)


def numeric_np(bits: np.ndarray, key_type: str) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint32)
    if key_type == "f32":
        return bits.view(np.float32).astype(np.float64)
    if key_type == "bf16":
        return (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    if key_type == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if key_type == "u32":
        return bits.astype(np.float64)
    return bits.view(np.int32).astype(np.float64)


def oracle_keys_view(bits_u32: np.ndarray, key_type: str) -> np.ndarray:
    if key_type in ("bf16", "f16"):
        return bits_u32.astype(np.uint16)
    if key_type == "f32":
        return bits_u32.view(np.float32)
    if key_type == "u32":
        return bits_u32
    return bits_u32.view(np.int32)


def run_gpu(keys, values, offsets, k, key_type, largest, determinism, tie_break, ordering):
    """Runs the library on device tensors with canary-filled outputs."""
    s = offsets.numel() - 1
    if os.environ.get("SEGTOPK_TEST_TRACE"):
        print(f"  call S={s} N={keys.numel()} k={k} {key_type} {'max' if largest else 'min'} "
              f"{determinism}/{tie_break}/{ordering} pairs={values is not None}", flush=True)
        sys.stdout.flush()
    dev = keys.device
    out_k = torch.empty((s, k), dtype=keys.dtype, device=dev)
    if keys.element_size() == 2:
        out_k.view(torch.int16).fill_(KEY_CANARY[key_type] - 65536)
    else:
        out_k.view(torch.int32).fill_(KEY_CANARY[key_type])
    out_v = None
    if values is not None:
        out_v = torch.full((s, k), VAL_CANARY, dtype=torch.int32, device=dev)
    st.batched_topk(keys, offsets, k, values=values, largest=largest, determinism=determinism,
                    tie_break=tie_break, ordering=ordering, key_type=key_type,
                    out_keys=out_k, out_values=out_v)
    torch.cuda.synchronize()
    gk = key_bits_np(out_k).reshape(s, k)
    gv = out_v.cpu().numpy().view(np.uint32).reshape(s, k) if out_v is not None else None
    return gk, gv


def host_problem(keys, values, offsets_np, rows=None):
    """Host copies (key bits as uint32, values as uint32, offsets) of all
    segments, or of the listed rows re-packed as consecutive segments."""
    if rows is None:
        kb = key_bits_np(keys)
        vb = values.cpu().numpy().view(np.uint32) if values is not None else None
        return kb, vb, offsets_np
    parts_k, parts_v, off = [], [], [0]
    for r in rows:
        b, e = int(offsets_np[r]), int(offsets_np[r + 1])
        n = max(0, e - b)
        parts_k.append(key_bits_np(keys[b:b + n]))
        if values is not None:
            parts_v.append(values[b:b + n].cpu().numpy().view(np.uint32))
        off.append(off[-1] + n)
    kb = np.concatenate(parts_k) if parts_k else np.zeros(0, np.uint32)
    vb = np.concatenate(parts_v) if values is not None else None
    return kb, vb, np.array(off, dtype=np.int64)


def run_oracle(keys_bits, values_u32, offsets_np, k, key_type, largest, prefer_larger):
    ok, ov = oracle.batched_topk(oracle_keys_view(keys_bits, key_type), offsets_np, k,
                                 key_type=key_type, values=values_u32, largest=largest,
                                 prefer_larger=prefer_larger)
    ok = ok.astype(np.uint32) if ok.dtype == np.uint16 else ok.view(np.uint32)
    return ok, ov


def _row_sizes(offsets_np, k):
    n = np.maximum(offsets_np[1:] - offsets_np[:-1], 0)
    return n, np.minimum(n, k)


def compare(gk, gv, ok, ov, offsets_np, k, key_type, determinism, ordering, keys_bits,
            values_are="index"):
    """Asserts that the GPU rows (gk, gv) agree with the oracle rows (ok, ov);
    offsets_np / keys_bits describe exactly these rows.  ``values_are`` says
    what the payload holds, for the not_guaranteed validity check: the source
    index inside the segment ("index") or the key's position in the whole key
    array ("position"; needed when segments overlap)."""
    n_all, ki = _row_sizes(offsets_np, k)
    rows = np.arange(gk.shape[0])
    col = np.arange(k)[None, :]
    valid = col < ki[:, None]
    key_canary = KEY_CANARY[key_type]

    # untouched tails
    assert np.all(gk[~valid] == key_canary), "key slot past k_i was written"
    if gv is not None:
        assert np.all(gv[~valid] == VAL_CANARY), "value slot past k_i was written"

    if determinism != "not_guaranteed":
        if ordering != "unsorted":
            bad = (gk != ok) & valid
            assert not bad.any(), f"key mismatch in rows {rows[np.nonzero(bad.any(1))[0][:8]]}"
            if gv is not None:
                badv = (gv != ov) & valid
                assert not badv.any(), f"value mismatch in rows {rows[np.nonzero(badv.any(1))[0][:8]]}"
        else:
            def canon(kk, vv):
                c = kk.astype(np.uint64) << np.uint64(32)
                if vv is not None:
                    c |= vv.astype(np.uint64)
                c = np.where(valid, c, np.uint64(0xFFFFFFFFFFFFFFFF))
                return np.sort(c, axis=1)
            a, b = canon(gk, gv), canon(ok, ov)
            bad = a != b
            assert not bad.any(), f"set mismatch in rows {rows[np.nonzero(bad.any(1))[0][:8]]}"
        return

    # not_guaranteed: multiset of numeric key values
    gnum = np.where(valid, numeric_np(gk, key_type), np.inf)
    onum = np.where(valid, numeric_np(ok, key_type), np.inf)
    assert np.array_equal(np.sort(gnum, axis=1), np.sort(onum, axis=1)), "key multiset mismatch"
    if gv is not None:
        starts = offsets_np[:-1]
        if values_are == "index":
            inb = (gv.astype(np.int64) < n_all[:, None]) | ~valid
            src = np.where(valid, starts[:, None] + gv.astype(np.int64), 0)
        else:
            g = gv.astype(np.int64)
            inb = ((g >= starts[:, None]) & (g < starts[:, None] + n_all[:, None])) | ~valid
            src = np.where(valid, g, 0)
        assert inb.all(), "value (index) out of the segment"
        back = keys_bits[src] if keys_bits.size else np.zeros_like(gk)
        assert np.all((back == gk) | ~valid), "returned key is not the key at the returned index"
        sv = np.sort(np.where(valid, gv.astype(np.int64), -1 - col), axis=1)
        assert np.all(np.diff(sv, axis=1) != 0), "an index was returned twice"


def check(keys, values, offsets, k, key_type, largest=True, determinism="gpu_to_gpu",
          tie_break="prefer_smaller_index", ordering="stable_sorted", rows=None,
          values_are="index"):
    """GPU call on device tensors, oracle on host copies, row comparison.
    With ``rows`` only those rows are checked (the GPU still runs all)."""
    gk, gv = run_gpu(keys, values, offsets, k, key_type, largest, determinism, tie_break,
                     ordering)
    off = offsets.cpu().numpy()
    kb, vb, sub_off = host_problem(keys, values, off, rows)
    ok, ov = run_oracle(kb, vb, sub_off, k, key_type, largest,
                        tie_break == "prefer_larger_index")
    if rows is not None:
        gk = gk[np.asarray(rows)]
        gv = gv[np.asarray(rows)] if gv is not None else None
    compare(gk, gv, ok, ov, sub_off, k, key_type, determinism, ordering, kb, values_are)
    return gk, gv


def check_all_rows(keys, values, offsets, k, key_type, largest=True, determinism="gpu_to_gpu",
                   tie_break="prefer_smaller_index", ordering="stable_sorted", chunk_rows=1024,
                   say=None):
    """One GPU call over the whole batch, then EVERY row compared with the
    oracle, in blocks of ``chunk_rows`` consecutive rows so that host memory
    stays bounded (segments must be laid out in order, as every workload's
    are).  Returns the number of rows compared."""
    gk, gv = run_gpu(keys, values, offsets, k, key_type, largest, determinism, tie_break,
                     ordering)
    off = offsets.cpu().numpy()
    s = off.shape[0] - 1
    for r0 in range(0, s, chunk_rows):
        r1 = min(s, r0 + chunk_rows)
        b, e = int(off[r0]), int(off[r1])
        assert np.all(np.diff(off[r0:r1 + 1]) >= 0), "check_all_rows needs ordered offsets"
        kb = key_bits_np(keys[b:e])
        vb = values[b:e].cpu().numpy().view(np.uint32) if values is not None else None
        sub_off = off[r0:r1 + 1] - b
        ok, ov = run_oracle(kb, vb, sub_off, k, key_type, largest,
                            tie_break == "prefer_larger_index")
        compare(gk[r0:r1], gv[r0:r1] if gv is not None else None, ok, ov, sub_off, k,
                key_type, determinism, ordering, kb)
        if say is not None and (r1 == s or (r0 // chunk_rows) % 4 == 0):
            say(f"  rows [{r0}, {r1}) of {s} equal the oracle")
        del kb, vb, ok, ov
    return s
