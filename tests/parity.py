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
              "f16": 0xFFBE, "u16": 0xFFBE, "i16": 0xFFBE, "u64": 0x7FF0DEADBEEFCAFE,
              "i64": 0x7FF0DEADBEEFCAFE, "f64": 0x7FF0DEADBEEFCAFE, "u8": 0xBE, "i8": 0xBE}
VAL_CANARY = 0x5EEDF00D
VAL_CANARY64 = 0x5EEDF00DCAFED00D

TORCH_KEY_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16,
                   "u32": torch.int32, "i32": torch.int32, "u16": torch.int16,
                   "i16": torch.int16, "u64": torch.int64, "i64": torch.int64,
                   "f64": torch.float64, "u8": torch.uint8, "i8": torch.int8}


def key_bits_np(t: torch.Tensor) -> np.ndarray:
    """Raw key bits of a CPU/GPU tensor as uint32 numpy (uint64 for 8-byte
    keys)."""
    t = t.detach().cpu().contiguous()
    if t.element_size() == 1:
        return t.view(torch.uint8).numpy().astype(np.uint32)
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16).astype(np.uint32)
    if t.element_size() == 8:
        return t.view(torch.int64).numpy().view(np.uint64)
    return t.view(torch.int32).numpy().view(np.uint32)


def numeric_np(bits: np.ndarray, key_type: str) -> np.ndarray:
    """Key values from raw bits: float64 for the float types and the 32- and
    16-bit integers (exact); the 64-bit integers stay integers (exact)."""
    if key_type == "u64":
        return np.asarray(bits, dtype=np.uint64)
    if key_type == "i64":
        return np.asarray(bits, dtype=np.uint64).view(np.int64)
    if key_type == "f64":
        return np.asarray(bits, dtype=np.uint64).view(np.float64)
    bits = np.asarray(bits, dtype=np.uint32)
    if key_type == "u8":
        return bits.astype(np.float64)
    if key_type == "i8":
        return bits.astype(np.uint8).view(np.int8).astype(np.float64)
    if key_type == "f32":
        return bits.view(np.float32).astype(np.float64)
    if key_type == "bf16":
        return (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    if key_type == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if key_type in ("u32", "u16"):
        return bits.astype(np.float64)
    if key_type == "i16":
        return bits.astype(np.uint16).view(np.int16).astype(np.float64)
    return bits.view(np.int32).astype(np.float64)


def oracle_keys_view(bits_u32: np.ndarray, key_type: str) -> np.ndarray:
    if key_type == "u8":
        return bits_u32.astype(np.uint8)
    if key_type == "i8":
        return bits_u32.astype(np.uint8).view(np.int8)
    if key_type == "u64":
        return bits_u32.astype(np.uint64)
    if key_type == "i64":
        return bits_u32.astype(np.uint64).view(np.int64)
    if key_type == "f64":
        return bits_u32.astype(np.uint64).view(np.float64)
    if key_type in ("bf16", "f16", "u16"):
        return bits_u32.astype(np.uint16)
    if key_type == "i16":
        return bits_u32.astype(np.uint16).view(np.int16)
    if key_type == "f32":
        return bits_u32.view(np.float32)
    if key_type == "u32":
        return bits_u32
    return bits_u32.view(np.int32)


def _vals_np(t):
    """A payload tensor as uint32 or uint64 numpy (by element size)."""
    a = t.detach().cpu().contiguous()
    if a.element_size() == 8:
        return a.view(torch.int64).numpy().view(np.uint64)
    return a.view(torch.int32).numpy().view(np.uint32)


def run_gpu(keys, values, offsets, k, key_type, largest, determinism, tie_break, ordering,
            k_per_segment=None, max_segment_size=None):
    """Runs the library on device tensors with canary-filled outputs."""
    s = offsets.numel() - 1
    if os.environ.get("SEGTOPK_TEST_TRACE"):
        print(f"  call S={s} N={keys.numel()} k={k} {key_type} {'max' if largest else 'min'} "
              f"{determinism}/{tie_break}/{ordering} pairs={values is not None}", flush=True)
        sys.stdout.flush()
    dev = keys.device
    out_k = torch.empty((s, k), dtype=keys.dtype, device=dev)
    if keys.element_size() == 1:
        out_k.view(torch.uint8).fill_(KEY_CANARY[key_type])
    elif keys.element_size() == 2:
        out_k.view(torch.int16).fill_(KEY_CANARY[key_type] - 65536)
    elif keys.element_size() == 8:
        out_k.view(torch.int64).fill_(KEY_CANARY[key_type])
    else:
        out_k.view(torch.int32).fill_(KEY_CANARY[key_type])
    out_v = None
    if values is not None:
        if values.element_size() == 8:
            out_v = torch.full((s, k), VAL_CANARY64, dtype=torch.int64, device=dev)
        else:
            out_v = torch.full((s, k), VAL_CANARY, dtype=torch.int32, device=dev)
    st.batched_topk(keys, offsets, k, values=values, largest=largest, determinism=determinism,
                    tie_break=tie_break, ordering=ordering, key_type=key_type,
                    out_keys=out_k, out_values=out_v, k_per_segment=k_per_segment,
                    max_segment_size=max_segment_size)
    torch.cuda.synchronize()
    gk = key_bits_np(out_k).reshape(s, k)
    gv = _vals_np(out_v).reshape(s, k) if out_v is not None else None
    return gk, gv


def host_problem(keys, values, offsets_np, rows=None):
    """Host copies (key bits as uint32, values as uint32, offsets) of all
    segments, or of the listed rows re-packed as consecutive segments."""
    if rows is None:
        kb = key_bits_np(keys)
        vb = _vals_np(values) if values is not None else None
        return kb, vb, offsets_np
    parts_k, parts_v, off = [], [], [0]
    for r in rows:
        b, e = int(offsets_np[r]), int(offsets_np[r + 1])
        n = max(0, e - b)
        parts_k.append(key_bits_np(keys[b:b + n]))
        if values is not None:
            parts_v.append(_vals_np(values[b:b + n]))
        off.append(off[-1] + n)
    kb = np.concatenate(parts_k) if parts_k else np.zeros(0, np.uint32)
    vb = np.concatenate(parts_v) if values is not None else None
    return kb, vb, np.array(off, dtype=np.int64)


def run_oracle(keys_bits, values_u32, offsets_np, k, key_type, largest, prefer_larger,
               k_per_segment=None):
    ok, ov = oracle.batched_topk(oracle_keys_view(keys_bits, key_type), offsets_np, k,
                                 key_type=key_type, values=values_u32, largest=largest,
                                 prefer_larger=prefer_larger, k_per_segment=k_per_segment)
    if ok.dtype.itemsize == 1:
        ok = ok.view(np.uint8).astype(np.uint32)
    elif ok.dtype.itemsize == 2:
        ok = ok.view(np.uint16).astype(np.uint32)
    elif ok.dtype.itemsize == 8:
        ok = ok.view(np.uint64)
    else:
        ok = ok.view(np.uint32)
    return ok, ov


def _row_sizes(offsets_np, k, kseg=None):
    n = np.maximum(offsets_np[1:] - offsets_np[:-1], 0)
    ki = np.minimum(n, k)
    if kseg is not None:
        ki = np.minimum(ki, np.clip(np.asarray(kseg, dtype=np.int64), 0, None))
    return n, ki


def compare(gk, gv, ok, ov, offsets_np, k, key_type, determinism, ordering, keys_bits,
            values_are="index", kseg=None):
    """Asserts that the GPU rows (gk, gv) agree with the oracle rows (ok, ov);
    offsets_np / keys_bits describe exactly these rows.  ``values_are`` says
    what the payload holds, for the not_guaranteed validity check: the source
    index inside the segment ("index") or the key's position in the whole key
    array ("position"; needed when segments overlap)."""
    n_all, ki = _row_sizes(offsets_np, k, kseg)
    rows = np.arange(gk.shape[0])
    col = np.arange(k)[None, :]
    valid = col < ki[:, None]
    key_canary = KEY_CANARY[key_type]

    # untouched tails
    assert np.all(gk[~valid] == key_canary), "key slot past k_i was written"
    if gv is not None:
        vcan = VAL_CANARY64 if gv.dtype == np.uint64 else VAL_CANARY
        assert np.all(gv[~valid] == vcan), "value slot past k_i was written"

    if determinism != "not_guaranteed":
        if ordering != "unsorted":
            bad = (gk != ok) & valid
            assert not bad.any(), f"key mismatch in rows {rows[np.nonzero(bad.any(1))[0][:8]]}"
            if gv is not None:
                badv = (gv != ov) & valid
                assert not badv.any(), f"value mismatch in rows {rows[np.nonzero(badv.any(1))[0][:8]]}"
        else:
            def canon(kk, vv):
                # each row's (key bits, value) pairs in a canonical order
                kcol = np.where(valid, kk.astype(np.uint64), np.uint64(2 ** 63))
                if vv is None:
                    return np.sort(kcol, axis=1)[:, None, :]
                vcol = np.where(valid, vv.astype(np.uint64), np.uint64(0))
                order = np.lexsort((vcol, kcol), axis=1)
                return np.stack([np.take_along_axis(kcol, order, 1),
                                 np.take_along_axis(vcol, order, 1)], axis=1)
            a, b = canon(gk, gv), canon(ok, ov)
            bad = (a != b).any(axis=1)
            assert not bad.any(), f"set mismatch in rows {rows[np.nonzero(bad.any(1))[0][:8]]}"
        return

    # not_guaranteed: multiset of numeric key values
    gn, on = numeric_np(gk, key_type), numeric_np(ok, key_type)
    fill = np.inf if gn.dtype.kind == "f" else np.iinfo(gn.dtype).max
    gnum = np.where(valid, gn, fill)
    onum = np.where(valid, on, fill)
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
          values_are="index", k_per_segment=None, max_segment_size=None):
    """GPU call on device tensors, oracle on host copies, row comparison.
    With ``rows`` only those rows are checked (the GPU still runs all)."""
    gk, gv = run_gpu(keys, values, offsets, k, key_type, largest, determinism, tie_break,
                     ordering, k_per_segment, max_segment_size)
    off = offsets.cpu().numpy()
    kb, vb, sub_off = host_problem(keys, values, off, rows)
    kseg = k_per_segment.cpu().numpy() if k_per_segment is not None else None
    if kseg is not None and rows is not None:
        kseg = kseg[np.asarray(rows)]
    ok, ov = run_oracle(kb, vb, sub_off, k, key_type, largest,
                        tie_break == "prefer_larger_index", kseg)
    if rows is not None:
        gk = gk[np.asarray(rows)]
        gv = gv[np.asarray(rows)] if gv is not None else None
    compare(gk, gv, ok, ov, sub_off, k, key_type, determinism, ordering, kb, values_are, kseg)
    return gk, gv


def check_all_rows(keys, values, offsets, k, key_type, largest=True, determinism="gpu_to_gpu",
                   tie_break="prefer_smaller_index", ordering="stable_sorted", chunk_rows=1024,
                   say=None, max_segment_size=None):
    """One GPU call over the whole batch, then EVERY row compared with the
    oracle, in blocks of ``chunk_rows`` consecutive rows so that host memory
    stays bounded (segments must be laid out in order, as every workload's
    are).  Returns the number of rows compared."""
    gk, gv = run_gpu(keys, values, offsets, k, key_type, largest, determinism, tie_break,
                     ordering, max_segment_size=max_segment_size)
    off = offsets.cpu().numpy()
    s = off.shape[0] - 1
    for r0 in range(0, s, chunk_rows):
        r1 = min(s, r0 + chunk_rows)
        b, e = int(off[r0]), int(off[r1])
        assert np.all(np.diff(off[r0:r1 + 1]) >= 0), "check_all_rows needs ordered offsets"
        kb = key_bits_np(keys[b:e])
        vb = _vals_np(values[b:e]) if values is not None else None
        sub_off = off[r0:r1 + 1] - b
        ok, ov = run_oracle(kb, vb, sub_off, k, key_type, largest,
                            tie_break == "prefer_larger_index")
        compare(gk[r0:r1], gv[r0:r1] if gv is not None else None, ok, ov, sub_off, k,
                key_type, determinism, ordering, kb)
        if say is not None and (r1 == s or (r0 // chunk_rows) % 4 == 0):
            say(f"  rows [{r0}, {r1}) of {s} equal the oracle")
        del kb, vb, ok, ov
    return s
