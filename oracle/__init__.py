"""Plain CPU reference ("oracle") for segmented top-k.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
cpu_baseline leg are the only callers.  The GPU library never imports, links or
runs anything in this directory, and this directory imports nothing from the
GPU library.

The arithmetic lives in ``oracle.c`` (sort-and-take per segment, see the header
comment there for the definition and the passages it follows).  This module only
builds that file with gcc and marshals numpy arrays into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# The oracle's own key-type codes (independent of the GPU library's header).
KEY_TYPES = {"f32": 0, "bf16": 1, "u32": 2, "i32": 3, "f16": 4, "u16": 5, "i16": 6,
             "u64": 7, "i64": 8, "f64": 9, "u8": 10, "i8": 11}
KEY_NUMPY = {"f32": np.float32, "bf16": np.uint16, "u32": np.uint32, "i32": np.int32,
             "f16": np.uint16, "u16": np.uint16, "i16": np.int16, "u64": np.uint64,
             "i64": np.int64, "f64": np.float64, "u8": np.uint8, "i8": np.int8}

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (OpenMP over segments)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.oracle_batched_topk.restype = ctypes.c_int
        lib.oracle_batched_topk.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_batched_topk_ex.restype = ctypes.c_int
        lib.oracle_batched_topk_ex.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_default_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    return int(_load().oracle_default_threads())


def batched_topk(keys, offsets, k, *, key_type="f32", values=None, largest=True,
                 prefer_larger=False, threads=0, out_keys=None, out_values=None,
                 k_per_segment=None):
    """Sort-and-take top-k per segment.

    keys           1-D numpy array of raw key patterns (float32, uint16 bf16/f16
                   bits, uint32, int32, uint16, int16, uint64, int64, float64,
                   uint8 or int8, matching ``key_type``)
    offsets        int64 array of num_segments + 1 offsets
    values         optional 1-D payload array of 4- or 8-byte items (viewed as
                   uint32 / uint64)
    k_per_segment  optional int32 array: segment i keeps
                   min(max(k_per_segment[i], 0), k, n_i) items; k stays the row
                   stride
    Returns (out_keys, out_values) of shape (num_segments, k); rows are filled
    with the stable (better first, then index ascending) order of the kept
    items.  Slots past the kept count keep whatever ``out_keys`` /
    ``out_values`` held on entry (zeros when they are allocated here).
    """
    lib = _load()
    dt = KEY_NUMPY[key_type]
    keys = np.ascontiguousarray(keys).view(dt)
    offsets = np.ascontiguousarray(offsets, dtype=np.int64)
    s = offsets.shape[0] - 1
    if out_keys is None:
        out_keys = np.zeros((s, k), dtype=dt)
    vals_ptr = None
    vbytes = 4
    if values is not None:
        values = np.ascontiguousarray(values)
        vbytes = values.dtype.itemsize
        if vbytes not in (4, 8):
            raise ValueError("values must be a 4- or 8-byte payload")
        vdt = np.uint32 if vbytes == 4 else np.uint64
        values = values.view(vdt)
        if out_values is None:
            out_values = np.zeros((s, k), dtype=vdt)
        vals_ptr = values.ctypes.data
    kseg_ptr = None
    if k_per_segment is not None:
        k_per_segment = np.ascontiguousarray(k_per_segment, dtype=np.int32)
        if k_per_segment.shape[0] < s:
            raise ValueError("k_per_segment needs one entry per segment")
        kseg_ptr = k_per_segment.ctypes.data
    rc = lib.oracle_batched_topk_ex(
        keys.ctypes.data, KEY_TYPES[key_type], vals_ptr, vbytes, offsets.ctypes.data,
        s, k, kseg_ptr, 1 if largest else 0, 1 if prefer_larger else 0,
        out_keys.ctypes.data, out_values.ctypes.data if values is not None else None,
        int(threads))
    if rc != 0:
        raise ValueError(f"oracle_batched_topk failed with status {rc}")
    return out_keys, out_values
