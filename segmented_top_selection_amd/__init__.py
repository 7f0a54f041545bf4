"""Segmented (batched) top-k on AMD Instinct MI355X.

A thin Python binding over the C-ABI library ``libsegtopk.so`` (declared in
``include/segtopk.h``).  It only marshals arguments: it allocates the output
tensors with torch when the caller does not pass them, and hands device
pointers and the current HIP stream to ``batched_topk``.  Every step of the
selection runs in the library's HIP kernels; there is no other code path, and
the binding raises if the library is missing.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsegtopk.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "segtopk.h")

# Values of the enums in include/segtopk.h.
KEY_TYPES = {"f32": 0, "bf16": 1, "u32": 2, "i32": 3, "f16": 4}
DIRECTIONS = {"max": 0, "min": 1}
DETERMINISM = {"not_guaranteed": 0, "run_to_run": 1, "gpu_to_gpu": 2}
TIE_BREAK = {"unspecified": 0, "prefer_smaller_index": 1, "prefer_larger_index": 2}
ORDERING = {"unsorted": 0, "sorted": 1, "stable_sorted": 2}
STATUS = {0: "ok", 1: "invalid argument", 2: "not supported", 3: "HIP error"}
MAX_SORTED_K = 4096

_DTYPE_KEY = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16",
              torch.int32: "i32"}
if hasattr(torch, "uint32"):
    _DTYPE_KEY[torch.uint32] = "u32"


class SegTopKError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"batched_topk failed: {STATUS.get(status, 'unknown')} (status {status})")
        self.status = status


class _Keys(ctypes.Structure):
    _fields_ = [("in_", ctypes.c_void_p), ("out", ctypes.c_void_p), ("type", ctypes.c_int32)]


class _Values(ctypes.Structure):
    _fields_ = [("in_", ctypes.c_void_p), ("out", ctypes.c_void_p)]


_lib = None


def library() -> ctypes.CDLL:
    """Loads libsegtopk.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library {LIB_PATH} is not built; run `python -c 'import "
                f"__graft_entry__; __graft_entry__.build()'` first")
        lib = ctypes.CDLL(LIB_PATH)
        lib.batched_topk.restype = ctypes.c_int
        lib.batched_topk.argtypes = [
            ctypes.POINTER(_Keys), ctypes.POINTER(_Values), ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_void_p]
        lib.segtopk_status_string.restype = ctypes.c_char_p
        lib.segtopk_status_string.argtypes = [ctypes.c_int]
        lib.segtopk_version.restype = ctypes.c_int
        _lib = lib
    return _lib


def header_functions() -> list:
    """Names of the functions include/segtopk.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text,
                      flags=re.M)


def raw_call(keys_in, keys_out, key_type, values_in, values_out, offsets, num_segments, k,
             direction, determinism, tie_break, ordering, stream=None) -> int:
    """Calls the C entry point with integer pointers; returns its status."""
    kd = _Keys(keys_in, keys_out, key_type)
    vd = _Values(values_in, values_out)
    return library().batched_topk(ctypes.byref(kd), ctypes.byref(vd) if values_in else None,
                                  offsets, num_segments, k, direction, determinism, tie_break,
                                  ordering, stream)


def batched_topk(keys: torch.Tensor, segment_offsets: torch.Tensor, k: int, *,
                 values: torch.Tensor | None = None, largest: bool = True,
                 determinism: str = "gpu_to_gpu", tie_break: str = "prefer_smaller_index",
                 ordering: str = "stable_sorted", key_type: str | None = None,
                 out_keys: torch.Tensor | None = None, out_values: torch.Tensor | None = None,
                 stream: torch.cuda.Stream | None = None):
    """Top-k of every segment of ``keys`` on the GPU.

    keys             1-D device tensor (float32, bfloat16, float16, int32; for
                     uint32 keys pass their bits as int32 with key_type="u32")
    segment_offsets  int64 device tensor of num_segments + 1 offsets
    values           optional 1-D 32-bit payload (int32/uint32/float32), same
                     length as keys
    Defaults follow the requirements page: gpu_to_gpu determinism,
    prefer_smaller_index ties, stable_sorted output.
    Returns (out_keys, out_values) of shape (num_segments, k); out_values is
    None for keys-only calls.  Row i holds min(k, n_i) results; the rest of the
    row is left as the caller's tensor had it (uninitialised when allocated
    here).
    """
    if key_type is None:
        if keys.dtype not in _DTYPE_KEY:
            raise TypeError(f"unsupported key dtype {keys.dtype}")
        key_type = _DTYPE_KEY[keys.dtype]
    if not keys.is_cuda or not segment_offsets.is_cuda:
        raise ValueError("keys and segment_offsets must be device tensors")
    if segment_offsets.dtype != torch.int64:
        raise TypeError("segment_offsets must be int64")
    keys = keys.contiguous()
    segment_offsets = segment_offsets.contiguous()
    s = segment_offsets.numel() - 1
    if out_keys is None:
        out_keys = torch.empty((max(s, 0), k), dtype=keys.dtype, device=keys.device)
    vin = vout = None
    if values is not None:
        if values.element_size() != 4:
            raise TypeError("values must be a 32-bit payload")
        values = values.contiguous()
        if out_values is None:
            out_values = torch.empty((max(s, 0), k), dtype=values.dtype, device=keys.device)
        vin, vout = values.data_ptr(), out_values.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream(keys.device)
    rc = raw_call(keys.data_ptr(), out_keys.data_ptr(), KEY_TYPES[key_type], vin, vout,
                  segment_offsets.data_ptr(), s, k, DIRECTIONS["max" if largest else "min"],
                  DETERMINISM[determinism], TIE_BREAK[tie_break], ORDERING[ordering],
                  stream.cuda_stream)
    if rc != 0:
        raise SegTopKError(rc)
    return out_keys, (out_values if values is not None else None)
