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
KEY_TYPES = {"f32": 0, "bf16": 1, "u32": 2, "i32": 3, "f16": 4, "u16": 5, "i16": 6,
             "u64": 7, "i64": 8, "f64": 9, "u8": 10, "i8": 11}
KEY_BYTES = {"f32": 4, "bf16": 2, "u32": 4, "i32": 4, "f16": 2, "u16": 2, "i16": 2,
             "u64": 8, "i64": 8, "f64": 8, "u8": 1, "i8": 1}
DIRECTIONS = {"max": 0, "min": 1}
DETERMINISM = {"not_guaranteed": 0, "run_to_run": 1, "gpu_to_gpu": 2}
TIE_BREAK = {"unspecified": 0, "prefer_smaller_index": 1, "prefer_larger_index": 2}
ORDERING = {"unsorted": 0, "sorted": 1, "stable_sorted": 2}
STATUS = {0: "ok", 1: "invalid argument", 2: "not supported", 3: "HIP error",
          4: "scratch too small"}
MAX_SORTED_K = 4096

_DTYPE_KEY = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16",
              torch.int32: "i32", torch.int16: "i16", torch.int64: "i64",
              torch.float64: "f64", torch.uint8: "u8", torch.int8: "i8"}
if hasattr(torch, "uint32"):
    _DTYPE_KEY[torch.uint32] = "u32"
if hasattr(torch, "uint16"):
    _DTYPE_KEY[torch.uint16] = "u16"
if hasattr(torch, "uint64"):
    _DTYPE_KEY[torch.uint64] = "u64"


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
        lib.batched_topk_ex.restype = ctypes.c_int
        lib.batched_topk_ex.argtypes = [
            ctypes.POINTER(_Keys), ctypes.POINTER(_Values), ctypes.c_int32, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.batched_topk_ex_noalloc.restype = ctypes.c_int
        lib.batched_topk_ex_noalloc.argtypes = lib.batched_topk_ex.argtypes
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
    """Calls batched_topk with integer pointers; returns its status."""
    kd = _Keys(keys_in, keys_out, key_type)
    vd = _Values(values_in, values_out)
    return library().batched_topk(ctypes.byref(kd), ctypes.byref(vd) if values_in else None,
                                  offsets, num_segments, k, direction, determinism, tie_break,
                                  ordering, stream)


def raw_call_ex(keys_in, keys_out, key_type, values_in, values_out, value_bytes, offsets,
                num_segments, k, k_per_segment, max_segment_size, direction, determinism,
                tie_break, ordering, stream=None) -> int:
    """Calls batched_topk_ex with integer pointers; returns its status."""
    kd = _Keys(keys_in, keys_out, key_type)
    vd = _Values(values_in, values_out)
    return library().batched_topk_ex(ctypes.byref(kd), ctypes.byref(vd) if values_in else None,
                                     value_bytes, offsets, num_segments, k, k_per_segment,
                                     max_segment_size, direction, determinism, tie_break,
                                     ordering, stream)


def raw_call_ex_noalloc(keys_in, keys_out, key_type, values_in, values_out, value_bytes,
                        offsets, num_segments, k, k_per_segment, max_segment_size, direction,
                        determinism, tie_break, ordering, stream=None) -> int:
    """Calls batched_topk_ex_noalloc (static scratch, no allocation)."""
    kd = _Keys(keys_in, keys_out, key_type)
    vd = _Values(values_in, values_out)
    return library().batched_topk_ex_noalloc(
        ctypes.byref(kd), ctypes.byref(vd) if values_in else None, value_bytes, offsets,
        num_segments, k, k_per_segment, max_segment_size, direction, determinism, tie_break,
        ordering, stream)


# torch's handle of the current stream without building a Stream object (about
# 2 us per call less on the host); the public route where it is missing.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _device_tensor(name, t, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a device tensor on {device} (got {t.device})")


def _output_tensor(name, t, device, elem_bytes, need):
    _device_tensor(name, t, device)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.element_size() != elem_bytes:
        raise TypeError(f"{name} must have {elem_bytes}-byte elements "
                        f"(got {t.element_size()})")
    if t.numel() < need:
        raise ValueError(f"{name} holds {t.numel()} elements; num_segments * k = {need} needed")


def batched_topk(keys: torch.Tensor, segment_offsets: torch.Tensor, k: int, *,
                 values: torch.Tensor | None = None, largest: bool = True,
                 determinism: str = "gpu_to_gpu", tie_break: str = "prefer_smaller_index",
                 ordering: str = "stable_sorted", key_type: str | None = None,
                 out_keys: torch.Tensor | None = None, out_values: torch.Tensor | None = None,
                 stream: torch.cuda.Stream | None = None,
                 k_per_segment: torch.Tensor | None = None,
                 max_segment_size: int | None = None):
    """Top-k of every segment of ``keys`` on the GPU.

    keys             1-D device tensor (float32, bfloat16, float16, float64,
                     int32, int16, int64, int8, uint8; for the other unsigned
                     keys pass their bits as the signed type of the same width
                     with key_type="u32" / "u16" / "u64")
    segment_offsets  int64 device tensor of num_segments + 1 offsets
    values           optional 1-D payload of 4- or 8-byte items (any dtype),
                     same length as keys
    k_per_segment    optional int32 device tensor: segment i keeps
                     min(max(k_per_segment[i], 0), k, n_i) items; k stays the
                     row stride of the outputs
    max_segment_size optional host-side hint: no segment is longer (it steers
                     the launch plan only); without one, the number of keys
                     is passed, which bounds every segment of valid offsets
    Defaults follow the requirements page: gpu_to_gpu determinism,
    prefer_smaller_index ties, stable_sorted output.
    Returns (out_keys, out_values) of shape (num_segments, k); out_values is
    None for keys-only calls.  Row i holds its k_i results; the rest of the row
    is left as the caller's tensor had it (uninitialised when allocated here).
    Bad tensors (host memory, another device, wrong element size, outputs too
    small or not contiguous) raise before anything is queued.
    """
    if not isinstance(keys, torch.Tensor):
        raise TypeError("keys must be a torch tensor")
    if key_type is None:
        if keys.dtype not in _DTYPE_KEY:
            raise TypeError(f"unsupported key dtype {keys.dtype}")
        key_type = _DTYPE_KEY[keys.dtype]
    if key_type not in KEY_TYPES:
        raise ValueError(f"unknown key_type {key_type!r}")
    if not keys.is_cuda:
        raise ValueError("keys must be a device tensor")
    dev = keys.device
    if keys.element_size() != KEY_BYTES[key_type]:
        raise TypeError(f"key_type {key_type} needs {KEY_BYTES[key_type]}-byte keys "
                        f"(got {keys.dtype})")
    _device_tensor("segment_offsets", segment_offsets, dev)
    if segment_offsets.dtype != torch.int64:
        raise TypeError("segment_offsets must be int64")
    if segment_offsets.dim() != 1 or segment_offsets.numel() < 1:
        raise ValueError("segment_offsets must be 1-D with num_segments + 1 entries")
    k = int(k)
    if k < 0:
        raise ValueError("k must be >= 0")
    if keys.dim() != 1 or not keys.is_contiguous():
        keys = keys.reshape(-1).contiguous()
    if not segment_offsets.is_contiguous():
        segment_offsets = segment_offsets.contiguous()
    s = segment_offsets.numel() - 1
    if out_keys is None:
        out_keys = torch.empty((s, k), dtype=keys.dtype, device=dev)
    _output_tensor("out_keys", out_keys, dev, keys.element_size(), s * k)
    vin = vout = None
    vbytes = 4
    if values is not None:
        _device_tensor("values", values, dev)
        vbytes = values.element_size()
        if vbytes not in (4, 8):
            raise TypeError("values must be a 4- or 8-byte payload")
        if values.dim() != 1 or not values.is_contiguous():
            values = values.reshape(-1).contiguous()
        if values.numel() < keys.numel():
            raise ValueError("values must hold one item per key")
        if out_values is None:
            out_values = torch.empty((s, k), dtype=values.dtype, device=dev)
        _output_tensor("out_values", out_values, dev, vbytes, s * k)
        vin, vout = values.data_ptr(), out_values.data_ptr()
    kseg_ptr = None
    if k_per_segment is not None:
        _device_tensor("k_per_segment", k_per_segment, dev)
        if k_per_segment.dtype != torch.int32:
            raise TypeError("k_per_segment must be int32")
        k_per_segment = k_per_segment.reshape(-1).contiguous()
        if k_per_segment.numel() < s:
            raise ValueError("k_per_segment needs one entry per segment")
        kseg_ptr = k_per_segment.data_ptr()
    if stream is not None:
        sp = stream.cuda_stream
    elif _raw_stream is not None:
        sp = _raw_stream(dev.index)  # the current stream's handle, no Stream object
    else:
        sp = torch.cuda.current_stream(dev).cuda_stream
    args = (DIRECTIONS["max" if largest else "min"], DETERMINISM[determinism],
            TIE_BREAK[tie_break], ORDERING[ordering], sp)
    # Offsets index the keys, so no segment of a valid call is longer than
    # the key count: a hint the plan can use when the caller gives none (a
    # batch of small segments then needs no splitting and no scratch).
    hint = keys.numel() if max_segment_size is None else int(max_segment_size)
    rc = raw_call_ex(keys.data_ptr(), out_keys.data_ptr(), KEY_TYPES[key_type], vin, vout,
                     vbytes, segment_offsets.data_ptr(), s, k, kseg_ptr, hint, *args)
    if rc != 0:
        raise SegTopKError(rc)
    return out_keys, (out_values if values is not None else None)
