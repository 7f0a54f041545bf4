"""Seeded synthetic inputs for segmented top-k.

This module only draws random numbers and lays them out as segments.  It holds
none of the selection arithmetic, imports neither the oracle nor the GPU
library, and is the single source of inputs for both sides of every parity
check and for the benchmark.

All generators use a ``torch.Generator`` on the requested device, seeded from
the arguments, so a given (workload, shape, seed, device) always yields the same
bytes.  Keys are returned as torch tensors holding the raw bit patterns the
library reads: float32, bfloat16, or int32 bits for uint32 keys.  Values are
int32 tensors holding the source index inside each segment.

Workloads (one call each; the seeds and shapes are in WORKLOADS below):
  uniform_f32   S x L float32 keys uniform in [-1, 1), keys only
  normal_f32    S x L float32 keys ~ N(0, 1), index values
  quantized     S variable-size segments (sizes uniform in [1, max_len]),
                float32 keys on 256 levels (L - 128) / 128 with 5% +0.0,
                5% -0.0, 1% +inf and 1% -inf, index values
  uniform_u32   S x L full-range uniform uint32 keys, index values
  normal10_f32  S x L float32 keys ~ 10 * N(0, 1), index values
  logits_bf16   S x L bfloat16 keys rounded from 3 * N(0, 1), index values
  (one segment of 2^28 float32 keys ~ 10 * N(0, 1): normal10_f32 with S = 1)
"""
from __future__ import annotations

import torch


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _index_values(num_segments, seg_len, device):
    # Source index inside each segment, as int32.
    return torch.arange(seg_len, dtype=torch.int32, device=device).repeat(num_segments)


def _fixed_offsets(num_segments, seg_len, device):
    return torch.arange(num_segments + 1, dtype=torch.int64, device=device) * seg_len


def uniform_f32(num_segments=16, seg_len=1000, seed=1001, device="cpu", values=False):
    g = _gen(device, seed)
    keys = torch.rand(num_segments * seg_len, generator=g, device=device) * 2.0 - 1.0
    vals = _index_values(num_segments, seg_len, device) if values else None
    return keys.float(), vals, _fixed_offsets(num_segments, seg_len, device)


def normal_f32(num_segments=4096, seg_len=4096, seed=1002, device="cpu", scale=1.0):
    g = _gen(device, seed)
    keys = torch.randn(num_segments * seg_len, generator=g, device=device) * scale
    return (keys.float(), _index_values(num_segments, seg_len, device),
            _fixed_offsets(num_segments, seg_len, device))


def quantized(num_segments=1024, max_len=65536, seed=1003, device="cpu"):
    g = _gen(device, seed)
    sizes = torch.randint(1, max_len + 1, (num_segments,), generator=g, device=device,
                          dtype=torch.int64)
    offsets = torch.zeros(num_segments + 1, dtype=torch.int64, device=device)
    offsets[1:] = torch.cumsum(sizes, 0)
    total = int(offsets[-1].item())
    level = torch.randint(0, 256, (total,), generator=g, device=device, dtype=torch.int32)
    keys = (level.float() - 128.0) / 128.0
    u = torch.rand(total, generator=g, device=device)
    keys = torch.where(u < 0.05, torch.zeros_like(keys), keys)
    keys = torch.where((u >= 0.05) & (u < 0.10), torch.full_like(keys, -0.0), keys)
    keys = torch.where((u >= 0.10) & (u < 0.11), torch.full_like(keys, float("inf")), keys)
    keys = torch.where((u >= 0.11) & (u < 0.12), torch.full_like(keys, float("-inf")), keys)
    starts = torch.repeat_interleave(offsets[:-1], sizes)
    vals = (torch.arange(total, dtype=torch.int64, device=device) - starts).to(torch.int32)
    return keys, vals, offsets


def uniform_u32(num_segments=32, seg_len=4194304, seed=1004, device="cpu"):
    g = _gen(device, seed)
    # Full 32-bit range, carried as int32 bit patterns.
    keys = torch.randint(-(2 ** 31), 2 ** 31, (num_segments * seg_len,), generator=g,
                         device=device, dtype=torch.int64).to(torch.int32)
    return (keys, _index_values(num_segments, seg_len, device),
            _fixed_offsets(num_segments, seg_len, device))


def normal10_f32(num_segments=32, seg_len=4194304, seed=1014, device="cpu"):
    return normal_f32(num_segments, seg_len, seed, device, scale=10.0)


def logits_bf16(num_segments=16384, seg_len=131072, seed=1005, device="cpu",
                chunk_rows=1024):
    """bf16(3 * N(0,1)) rounded to nearest even, generated in row chunks so
    that the float32 intermediate stays small."""
    g = _gen(device, seed)
    keys = torch.empty(num_segments * seg_len, dtype=torch.bfloat16, device=device)
    for r0 in range(0, num_segments, chunk_rows):
        r1 = min(num_segments, r0 + chunk_rows)
        x = torch.randn((r1 - r0) * seg_len, generator=g, device=device) * 3.0
        keys[r0 * seg_len:r1 * seg_len] = x.to(torch.bfloat16)
        del x
    return (keys, _index_values(num_segments, seg_len, device),
            _fixed_offsets(num_segments, seg_len, device))


# The five benchmark workloads, with their request parameters.  Shapes are
# the full sizes; tests call the generators above with smaller shapes.
WORKLOADS = {
    "uniform_f32_16x1000_k10": dict(
        gen=uniform_f32, args=dict(num_segments=16, seg_len=1000, seed=1001),
        key_type="f32", k=10, largest=True, determinism="gpu_to_gpu",
        tie_break="prefer_smaller_index", ordering="unsorted", pairs=False),
    "normal_f32_4096x4096_k64": dict(
        gen=normal_f32, args=dict(num_segments=4096, seg_len=4096, seed=1002),
        key_type="f32", k=64, largest=True, determinism="gpu_to_gpu",
        tie_break="prefer_smaller_index", ordering="stable_sorted", pairs=True),
    "quantized_f32_1024xU65536_k256": dict(
        gen=quantized, args=dict(num_segments=1024, max_len=65536, seed=1003),
        key_type="f32", k=256, largest=False, determinism="gpu_to_gpu",
        tie_break="prefer_smaller_index", ordering="stable_sorted", pairs=True),
    "uniform_u32_32x4Mi_k2048": dict(
        gen=uniform_u32, args=dict(num_segments=32, seg_len=4194304, seed=1004),
        key_type="u32", k=2048, largest=True, determinism="gpu_to_gpu",
        tie_break="prefer_larger_index", ordering="unsorted", pairs=True),
    "normal10_f32_32x4Mi_k2048": dict(
        gen=normal10_f32, args=dict(num_segments=32, seg_len=4194304, seed=1014),
        key_type="f32", k=2048, largest=True, determinism="gpu_to_gpu",
        tie_break="prefer_larger_index", ordering="unsorted", pairs=True),
    "normal10_f32_1x256Mi_k2048": dict(
        gen=normal10_f32, args=dict(num_segments=1, seg_len=1 << 28, seed=1024),
        key_type="f32", k=2048, largest=True, determinism="gpu_to_gpu",
        tie_break="prefer_smaller_index", ordering="unsorted", pairs=True),
    "logits_bf16_16384x128Ki_k50": dict(
        gen=logits_bf16, args=dict(num_segments=16384, seg_len=131072, seed=1005),
        key_type="bf16", k=50, largest=True, determinism="not_guaranteed",
        tie_break="unspecified", ordering="unsorted", pairs=True),
}
