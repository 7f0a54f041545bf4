"""CPU-side checks of the C-ABI library: it loads, exports every function the
header declares, and rejects bad requests before touching the GPU."""
import ctypes

import pytest

import segmented_top_selection_amd as st


def test_library_exports_every_declared_function():
    lib = st.library()
    names = st.header_functions()
    assert set(names) >= {"batched_topk", "batched_topk_ex", "segtopk_status_string",
                          "segtopk_version"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    lib = st.library()
    assert lib.segtopk_status_string(0) == b"ok"
    assert lib.segtopk_status_string(1) == b"invalid argument"
    assert lib.segtopk_status_string(2) == b"not supported"
    assert lib.segtopk_status_string(3) == b"HIP error"
    assert lib.segtopk_version() >= 100


# Fake, aligned "device" addresses: every call below must be refused (or be a
# no-op) before any of them is dereferenced or any HIP call is made.
K_IN, K_OUT, V_IN, V_OUT, OFF = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000


def call(**kw):
    a = dict(keys_in=K_IN, keys_out=K_OUT, key_type=0, values_in=V_IN, values_out=V_OUT,
             offsets=OFF, num_segments=4, k=8, direction=0, determinism=2, tie_break=1,
             ordering=2)
    a.update(kw)
    return st.raw_call(a["keys_in"], a["keys_out"], a["key_type"], a["values_in"],
                       a["values_out"], a["offsets"], a["num_segments"], a["k"],
                       a["direction"], a["determinism"], a["tie_break"], a["ordering"])


def test_null_keys_descriptor():
    lib = st.library()
    assert lib.batched_topk(None, None, OFF, 4, 8, 0, 2, 1, 2, None) == 1


@pytest.mark.parametrize("kw", [
    dict(keys_in=0), dict(keys_out=0), dict(offsets=0), dict(values_out=0),
    dict(key_type=-1), dict(key_type=12), dict(direction=2), dict(determinism=3),
    dict(tie_break=3), dict(ordering=3), dict(k=-1), dict(k=2 ** 31),
    dict(num_segments=-1), dict(num_segments=2 ** 31),
    dict(keys_in=K_IN + 2), dict(key_type=1, keys_out=K_OUT + 1), dict(values_in=V_IN + 2),
    dict(offsets=OFF + 4),
])
def test_invalid_arguments(kw):
    assert call(**kw) == 1


@pytest.mark.parametrize("det,tb", [(0, 1), (0, 2), (1, 1), (1, 2)])
def test_tie_break_requires_gpu_to_gpu(det, tb):
    assert call(determinism=det, tie_break=tb) == 1


def test_sorted_k_limit_not_supported():
    assert call(k=4097, ordering=1) == 2
    assert call(k=4097, ordering=2) == 2


def test_empty_requests_are_noops():
    assert call(k=0) == 0
    assert call(num_segments=0) == 0
    assert call(k=0, keys_in=0, keys_out=0, offsets=0) == 0


def call_ex(**kw):
    a = dict(keys_in=K_IN, keys_out=K_OUT, key_type=0, values_in=V_IN, values_out=V_OUT,
             value_bytes=4, offsets=OFF, num_segments=4, k=8, k_per_segment=None,
             max_segment_size=0, direction=0, determinism=2, tie_break=1, ordering=2)
    a.update(kw)
    return st.raw_call_ex(a["keys_in"], a["keys_out"], a["key_type"], a["values_in"],
                          a["values_out"], a["value_bytes"], a["offsets"], a["num_segments"],
                          a["k"], a["k_per_segment"], a["max_segment_size"], a["direction"],
                          a["determinism"], a["tie_break"], a["ordering"])


@pytest.mark.parametrize("kw", [
    dict(value_bytes=2), dict(value_bytes=0), dict(value_bytes=16),
    dict(value_bytes=8, values_in=V_IN + 4), dict(k_per_segment=0x60002),
    dict(keys_in=0), dict(key_type=12), dict(k=-1), dict(determinism=1, tie_break=2),
])
def test_ex_invalid_arguments(kw):
    assert call_ex(**kw) == 1


def test_ex_empty_requests_are_noops():
    assert call_ex(k=0, k_per_segment=0x60000) == 0
    assert call_ex(num_segments=0, value_bytes=8) == 0


def test_ex_sorted_k_limit_not_supported():
    assert call_ex(k=4097, ordering=2, max_segment_size=10) == 2


# --------------------------------------------------------------------------
# The Python binding refuses bad tensors before anything is queued (these run
# without a GPU: every check fires on host-side tensor metadata).
# --------------------------------------------------------------------------
import torch  # noqa: E402


def test_binding_rejects_host_tensors():
    keys = torch.zeros(10)
    off = torch.tensor([0, 10], dtype=torch.int64)
    with pytest.raises(ValueError):
        st.batched_topk(keys, off, 3)


def test_binding_rejects_unknown_key_type_and_negative_k():
    keys = torch.zeros(10)
    off = torch.tensor([0, 10], dtype=torch.int64)
    with pytest.raises(TypeError):
        st.batched_topk(keys.to(torch.complex64), off, 3)
    with pytest.raises(ValueError):
        st.batched_topk(keys, off, 3, key_type="x")
