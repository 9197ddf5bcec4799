"""C-ABI boundary checks that need no GPU.

The library must load, export every function ``include/vattn.h`` declares,
and reject bad arguments synchronously with the documented status codes
before any HIP call (the pointers passed here are never dereferenced).
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch  # noqa: F401  (loads the HIP runtime the library binds to)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vattn.h")

import non_causal_flash_amd as vattn  # noqa: E402


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vattn_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert _declared_functions() == sorted(vattn.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(vattn.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_library_links_only_one_hip_runtime():
    maps = open("/proc/self/maps").read()
    hip = {m for m in re.findall(r"\S*libamdhip64\S*", maps)}
    assert len(hip) == 1, hip


def test_status_strings():
    lib = vattn.lib
    for code in range(9):
        s = lib.vattn_status_string(code)
        assert s and s != b"unknown status"
    assert lib.vattn_status_string(99) == b"unknown status"
    assert lib.vattn_status_string(-1) == b"unknown status"


# Fake, 16-byte aligned, non-overlapping device addresses: validation fails
# (or succeeds trivially) before anything would touch them.
A, B, C, O = 0x10000000, 0x20000000, 0x30000000, 0x40000000


@pytest.mark.parametrize("args,status", [
    ((A, B, C, O, -1, 64, 64), vattn.VATTN_ERR_SIZE),
    ((A, B, C, O, 4, -5, 64), vattn.VATTN_ERR_SIZE),
    ((A, B, C, O, 4, 64, 65), vattn.VATTN_ERR_HEAD_DIM),
    ((A, B, C, O, 4, 64, 128), vattn.VATTN_ERR_HEAD_DIM),
    ((A, B, C, O, 4, 64, 0), vattn.VATTN_ERR_HEAD_DIM),
    ((0, B, C, O, 4, 64, 64), vattn.VATTN_ERR_NULL),
    ((A, 0, C, O, 4, 64, 64), vattn.VATTN_ERR_NULL),
    ((A, B, 0, O, 4, 64, 64), vattn.VATTN_ERR_NULL),
    ((A, B, C, 0, 4, 64, 64), vattn.VATTN_ERR_NULL),
    ((A + 4, B, C, O, 4, 64, 64), vattn.VATTN_ERR_ALIGN),
    ((A, B, C, O + 8, 4, 64, 64), vattn.VATTN_ERR_ALIGN),
    ((A, B, C, A, 4, 64, 64), vattn.VATTN_ERR_ALIAS),
    ((A, B, C, C + 4096, 4, 64, 64), vattn.VATTN_ERR_ALIAS),
    ((A, B, C, B - 1024, 1, 64, 64), vattn.VATTN_ERR_ALIAS),
    ((A, B, C, O, 1, 1 << 26, 64), vattn.VATTN_ERR_SIZE),
    ((A, B, C, O, 1, 1 << 24, 32), vattn.VATTN_ERR_SIZE),
    ((A, B, C, O, 1, (1 << 22) - 63, 64), vattn.VATTN_ERR_SIZE),
    ((A + 4, B, C, O, 4, 64, 40), vattn.VATTN_ERR_ALIGN),
    ((A, B, C, O, 1 << 30, 1 << 10, 32), vattn.VATTN_ERR_SIZE),
    ((0, 0, 0, 0, 0, 64, 64), vattn.VATTN_OK),
    ((0, 0, 0, 0, 4, 0, 64), vattn.VATTN_OK),
])
def test_argument_validation(args, status):
    assert vattn.forward_raw(*args) == status
    assert vattn.vattn_forward(*args) == status


H, N = 4, 100
# (args after the pointers: n_heads, n_patches, head_dim, stride_head, stride_patch)
STRIDED_CASES = [
    ((H, N, 64, 64, 64), vattn.VATTN_ERR_SIZE),            # heads overlap patches
    ((H, N, 64, N * 64, 32), vattn.VATTN_ERR_SIZE),        # stride_patch < head_dim
    ((H, N, 64, 32, H * 64), vattn.VATTN_ERR_SIZE),        # stride_head < head_dim
    ((H, N, 64, 64, H * 64 - 4), vattn.VATTN_ERR_SIZE),    # patch rows overlap
    ((H, N, 40, N * 48 - 4, 48), vattn.VATTN_ERR_SIZE),    # heads overlap
    ((H, 1 << 20, 64, 64, H * 64), vattn.VATTN_ERR_SIZE),  # span past 2^28
    ((H, N, 0, N * 64, 64), vattn.VATTN_ERR_HEAD_DIM),
    ((H, N, 65, N * 65, 65), vattn.VATTN_ERR_HEAD_DIM),
    ((0, N, 64, 64, 0), vattn.VATTN_OK),                   # nothing to do
]


@pytest.mark.parametrize("args,status", STRIDED_CASES)
def test_strided_argument_validation(args, status):
    assert vattn.forward_strided_raw(A, B, C, O, *args) == status


@pytest.mark.parametrize("args,offset,status", [
    # 16-byte alignment needed unless head_dim or a stride is not a multiple of 4
    ((H, N, 64, 64, H * 64), 4, vattn.VATTN_ERR_ALIGN),
    ((H, N, 40, N * 48, 48), 8, vattn.VATTN_ERR_ALIGN),
    ((H, N, 41, N * 41, 41), 2, vattn.VATTN_ERR_ALIGN),
])
def test_strided_alignment(args, offset, status):
    assert vattn.forward_strided_raw(A + offset, B, C, O, *args) == status


def test_strided_alias_uses_the_strided_extent():
    # patch-major: the tensor spans N * H * d floats; out starting inside it aliases
    span = N * H * 64 * 4
    assert vattn.forward_strided_raw(A, B, C, A + span - 256, H, N, 64, 64, H * 64) == \
        vattn.VATTN_ERR_ALIAS


def test_scalar_mode_accepts_4_byte_alignment():
    if torch.cuda.is_available():
        pytest.skip("launch would run on the GPU")
    # head_dim 41: single-float accesses, so a 4-byte aligned base reaches the launch
    assert vattn.forward_strided_raw(A + 4, B, C, O, H, N, 41, N * 41, 41) == vattn.VATTN_ERR_HIP


@pytest.mark.parametrize("args,offset,status", [
    # f16: vectors of 4 elements need 8-byte alignment; odd shapes only 2 bytes
    ((H, N, 64, N * 64, 64), 4, vattn.VATTN_ERR_ALIGN),
    ((H, N, 64, N * 64, 64), 2, vattn.VATTN_ERR_ALIGN),
    ((H, N, 41, N * 41, 41), 1, vattn.VATTN_ERR_ALIGN),
    ((H, N, 65, N * 65, 65), 0, vattn.VATTN_ERR_HEAD_DIM),
    ((H, N, 64, 64, 64), 0, vattn.VATTN_ERR_SIZE),
])
def test_f16_validation(args, offset, status):
    assert vattn.forward_f16_raw(A + offset, B, C, O, *args) == status


def test_f16_reaches_launch_with_8_byte_alignment():
    if torch.cuda.is_available():
        pytest.skip("launch would run on the GPU")
    assert vattn.forward_f16_raw(A + 8, B, C, O, H, N, 64, N * 64, 64) == vattn.VATTN_ERR_HIP
    assert vattn.forward_f16_raw(A + 2, B, C, O, H, N, 41, N * 41, 41) == vattn.VATTN_ERR_HIP


def test_unknown_precision_mode():
    assert vattn.forward_raw(A, B, C, O, 4, 64, 64, 0, 3) == vattn.VATTN_ERR_ARG
    assert vattn.forward_raw(A, B, C, O, 4, 64, 64, 0, -1) == vattn.VATTN_ERR_ARG
    # an unknown mode name is the binding's error, before any call
    with pytest.raises(ValueError, match="precision"):
        vattn.forward_raw(A, B, C, O, 4, 64, 64, 0, "fastest")
    with pytest.raises(ValueError, match="precision"):
        vattn.forward_rope_raw(A, B, C, O, 4, 64, 64, 64 * 64, 64, 64, T, 0, "exact")


def test_inputs_may_alias_each_other():
    # q == k == v is allowed; only out must be disjoint.  Valid sizes reach
    # the launch, so only check the no-device case on a machine without GPU.
    if torch.cuda.is_available():
        pytest.skip("launch would run on the GPU")
    assert vattn.forward_raw(A, A, A, O, 1, 8, 32) == vattn.VATTN_ERR_HIP


def test_no_device_reports_hip_error():
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert vattn.forward_raw(A, B, C, O, 2, 100, 64) == vattn.VATTN_ERR_HIP
    assert vattn.lib.vattn_last_hip_error() != 0


def test_python_wrapper_rejects_bad_tensors():
    x = torch.zeros(2, 8, 64)
    with pytest.raises(ValueError):
        vattn.forward(x, x, x)  # CPU tensors
    with pytest.raises(TypeError):
        vattn.forward(x.double(), x, x)
    with pytest.raises(TypeError):
        vattn.forward(x.half(), x, x)  # mixed dtypes
    with pytest.raises(ValueError):
        vattn.forward(x, x, x.transpose(1, 2).contiguous().transpose(1, 2))  # strided last dim


# ------------------------------------------------------------------ rotary
T = 0x50000000  # fake 16-byte aligned table address


@pytest.mark.parametrize("rope_dims,table,status", [
    (0, T, vattn.VATTN_ERR_ROPE),        # the rope entry needs rotary dims
    (4, T, vattn.VATTN_ERR_ROPE),        # below 8
    (12, T, vattn.VATTN_ERR_ROPE),       # not a multiple of 8
    (72, T, vattn.VATTN_ERR_ROPE),       # above head_dim
    (64, 0, vattn.VATTN_ERR_NULL),
    (64, T + 8, vattn.VATTN_ERR_ALIGN),
    (64, O + 64, vattn.VATTN_ERR_ALIAS),  # out overlaps the table
])
def test_rope_forward_validation(rope_dims, table, status):
    for f16 in (False, True):
        assert vattn.forward_rope_raw(A, B, C, O, H, N, 64, N * 64, 64, rope_dims, table,
                                      f16=f16) == status


def test_rope_dims_above_head_dim():
    assert vattn.forward_rope_raw(A, B, C, O, H, N, 40, N * 40, 40, 48, T) == vattn.VATTN_ERR_ROPE


def test_rope_empty_shapes_are_no_ops():
    assert vattn.forward_rope_raw(0, 0, 0, 0, 0, N, 64, 64, 64, 64, 0) == vattn.VATTN_OK
    # invalid rotary dims are reported even when there is nothing to do
    assert vattn.forward_rope_raw(0, 0, 0, 0, 0, N, 64, 64, 64, 6, 0) == vattn.VATTN_ERR_ROPE


def test_rope_forward_reaches_launch():
    if torch.cuda.is_available():
        pytest.skip("launch would run on the GPU")
    assert vattn.forward_rope_raw(A, B, C, O, H, N, 64, N * 64, 64, 32, T) == vattn.VATTN_ERR_HIP


@pytest.mark.parametrize("args,status", [
    ((T, 10, 0, 10000.0), vattn.VATTN_ERR_ROPE),
    ((T, 10, 7, 10000.0), vattn.VATTN_ERR_ROPE),
    ((T, 10, 66, 10000.0), vattn.VATTN_ERR_ROPE),
    ((T, 10, 8, 0.0), vattn.VATTN_ERR_ROPE),
    ((T, 10, 8, -5.0), vattn.VATTN_ERR_ROPE),
    ((T, 10, 8, float("inf")), vattn.VATTN_ERR_ROPE),
    ((T, 10, 8, float("nan")), vattn.VATTN_ERR_ROPE),
    ((T, -1, 8, 10000.0), vattn.VATTN_ERR_SIZE),
    ((0, 10, 8, 10000.0), vattn.VATTN_ERR_NULL),
    ((T + 4, 10, 8, 10000.0), vattn.VATTN_ERR_ALIGN),
    ((0, 0, 8, 10000.0), vattn.VATTN_OK),
])
def test_rope_table_validation(args, status):
    assert vattn.rope_table_raw(*args) == status


def test_rope_table_factors_and_positions():
    assert vattn.rope_table_raw(T, 10, 8, 100.0, [1.0, 2.0, 0.0, 1.0]) == vattn.VATTN_ERR_ROPE
    assert vattn.rope_table_raw(T, 10, 8, 100.0, [1.0, float("nan"), 1.0, 1.0]) == \
        vattn.VATTN_ERR_ROPE
    assert vattn.rope_table_raw(T, 10, 8, 100.0, None, -1) == vattn.VATTN_ERR_ROPE
    assert vattn.rope_table_raw(T, 10, 8, 100.0, None, 2**31 - 5) == vattn.VATTN_ERR_ROPE
    with pytest.raises(ValueError):
        vattn.rope_table_raw(T, 10, 8, 100.0, [1.0, 2.0])  # host array too short


def test_rope_table_reaches_launch():
    if torch.cuda.is_available():
        pytest.skip("launch would run on the GPU")
    assert vattn.rope_table_raw(T, 10, 8, 100.0, [1.0, 2.0, 3.0, 4.0], 7) == vattn.VATTN_ERR_HIP


def test_python_wrapper_rejects_bad_rope_table():
    x = torch.zeros(2, 8, 64)
    with pytest.raises(ValueError):
        vattn.forward(x, x, x, rope=torch.zeros(8, 32, 2))  # CPU tensors are rejected first
