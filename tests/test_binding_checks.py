"""The Python binding's host-side argument checks, on CPU tensors (the checks
read shapes, dtypes and byte counts only; nothing is launched).

A packed weight or a scale tensor that does not match (bits, K, N) is rejected
before the C ABI is called: the library takes plain pointers and could not
tell a wrong-sized buffer from a right one, so such a call would read out of
bounds or silently use the wrong scale order.
"""

import pytest
import torch

from int8_group_quantized_amd import binding as b

K, N = 256, 64


def _w(bits, K=K, N=N):
    return torch.zeros(b.packed_bytes(bits, K, N), dtype=torch.uint8)


@pytest.mark.parametrize("bits", [4, 8])
def test_matching_weight_passes(bits):
    s = torch.zeros((K // 128, N), dtype=torch.float16)
    b.check_weight(_w(bits), s, bits, K, N)
    cbm = torch.zeros((N // 16, K // 128, 16), dtype=torch.bfloat16)
    b.check_weight(_w(bits), cbm, bits, K, N, scales_cbm=True)


@pytest.mark.parametrize("bits", [4, 8])
def test_packed_size_must_match(bits):
    s = torch.zeros((K // 128, N), dtype=torch.float16)
    with pytest.raises(ValueError, match="packed_w"):
        b.check_weight(_w(bits, K, N + 16), s, bits, K, N)
    with pytest.raises(ValueError, match="packed_w"):
        b.check_weight(_w(12 - bits), s, bits, K, N)     # INT8 bytes passed as INT4 and back


def test_scale_shape_must_match():
    with pytest.raises(ValueError, match=r"\[K/128, N\]"):
        b.check_weight(_w(4), torch.zeros((K // 128, N + 16), dtype=torch.float16), 4, K, N)
    with pytest.raises(ValueError, match=r"\[K/128, N\]"):
        b.check_weight(_w(4), torch.zeros((N, K // 128), dtype=torch.float16), 4, K, N)


def test_column_block_major_scales_need_the_flag_and_the_shape():
    cbm = torch.zeros((N // 16, K // 128, 16), dtype=torch.float16)
    with pytest.raises(ValueError, match="scales_cbm=True"):
        b.check_weight(_w(4), cbm, 4, K, N)
    logical = torch.zeros((K // 128, N), dtype=torch.float16)
    with pytest.raises(ValueError, match="column-block-major"):
        b.check_weight(_w(4), logical, 4, K, N, scales_cbm=True)


def test_scale_dtype_and_bits():
    with pytest.raises(TypeError):
        b.check_weight(_w(4), torch.zeros((K // 128, N), dtype=torch.float32), 4, K, N)
    with pytest.raises(ValueError):
        b.check_weight(_w(4), torch.zeros((K // 128, N), dtype=torch.float16), 3, K, N)


def test_invalid_shapes_are_left_to_the_library():
    # K not a multiple of 128: the library answers QG_ERR_SHAPE; the binding
    # does not second-guess it with a size message
    b.check_weight(torch.zeros(10, dtype=torch.uint8), torch.zeros((1, N), dtype=torch.float16),
                   4, 100, N)
