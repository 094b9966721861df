"""Pins for oracle.numerics: the bit-level 16-bit float conversions.

Each conversion is checked against an independent library routine (torch's
bfloat16 cast, Python's struct 'e' half-precision codec) and against a few
hand-worked tie cases.
"""

import struct

import numpy as np
import pytest
import torch

from oracle import numerics


def _special_f32():
    vals = [0.0, -0.0, 1.0, -1.0, 1.00390625, 1.01171875, 3.0e38, -3.0e38,
            3.3895313892515355e38, 1e-40, -1e-45, 1.1754942e-38, 65504.0,
            65520.0, 6.0e-8, 2.9e-8, np.inf, -np.inf]
    return np.array(vals, dtype=np.float32)


def _random_f32(n, seed):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    return x[~np.isnan(x)]


def test_bf16_encode_matches_torch_cast():
    x = np.concatenate([_special_f32(), _random_f32(200000, 1),
                        np.random.default_rng(2).standard_normal(10000).astype(np.float32)])
    ours = numerics.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_ties_by_hand():
    # 1 + 2^-8 lies halfway between 1.0 (0x3F80) and 1 + 2^-7 (0x3F81): even wins.
    # 1 + 3*2^-8 lies halfway between 0x3F81 and 0x3F82: even (0x3F82) wins.
    x = np.array([1.00390625, 1.01171875, -1.00390625], dtype=np.float32)
    assert numerics.f32_to_bf16(x).tolist() == [0x3F80, 0x3F82, 0xBF80]


def test_bf16_nan_stays_nan():
    x = np.array([np.nan, -np.nan], dtype=np.float32)
    b = numerics.f32_to_bf16(x)
    assert np.all(np.isnan(numerics.bf16_to_f64(b)))


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    ours = numerics.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_f16_decode_matches_struct():
    bits = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    ours = numerics.f16_to_f64(bits)
    ref = np.array([struct.unpack("<e", int(b).to_bytes(2, "little"))[0] for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_f16_encode_matches_struct():
    x = np.concatenate([_special_f32()[np.abs(_special_f32()) < 65520],
                        np.random.default_rng(3).standard_normal(20000).astype(np.float32) * 0.01,
                        np.random.default_rng(4).standard_normal(2000).astype(np.float32) * 1e4])
    ours = numerics.f32_to_f16(x)
    ref = np.array([int.from_bytes(struct.pack("<e", float(v)), "little") for v in x],
                   dtype=np.uint16)
    assert np.array_equal(ours, ref)


def test_f16_overflow_rounds_to_inf():
    # 65520 is the midpoint between 65504 and the next (non-existent) step: RNE -> inf.
    x = np.array([65519.0, 65520.0, 1e9], dtype=np.float32)
    assert numerics.f32_to_f16(x).tolist() == [0x7BFF, 0x7C00, 0x7C00]


def test_exact_bf16_refuses_inexact():
    with pytest.raises(ValueError):
        numerics.f64_exact_to_bf16(np.array([1.0 + 2.0**-30]))
    assert numerics.f64_exact_to_bf16(np.array([0.5])).tolist() == [0x3F00]
