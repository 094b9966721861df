"""Bit-level conversions between fp32/fp64 and the 16-bit float formats.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The oracle carries its own bf16 encoder because numpy has no bfloat16 type.
Rounding is round-to-nearest, ties-to-even (RNE) throughout: the pages do not
name a rounding mode for any conversion (QAD paragraph of arXiv 2607.04244
only says weights are rounded "back onto the same quantization grid"), and RNE
is the IEEE default that both the fp32->fp16 scale store and the bf16 output
store take here.

Formats
  bf16: 1 sign, 8 exponent, 7 mantissa bits -- the upper half of an fp32.
  fp16: 1 sign, 5 exponent, 10 mantissa bits (IEEE binary16).
"""

import numpy as np


def bf16_to_f64(bits):
    """Decode bf16 bit patterns (uint16 array) to float64, exactly.

    A bf16 value is the fp32 whose upper 16 bits are the pattern and whose
    lower 16 bits are zero, so the decode is a shift and a reinterpretation.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f16_to_f64(bits):
    """Decode IEEE binary16 bit patterns (uint16 array) to float64, exactly."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f32_to_bf16(x):
    """Round fp32 values to bf16 with RNE; returns uint16 bit patterns.

    Adding 0x7FFF plus the lowest kept bit to the 32-bit pattern and keeping
    the upper half rounds to nearest with ties to even; a carry out of the
    mantissa moves into the exponent, which is the correct result (and turns
    values above the largest finite bf16 into infinity). NaN inputs become the
    canonical quiet NaN with the input's sign.
    """
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if np.any(nan):
        sign = ((u >> np.uint64(16)) & np.uint64(0x8000)).astype(np.uint16)
        r = np.where(nan, sign | np.uint16(0x7FC0), r).astype(np.uint16)
    return r


def f32_to_f16(x):
    """Round fp32 values to IEEE binary16 with RNE; returns uint16 patterns.

    numpy's float32 -> float16 cast is a single correctly rounded conversion
    (subnormals and overflow to infinity included), so it is used directly.
    """
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _exact_f32(x):
    """float64 -> fp32 for values that fp32 holds exactly; magnitudes of 2^128
    and beyond (past the fp32 range, so also past every 16-bit format's
    overflow threshold) become infinities of the same sign. Anything else
    that fp32 cannot hold is refused rather than rounded twice."""
    x = np.asarray(x, dtype=np.float64)
    big = np.abs(x) >= 2.0 ** 128
    with np.errstate(over="ignore"):
        x32 = np.where(big, np.copysign(np.inf, x), x).astype(np.float32)
    check = np.isfinite(x) & ~big
    if not np.array_equal(x32.astype(np.float64)[check], x[check]):
        raise ValueError("value not exactly representable in fp32")
    return x32


def f64_exact_to_bf16(x):
    """bf16 RNE of float64 values that are exactly representable in fp32
    (beyond the fp32 range: infinity).

    Used only where a result is known to be fp32-exact (the products s*q of
    the identity probe and of dequantization); refuses anything else rather
    than double-rounding.
    """
    return f32_to_bf16(_exact_f32(x))


def f64_exact_to_f16(x):
    """IEEE binary16 RNE of float64 values that are exactly representable in
    fp32 (same contract as f64_exact_to_bf16); overflow gives infinity."""
    return f32_to_f16(_exact_f32(x))


def act_to_f64(bits, dtype):
    """Decode 16-bit activations; ``dtype`` is "bf16" or "f16"."""
    if dtype == "bf16":
        return bf16_to_f64(bits)
    if dtype == "f16":
        return f16_to_f64(bits)
    raise ValueError(dtype)


def scale_bits_to_f64(bits, dtype):
    """Decode stored scales; ``dtype`` is "f16" or "bf16"."""
    if dtype == "f16":
        return f16_to_f64(bits)
    if dtype == "bf16":
        return bf16_to_f64(bits)
    raise ValueError(dtype)
