"""Scale choice and the fixed-grid quantizer Q_s, written out plainly.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources
  * arXiv 2607.04244, QAD method paragraph: the student keeps the frozen
    symmetric per-group scales s, its weights W start at s (.) W_q and pass
    through a fixed-grid fake quantizer Q_s; at packing time the updated
    bf16 weights are rounded back onto the same grid, giving new INT4 codes
    under the original scales.
  * same paper, drafter-PTQ calibration paragraph: group-wise symmetric INT4
    with group size 128.
  * Qwen3.5-4B-DFlash-W8A16 model card, "What changed vs upstream" table and
    the recipe paragraph below it: int8 weight-only, RTN, symmetric,
    group = 128, bf16 scales, no calibration data.

Readings taken where the pages are silent (each is listed in the design
notes of the repository):
  * groups run along K (the input-feature axis), one scale per (group, output
    column); scales are stored [K/128, N];
  * INT4 codes lie in [-8, 7], INT8 codes in [-127, 127];
  * RTN picks s = max|w| / 7 (INT4) or max|w| / 127 (INT8), divided in fp32
    and stored as fp16 (INT4) or bf16 (INT8) with RNE; a NaN weight counts as
    0 for the maximum;
  * Q_s divides in fp32 with IEEE (correctly rounded) division -- never a
    multiply by a reciprocal -- rounds the quotient to nearest with ties to
    even, then clamps; a zero scale or a NaN quotient gives code 0 and an
    infinite quotient saturates to the end of the range.
"""

import numpy as np

from . import numerics

GROUP = 128

RANGE = {4: (-8, 7), 8: (-127, 127)}
RTN_DIVISOR = {4: 7.0, 8: 127.0}
SCALE_DTYPE = {4: "f16", 8: "bf16"}


def group_count(K):
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    return K // GROUP


def expand_groups(s, K):
    """Repeat a [K/128, N] per-group array along K to [K, N]."""
    return np.repeat(np.asarray(s), GROUP, axis=0)[:K]


def rtn_scales(W, bits):
    """Round-to-nearest scale choice; returns stored scale bit patterns.

    W: float32 [K, N]. For each group g and column n the scale is the largest
    magnitude in W[128g : 128g+128, n] divided (fp32) by 7 or 127, rounded to
    fp16 (bits=4) or bf16 (bits=8). Returns uint16 [K/128, N].
    """
    W = np.asarray(W, dtype=np.float32)
    K, N = W.shape
    G = group_count(K)
    mag = np.abs(W)
    mag = np.where(np.isnan(mag), np.float32(0.0), mag)
    amax = mag.reshape(G, GROUP, N).max(axis=1).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        s32 = amax / np.float32(RTN_DIVISOR[bits])
    if bits == 4:
        return numerics.f32_to_f16(s32)
    return numerics.f32_to_bf16(s32)


def q_s(W, scale_values, bits):
    """Fixed-grid quantizer: codes = clamp(rne(W / s), lo, hi).

    W: float32 [K, N] (bf16 weights are passed as their exact fp32 values).
    scale_values: the stored scales decoded to real numbers, [K/128, N].
    Returns int8 codes [K, N].
    """
    W = np.asarray(W, dtype=np.float32)
    K, _ = W.shape
    s = expand_groups(np.asarray(scale_values, dtype=np.float64), K).astype(np.float32)
    lo, hi = RANGE[bits]
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        t = W / s                         # IEEE fp32 division, elementwise
    q = np.rint(t)                        # ties to even
    q = np.clip(q, lo, hi)
    q = np.where((s == 0) | np.isnan(t), 0.0, q)
    return q.astype(np.int8)


def rtn_quantize(W, bits):
    """RTN from scratch: scales from the weights, then Q_s under them.

    Returns (codes int8 [K,N], scale bit patterns uint16 [K/128,N]).
    """
    sb = rtn_scales(W, bits)
    sv = numerics.scale_bits_to_f64(sb, SCALE_DTYPE[bits])
    return q_s(W, sv, bits), sb


def dequant(codes, scale_values):
    """s (.) W_q as float64: every element is exact (at most 15 significant
    bits: an 11-bit fp16 or 8-bit bf16 scale times a code of magnitude <= 127).
    """
    c = np.asarray(codes).astype(np.float64)
    return c * expand_groups(np.asarray(scale_values, dtype=np.float64), c.shape[0])


def dequant_bits(codes, scale_bits, scale_dtype, out_dtype):
    """The dense dequantized weight s (.) W_q stored in a 16-bit format: the
    exact product (see dequant) rounded once, to nearest even, into bf16 or
    fp16 ("bf16" / "f16"); returns uint16 bit patterns [K, N].

    QAD paragraph of arXiv 2607.04244: the student starts from the
    dequantized weights s (.) W_q; the adaptfm-quant-dflash README (Stage 2)
    keeps a dense dequantized bf16 twin of the INT4 model.
    """
    w = dequant(codes, numerics.scale_bits_to_f64(scale_bits, scale_dtype))
    if out_dtype == "bf16":
        return numerics.f64_exact_to_bf16(w)
    if out_dtype == "f16":
        return numerics.f64_exact_to_f16(w)
    raise ValueError(out_dtype)


def fake_quant(W, scale_bits, scale_dtype, bits, out_dtype):
    """The fixed-grid fake quantizer of QAD, s (.) Q_s(W), as stored values.

    QAD paragraph of arXiv 2607.04244: the student's weights W pass through
    Q_s under the frozen scales in the forward pass; the codes are those of
    q_s (same division and rounding), the product s * q is exact in fp32, and
    the one rounding is into out_dtype: "bf16" / "f16" give uint16 bit
    patterns, "f32" gives float32 values.

    The straight-through estimator of the same paragraph (Bengio et al. 2013)
    passes the gradient through Q_s unchanged, so its backward is the
    identity on the incoming gradient and needs no separate definition here.
    """
    sv = numerics.scale_bits_to_f64(scale_bits, scale_dtype)
    w = dequant(q_s(W, sv, bits), sv)
    if out_dtype == "bf16":
        return numerics.f64_exact_to_bf16(w)
    if out_dtype == "f16":
        return numerics.f64_exact_to_f16(w)
    if out_dtype == "f32":
        return w.astype(np.float32)
    raise ValueError(out_dtype)
