"""Reference product out = x . (s (.) W_q) and the parity acceptance test.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources
  * arXiv 2607.04244, QAD method paragraph: the effective weight of a
    quantized Linear is the dequantized s (.) W_q; the target is served as
    W4A16 (4-bit weights, 16-bit activations).
  * adaptfm-quant-dflash README, "Stage 2: Target Model": the grid is served
    as INT4-weight with 16-bit activations.
  * Qwen3.5-4B-DFlash-W8A16 model card, "What changed vs upstream" table:
    the INT8 variant with bf16 scales.

The reference is the plain definition: decode x (bf16) and the scales
exactly, form s (.) W_q exactly, and take the matrix product in float64 with
a library matmul. Every product x*s*q is exact in float64 and the only
rounding is float64 summation, some 2^-29 below fp32's, so this stands in for
the exact sum. No blocking, no reordering beyond the library call.

Acceptance for floating-point parity (the reading used for the tolerance):
  |gpu - ref| <= 1e-2 * |ref| + 1e-3 * rms(ref)   elementwise,
where ref is the float64 result before any output rounding and rms is taken
over the whole [M, N] output of one call.
"""

import numpy as np

from . import numerics
from .quant import dequant


def gemm_ref(x_bits, codes, scale_bits, scale_dtype, x_dtype="bf16"):
    """x_bits: 16-bit activation patterns [M, K] (bf16, or fp16 with
    x_dtype="f16"); codes int8 [K, N]; scale_bits [K/128, N].

    Returns the float64 product [M, N].
    """
    x = numerics.act_to_f64(x_bits, x_dtype)
    w = dequant(codes, numerics.scale_bits_to_f64(scale_bits, scale_dtype))
    return x @ w


def gemm_ref_at(x_bits, codes, scale_bits, scale_dtype, rows, cols, x_dtype="bf16"):
    """The same definition evaluated only at output positions (rows[i], cols[i]).

    For full-size shapes, where the whole product is too slow on a CPU, each
    requested output is one dot product over K in float64.
    """
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    x = numerics.act_to_f64(np.asarray(x_bits)[rows], x_dtype)        # [P, K]
    sv = numerics.scale_bits_to_f64(np.asarray(scale_bits)[:, cols], scale_dtype)
    w = dequant(np.asarray(codes)[:, cols], sv)                         # [K, P]
    return np.einsum("pk,kp->p", x, w)


def rms(ref):
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0


def within_tolerance(gpu, ref, ref_rms=None):
    """Boolean mask of elements meeting the acceptance bound."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    r = rms(ref) if ref_rms is None else ref_rms
    return np.abs(gpu - ref) <= 1e-2 * np.abs(ref) + 1e-3 * r
