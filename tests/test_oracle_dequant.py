"""Pins for the oracle's dense dequantization (quant.dequant_bits) and for
the fp16-activation reading of the reference product.

dequant_bits is pinned by hand-derived bit patterns (tests/golden/
dequant_cases.json: ties to even both ways, overflow, subnormals, INT8 with
bf16 scales), by torch's own float64 -> bf16 / fp16 casts on random scales
and codes (an implementation independent of the oracle's encoders), and by
the identity probe: x = I_K through the product reads back the dequantized
weight before its final rounding. The fp16-activation product is pinned by
exact rational sums with activations decoded by Python's struct half format.
"""

import json
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import gemm, numerics, quant
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "dequant_cases.json")


def _torch_bits(values, out_dtype):
    t = torch.from_numpy(np.asarray(values, dtype=np.float64))
    t = t.to(torch.bfloat16 if out_dtype == "bf16" else torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_golden_cases():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        sb = np.array([[int(c["s_bits"], 16)]], dtype=np.uint16)
        q = np.full((128, 1), c["q"], dtype=np.int8)
        for out in ("bf16", "f16"):
            got = quant.dequant_bits(q, sb, c["s_dtype"], out)
            assert np.all(got == int(c[out], 16)), (c["note"], out, hex(int(got[0, 0])))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("s_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
def test_matches_torch_casts(bits, s_dtype, out_dtype):
    K, N = 384, 48
    q = workloads.codes(K, N, bits, 31)
    q[::7, ::3] = -8 if bits == 4 else -127
    sb = workloads.scales(K // 128, N, s_dtype, 32)
    sb[1, :5] = np.array([0x7BFF, 0x0001, 0x3C04, 0x3C0C, 0], dtype=np.uint16) if s_dtype == "f16" \
        else np.array([0x7F7F, 0x0001, 0x3F81, 0x3F83, 0], dtype=np.uint16)
    sv = np.asarray(sb).view(np.float16).astype(np.float64) if s_dtype == "f16" else \
        torch.from_numpy(np.asarray(sb).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    exact = q.astype(np.float64) * np.repeat(sv, 128, axis=0)
    assert np.array_equal(quant.dequant_bits(q, sb, s_dtype, out_dtype), _torch_bits(exact, out_dtype))


@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
def test_identity_probe_reads_the_dequantized_weight(out_dtype):
    K, N = 256, 32
    q = workloads.codes(K, N, 4, 41)
    sb = workloads.scales(2, N, "f16", 42)
    eye = np.where(np.eye(K, dtype=bool), np.uint16(0x3C00), np.uint16(0))   # fp16 1.0
    ref = gemm.gemm_ref(eye, q, sb, "f16", x_dtype="f16")
    enc = numerics.f64_exact_to_bf16 if out_dtype == "bf16" else numerics.f64_exact_to_f16
    assert np.array_equal(enc(ref), quant.dequant_bits(q, sb, "f16", out_dtype))


def _struct_f16(bits):
    return np.array([[struct.unpack("<e", struct.pack("<H", int(b)))[0] for b in row]
                     for row in np.asarray(bits)])


@pytest.mark.parametrize("bits,M,K,N", [(4, 2, 128, 16), (8, 3, 256, 16)])
def test_f16_activations_exact_rational_sum(bits, M, K, N):
    dt = quant.SCALE_DTYPE[bits]
    xb = numerics.f32_to_f16(np.random.default_rng(5).standard_normal((M, K)).astype(np.float32))
    q = workloads.codes(K, N, bits, 6)
    sb = workloads.scales(K // 128, N, dt, 7)
    xs = _struct_f16(xb)
    ss = numerics.scale_bits_to_f64(sb, dt)
    ref = gemm.gemm_ref(xb, q, sb, dt, x_dtype="f16")
    for m in range(M):
        for n in range(N):
            exact = sum((Fraction(float(xs[m, k])) * Fraction(float(ss[k // 128, n]))
                         * int(q[k, n]) for k in range(K)), Fraction(0))
            assert abs(Fraction(float(ref[m, n])) - exact) <= abs(exact) * Fraction(1, 2**40) \
                + Fraction(1, 2**80)


def test_f16_one_hot_rows():
    K, N = 256, 16
    q = workloads.codes(K, N, 4, 51)
    sb = workloads.scales(2, N, "f16", 52)
    ss = numerics.f16_to_f64(sb)
    x = np.zeros((2, K), dtype=np.uint16)
    x[0, 3] = 0x4400      # fp16 4.0 (as bf16 bits this would be 4.0 * 2^-120-ish garbage)
    x[1, 250] = 0xBC00    # fp16 -1.0
    ref = gemm.gemm_ref(x, q, sb, "f16", x_dtype="f16")
    assert np.array_equal(ref[0], 4.0 * ss[0] * q[3])
    assert np.array_equal(ref[1], -1.0 * ss[1] * q[250])
