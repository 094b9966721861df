"""Pins for oracle.gemm: the reference product and the acceptance test.

The product is pinned by exact rational arithmetic on tiny shapes (inputs
decoded by library routines, not by the oracle), by closed forms -- the
identity probe of the W8A16 model card's "Required vLLM patches" section,
one-hot and all-ones activations, constant codes -- and by linearity. Shapes
are non-square and scales differ per group and column, so a transposed
operand or a group axis taken along N fails.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import gemm, numerics, quant
import workloads


def _lib_bf16(bits):
    return torch.from_numpy(np.asarray(bits).view(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()


def _lib_scale(bits, dtype):
    if dtype == "f16":
        return np.asarray(bits).view(np.float16).astype(np.float64)
    return _lib_bf16(bits)


@pytest.mark.parametrize("bits,M,K,N", [(4, 1, 128, 16), (4, 3, 256, 32),
                                        (8, 2, 256, 16), (8, 4, 128, 32)])
def test_matches_exact_rational_sum(bits, M, K, N):
    dt = quant.SCALE_DTYPE[bits]
    x = workloads.activations(M, K, 1)
    q = workloads.codes(K, N, bits, 2)
    sb = workloads.scales(K // 128, N, dt, 3)
    xs = _lib_bf16(x)
    ss = _lib_scale(sb, dt)
    ref = gemm.gemm_ref(x, q, sb, dt)
    for m in range(M):
        for n in range(N):
            exact = sum((Fraction(float(xs[m, k])) * Fraction(float(ss[k // 128, n]))
                         * int(q[k, n]) for k in range(K)), Fraction(0))
            assert abs(Fraction(float(ref[m, n])) - exact) <= abs(exact) * Fraction(1, 2**40) \
                + Fraction(1, 2**80)


@pytest.mark.parametrize("bits", [4, 8])
def test_identity_probe(bits):
    """x = I_K reads the effective weight back: out[k, n] = s[k//128, n] q[k, n]."""
    K, N = 256, 48
    dt = quant.SCALE_DTYPE[bits]
    q = workloads.codes(K, N, bits, 11)
    sb = workloads.scales(K // 128, N, dt, 12)
    eye = np.where(np.eye(K, dtype=bool), np.uint16(0x3F80), np.uint16(0))
    ref = gemm.gemm_ref(eye, q, sb, dt)
    ss = _lib_scale(sb, dt)
    want = np.array([[ss[k // 128, n] * int(q[k, n]) for n in range(N)] for k in range(K)])
    assert np.array_equal(ref, want)
    # the bf16 image of the probe is exact: s*q fits fp32
    b = numerics.f64_exact_to_bf16(ref)
    assert b.shape == (K, N)


def test_one_hot_power_of_two_rows():
    K, N = 384, 32
    q = workloads.codes(K, N, 4, 21)
    sb = workloads.scales(3, N, "f16", 22)
    ss = _lib_scale(sb, "f16")
    x = np.zeros((3, K), dtype=np.uint16)
    x[0, 5] = 0x4000           # 2.0
    x[1, 200] = 0x3E80         # 0.25
    x[2, 383] = 0xC100         # -8.0
    ref = gemm.gemm_ref(x, q, sb, "f16")
    assert np.array_equal(ref[0], 2.0 * ss[0] * q[5])
    assert np.array_equal(ref[1], 0.25 * ss[1] * q[200])
    assert np.array_equal(ref[2], -8.0 * ss[2] * q[383])


def test_all_ones_gives_integer_group_sums():
    K, N = 512, 32
    q = workloads.codes(K, N, 4, 31)
    sb = workloads.scales(4, N, "f16", 32)
    ss = _lib_scale(sb, "f16")
    x = np.full((1, K), 0x3F80, dtype=np.uint16)
    ref = gemm.gemm_ref(x, q, sb, "f16")[0]
    isums = q.astype(np.int64).reshape(4, 128, N).sum(axis=1)       # exact integers
    want = (ss * isums).sum(axis=0)
    assert np.allclose(ref, want, rtol=1e-15, atol=0)


def test_constant_code():
    K, N, M = 256, 16, 2
    x = workloads.activations(M, K, 41)
    sb = workloads.scales(2, N, "f16", 42)
    q = np.full((K, N), -3, dtype=np.int8)
    ref = gemm.gemm_ref(x, q, sb, "f16")
    xs = _lib_bf16(x).reshape(M, 2, 128).sum(axis=2)                  # [M, G]
    want = -3 * xs @ _lib_scale(sb, "f16")
    assert np.allclose(ref, want, rtol=1e-13, atol=1e-15)


def test_linearity():
    K, N, M = 256, 32, 3
    q = workloads.codes(K, N, 8, 51)
    sb = workloads.scales(2, N, "bf16", 52)
    xa = workloads.activations(M, K, 53)
    xb = workloads.activations(M, K, 54)
    a = _lib_bf16(xa)
    b = _lib_bf16(xb)
    ssum = workloads.to_bf16_bits((a + b).astype(np.float32))
    exact_sum = np.array_equal(_lib_bf16(ssum), a + b)
    ra = gemm.gemm_ref(xa, q, sb, "bf16")
    rb = gemm.gemm_ref(xb, q, sb, "bf16")
    if exact_sum:
        assert np.allclose(gemm.gemm_ref(ssum, q, sb, "bf16"), ra + rb, rtol=1e-12, atol=1e-12)
    # scaling the scales by 2 doubles the result exactly
    s2 = workloads.to_bf16_bits(_lib_bf16(sb).astype(np.float32) * 2)
    assert np.array_equal(gemm.gemm_ref(xa, q, s2, "bf16"), 2 * ra)


def test_sampled_equals_full():
    K, N, M = 384, 64, 5
    q = workloads.codes(K, N, 4, 61)
    sb = workloads.scales(3, N, "f16", 62)
    x = workloads.activations(M, K, 63)
    full = gemm.gemm_ref(x, q, sb, "f16")
    rows = np.array([0, 4, 2, 3])
    cols = np.array([63, 0, 17, 40])
    assert np.allclose(gemm.gemm_ref_at(x, q, sb, "f16", rows, cols), full[rows, cols],
                       rtol=1e-14, atol=1e-14)


def test_tolerance_rule():
    ref = np.array([1.0, -2.0, 0.0, 100.0])
    r = gemm.rms(ref)
    ok = gemm.within_tolerance(ref + np.array([0.0099, -0.0199, 0.9e-3 * r, 0.0]), ref)
    assert ok.all()
    bad = gemm.within_tolerance(ref + np.array([0.0, 0.0, 1.1e-3 * r, 0.0]), ref)
    assert bad.tolist() == [True, True, False, True]
    assert not gemm.within_tolerance(np.array([np.nan]), np.array([1.0])).any()
    # an all-zero reference admits only exact zeros
    z = np.zeros(3)
    assert gemm.within_tolerance(np.array([0.0, -0.0, 0.0]), z).all()
    assert not gemm.within_tolerance(np.array([1e-30, 0.0, 0.0]), z)[0]
