"""Pins for the oracle's fixed-grid fake quantizer quant.fake_quant.

Pinned by the ties table worked by hand (tests/golden/qs_ties.json: the codes
that round-to-nearest-even plus clamping give, times the scale), by the grid
fixed point the QAD paragraph relies on (a weight already on the grid,
s * q, comes back unchanged), by idempotence, by the error bound |fq(W) - W|
<= s/2 inside the clamp range, and by a brute-force scalar loop in Python
floats for a small matrix.
"""

import json
import os
import struct

import numpy as np
import pytest

from oracle import numerics, quant
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


def _f16(b):
    return struct.unpack("<e", struct.pack("<H", int(b)))[0]


@pytest.mark.parametrize("bits", [4, 8])
def test_ties_table_times_scale(bits):
    ties = json.load(open(os.path.join(HERE, "golden", "qs_ties.json")))["int%d" % bits]
    sb = np.array([[0x3800]], dtype=np.uint16)       # fp16 0.5: every product exact
    for t, code in ties:
        W = np.full((128, 1), t * 0.5, dtype=np.float32)
        got = quant.fake_quant(W, sb, "f16", bits, "f32")
        assert np.all(got == np.float32(code * 0.5)), (t, code, got[0, 0])


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("out", ["bf16", "f16", "f32"])
def test_grid_points_are_fixed(bits, out):
    K, N = 256, 48
    sdt = quant.SCALE_DTYPE[bits]
    q = workloads.codes(K, N, bits, 3)
    sb = workloads.scales(K // 128, N, sdt, 4)
    W = quant.dequant(q, numerics.scale_bits_to_f64(sb, sdt)).astype(np.float32)   # exact
    got = quant.fake_quant(W, sb, sdt, bits, out)
    enc = {"bf16": numerics.f64_exact_to_bf16, "f16": numerics.f64_exact_to_f16,
           "f32": lambda v: np.asarray(v, dtype=np.float32)}[out]
    assert np.array_equal(got, enc(W.astype(np.float64)))


@pytest.mark.parametrize("bits", [4, 8])
def test_idempotent_and_within_half_step(bits):
    K, N = 384, 64
    sdt = quant.SCALE_DTYPE[bits]
    W = workloads.weights(K, N, 5)
    sb = quant.rtn_scales(W, bits)
    s = quant.expand_groups(numerics.scale_bits_to_f64(sb, sdt), K)
    f1 = quant.fake_quant(W, sb, sdt, bits, "f32")
    assert np.array_equal(quant.fake_quant(f1, sb, sdt, bits, "f32"), f1)
    lo, hi = quant.RANGE[bits]
    inside = (W / s >= lo - 0.5) & (W / s <= hi + 0.5)
    assert np.all(np.abs(f1.astype(np.float64) - W)[inside] <= s[inside] / 2 * (1 + 1e-6))


def test_brute_force_small():
    K, N = 128, 4
    W = workloads.weights(K, N, 9, dist="student_t") * np.float32(3)
    sb = np.array([[0x2400, 0x2C00, 0x1E00, 0x0000]], dtype=np.uint16)   # fp16 scales, one zero
    got = quant.fake_quant(W, sb, "f16", 4, "bf16")
    for k in range(K):
        for n in range(N):
            s = np.float32(_f16(sb[0, n]))
            if s == 0:
                q = 0
            else:
                t = np.float32(W[k, n]) / s                       # fp32 division
                q = int(min(max(np.rint(t), -8), 7))
            v = float(s) * q
            want = numerics.f32_to_bf16(np.float32(v))
            assert got[k, n] == want, (k, n)
