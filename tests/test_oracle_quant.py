"""Pins for oracle.quant: RTN scale choice and the fixed-grid quantizer Q_s.

What the pages fix (arXiv 2607.04244, QAD paragraph; drafter-PTQ paragraph;
W8A16 model card table): the grid is symmetric per group of 128 with frozen
scales, the student starts at s (.) W_q, and packing rounds the updated bf16
weights back onto that same grid. Hence the pins below: codes stay in range,
s (.) W_q is a fixed point (also after bf16 rounding), Q_s is idempotent and
monotone with error at most s/2, ties follow the hand-worked table, and RTN
scales make the largest code of every non-zero group hit the range end.
"""

import json
import math
import os
import struct

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import numerics, quant

GOLD = os.path.join(os.path.dirname(__file__), "golden")
RANGE = {4: (-8, 7), 8: (-127, 127)}


def _scales(bits, n, seed):
    """Positive scales spread over many binades, decoded to float64."""
    rng = np.random.default_rng(seed)
    s = np.exp(rng.uniform(np.log(1e-4), np.log(50.0), size=n)).astype(np.float32)
    if bits == 4:
        return s.astype(np.float16).astype(np.float64)
    t = torch.from_numpy(s).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


@pytest.mark.parametrize("bits", [4, 8])
def test_fixed_point_of_dequantized_grid(bits):
    """Q_s(s (.) W_q) = W_q for every code and 4000 scales (exact products)."""
    lo, hi = RANGE[bits]
    codes = np.arange(lo, hi + 1)
    s = _scales(bits, 4000, 10 + bits)
    K = 128
    # one group per column: column c uses scale s[c]; rows cycle through all codes
    q = np.resize(codes, K)[:, None].repeat(len(s), axis=1).astype(np.int8)
    W = (q.astype(np.float64) * s[None, :]).astype(np.float32)   # exact in fp32
    assert np.array_equal(W.astype(np.float64), q * s[None, :])
    got = quant.q_s(W, s[None, :], bits)
    assert np.array_equal(got, q)


@pytest.mark.parametrize("bits", [4, 8])
def test_fixed_point_survives_bf16_rounding(bits):
    """Packing starts from bf16 weights: Q_s(bf16(s (.) W_q)) = W_q."""
    lo, hi = RANGE[bits]
    s = _scales(bits, 4000, 20 + bits)
    q = np.resize(np.arange(lo, hi + 1), 128)[:, None].repeat(len(s), axis=1).astype(np.int8)
    W = (q.astype(np.float64) * s[None, :]).astype(np.float32)
    Wb = torch.from_numpy(W).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(quant.q_s(Wb, s[None, :], bits), q)


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), bits=st.sampled_from([4, 8]),
       spread=st.floats(1e-3, 1e3))
def test_codes_always_in_range(seed, bits, spread):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((256, 16)) * spread).astype(np.float32)
    W[rng.random(W.shape) < 0.01] = np.inf
    W[rng.random(W.shape) < 0.01] = -np.inf
    W[rng.random(W.shape) < 0.01] = np.nan
    s = _scales(bits, 32, seed % 1000).reshape(2, 16)
    s[0, 0] = 0.0
    q = quant.q_s(W, s, bits)
    lo, hi = RANGE[bits]
    assert q.min() >= lo and q.max() <= hi


@pytest.mark.parametrize("bits", [4, 8])
def test_idempotent_and_error_bound(bits):
    rng = np.random.default_rng(5 + bits)
    lo, hi = RANGE[bits]
    s = _scales(bits, 64, 30 + bits).reshape(1, 64)
    t = rng.uniform(lo - 0.5, hi + 0.5, size=(128, 64))
    W = (t * s).astype(np.float32)
    q = quant.q_s(W, s, bits)
    # |W - s q| <= s/2 inside the representable interval
    err = np.abs(W.astype(np.float64) - q * s)
    assert np.all(err <= s / 2 * (1 + 1e-6))
    # idempotence: quantizing the dequantized weights returns the same codes
    W2 = (q.astype(np.float64) * s).astype(np.float32)
    assert np.array_equal(quant.q_s(W2, s, bits), q)


@pytest.mark.parametrize("bits", [4, 8])
def test_monotone_in_w(bits):
    s = np.array([[0.0123]])
    s = s.astype(np.float16).astype(np.float64) if bits == 4 else s
    lo, hi = RANGE[bits]
    W = np.linspace((lo - 3) * s[0, 0], (hi + 3) * s[0, 0], 128 * 40).astype(np.float32)
    q = np.concatenate([quant.q_s(W[i:i + 128, None], s, bits)[:, 0]
                        for i in range(0, W.size, 128)])
    assert np.all(np.diff(q.astype(int)) >= 0)
    assert q[0] == lo and q[-1] == hi


@pytest.mark.parametrize("bits", [4, 8])
def test_ties_follow_hand_table(bits):
    table = json.load(open(os.path.join(GOLD, "qs_ties.json")))["int%d" % bits]
    # scales that are exact in fp16 and bf16 and whose tie multiples are exact in fp32
    for sval in [1.0, 0.0078125, 0.375, 3.0, 0.01171875]:
        t = np.array([row[0] for row in table])
        expect = np.array([row[1] for row in table])
        W = np.zeros((128, 1), dtype=np.float32)
        W[:len(t), 0] = (t * sval).astype(np.float32)
        assert np.array_equal(W[:len(t), 0].astype(np.float64), t * sval)
        q = quant.q_s(W, np.array([[sval]]), bits)[:len(t), 0]
        assert q.tolist() == expect.tolist(), sval


def test_ties_many_scales_need_true_division():
    """Exact ties (c + 1/2) * s over many fp16 scales: RNE of the IEEE quotient.

    W = (c + 1/2) * s is exact in fp32 for fp16 s, and so is the quotient
    W / s = c + 1/2, so the only correct code is the even neighbour. A
    quantizer that multiplies by a rounded reciprocal misses some of these.
    """
    rng = np.random.default_rng(77)
    s = rng.uniform(1e-3, 1.0, size=20000).astype(np.float16).astype(np.float64)
    halves = np.arange(-8, 7) + 0.5
    t = np.resize(halves, 128)
    W = (t[:, None] * s[None, :]).astype(np.float32)
    q = quant.q_s(W, s[None, :], 4)
    expect = np.clip(2 * np.round(t / 2), -8, 7)     # nearest even integer
    assert np.array_equal(q, np.broadcast_to(expect[:, None], q.shape).astype(np.int8))


@pytest.mark.parametrize("bits", [4, 8])
def test_special_values(bits):
    lo, hi = RANGE[bits]
    W = np.zeros((128, 4), dtype=np.float32)
    W[0] = [np.nan, np.inf, -np.inf, -0.0]
    W[1] = [1.0, 1.0, 1.0, 1.0]
    s = np.array([[0.5, 0.5, 0.5, 0.0]])
    q = quant.q_s(W, s, bits)
    assert q[0].tolist() == [0, hi, lo, 0]
    assert q[1].tolist() == [2, 2, 2, 0]          # zero scale -> 0
    s_nan = np.array([[np.nan, np.inf, 0.5, 0.5]])
    q = quant.q_s(W, s_nan, bits)
    assert q[1, 0] == 0 and q[1, 1] == 0


def _py_f16(x):
    return struct.unpack("<e", struct.pack("<e", x))[0]


def _py_bf16(x):
    return float(torch.tensor([x], dtype=torch.float32).to(torch.bfloat16).item())


@pytest.mark.parametrize("bits", [4, 8])
def test_rtn_scales_brute_force(bits):
    """Per group: max |w| with Python floats, fp32 division, then 16-bit RNE."""
    rng = np.random.default_rng(100 + bits)
    W = (rng.standard_normal((384, 24)) * 0.02).astype(np.float32)
    W[:128, 3] = 0.0
    sb = quant.rtn_scales(W, bits)
    div = 7.0 if bits == 4 else 127.0
    for g in range(3):
        for n in range(24):
            amax = max(abs(float(v)) for v in W[128 * g:128 * g + 128, n])
            q32 = float(np.float32(amax / div))   # double rounding is safe for division
            want = _py_f16(q32) if bits == 4 else _py_bf16(q32)
            got = numerics.scale_bits_to_f64(sb[g, n], "f16" if bits == 4 else "bf16")
            assert got == want, (g, n)


@pytest.mark.parametrize("bits", [4, 8])
def test_rtn_largest_code_hits_range_end(bits):
    W = (np.random.default_rng(9).standard_normal((1280, 64)) * 0.02).astype(np.float32)
    W[128:256, 5] = 0.0                                  # an all-zero group
    q, sb = quant.rtn_quantize(W, bits)
    amax = np.abs(q.astype(int)).reshape(10, 128, 64).max(axis=1)
    want = 7 if bits == 4 else 127
    zero = np.abs(W).reshape(10, 128, 64).max(axis=1) == 0
    assert np.all(amax[~zero] == want)
    assert np.all(amax[zero] == 0)
    sv = numerics.scale_bits_to_f64(sb, "f16" if bits == 4 else "bf16")
    assert np.all(sv[zero] == 0)
    # RTN never produces the asymmetric end of the INT4 range
    assert q.min() >= -want


def test_rtn_nan_counts_as_zero():
    W = np.zeros((128, 2), dtype=np.float32)
    W[:, 0] = 0.07
    W[5, 0] = np.nan
    W[:, 1] = np.nan
    sb = quant.rtn_scales(W, 4)
    assert numerics.f16_to_f64(sb[0, 0]) == _py_f16(float(np.float32(np.float32(0.07) / np.float32(7.0))))
    assert numerics.f16_to_f64(sb[0, 1]) == 0.0
