"""GPU parity for the fixed-grid fake quantizer (QAD forward pass) and its
straight-through backward.

The forward is bit-exact against the oracle's quant.fake_quant for every
weight, scale and output format, on crafted cases (exact ties, clamp ends,
zero scales, NaN / infinite / subnormal weights) and at full size; it also
agrees with pack_to_grid followed by dequant (two independent GPU paths to
s (.) Q_s(W)). The backward is the identity on the gradient (the straight-
through estimator of the QAD paragraph). Outputs are NaN-poisoned (the
fake quantizer never produces NaN: a NaN weight maps to code 0) between
canary bands, so an unwritten element or a stray store fails the test.
"""

import numpy as np
import pytest
import torch

import int8_group_quantized_amd as q
from oracle import numerics, quant
import workloads
from gpu_helpers import DEV, Guarded, dev_bf16, dev_f32, dev_scales, host_u16

pytestmark = pytest.mark.gpu

SDT = {4: "f16", 8: "bf16"}
TDT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _crafted(bits, K=256, N=64, seed=5):
    W = workloads.weights(K, N, seed)
    sb = quant.rtn_scales(W, bits)
    s = numerics.scale_bits_to_f64(sb, SDT[bits]).astype(np.float32)
    lo, hi = quant.RANGE[bits]
    t = np.arange(lo - 1, hi + 2, dtype=np.float32) + np.float32(0.5)
    ties = np.unique(np.r_[t[:8], t[-8:], t[len(t) // 2 - 8: len(t) // 2 + 8]])   # ends + middle
    W[1, :len(ties)] = ties * s[0, :len(ties)]               # exact ties and clamp ends
    W[0, :8] = [np.nan, np.inf, -np.inf, -0.0, 1e-40, -1e-45, 3e38, -3e38]
    sb[1, 3:6] = 0                                           # zero scales
    return W, sb


def _fq(Wd, sd, bits, out_dt):
    """fake_quant into a NaN-poisoned, guarded output."""
    g = Guarded(tuple(Wd.shape), TDT[out_dt])
    q.fake_quant(Wd, sd, bits, out=g.t)
    return g.check("fake quant")


def _gpu(W, w_dt, sb, bits, out_dt):
    Wd = dev_f32(W) if w_dt == "f32" else dev_bf16(workloads.to_bf16_bits(W))
    out = _fq(Wd, dev_scales(sb, SDT[bits]), bits, out_dt)
    if out_dt == "f32":
        return out.cpu().numpy()
    return host_u16(out)


def _oracle(W, w_dt, sb, bits, out_dt):
    if w_dt == "bf16":                     # the kernel reads the bf16 weights exactly
        W = numerics.bf16_to_f64(workloads.to_bf16_bits(W)).astype(np.float32)
    return quant.fake_quant(W, sb, SDT[bits], bits, out_dt)


def _same(a, b):
    if a.dtype == np.float32:
        return np.array_equal(a.view(np.uint32), b.astype(np.float32).view(np.uint32))
    return np.array_equal(a, b)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("w_dt", ["f32", "bf16"])
@pytest.mark.parametrize("out_dt", ["bf16", "f16", "f32"])
def test_crafted_bit_exact(bits, w_dt, out_dt):
    W, sb = _crafted(bits)
    got = _gpu(W, w_dt, sb, bits, out_dt)
    want = _oracle(W, w_dt, sb, bits, out_dt)
    assert _same(got, want), int((got != want).sum())


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("K,N", [(128, 16), (384, 272), (1280, 2000)])
def test_shapes_and_other_scale_dtype(bits, K, N):
    W = workloads.weights(K, N, K + N, dist="student_t")
    other = "bf16" if bits == 4 else "f16"
    sb = workloads.scales(K // 128, N, other, K)
    Wd = dev_f32(W)
    got = host_u16(_fq(Wd, dev_scales(sb, other), bits, "bf16"))
    want = quant.fake_quant(W, sb, other, bits, "bf16")
    assert np.array_equal(got, want)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("K,N", [(1 << 20, 16), (128, 1 << 20)])
def test_maximum_extents(bits, K, N):
    """The largest K and N the boundary accepts (2^20), bit-exact."""
    W = workloads.weights(K, N, 13 + (K >> 7))
    sb = quant.rtn_scales(W, bits)
    got = host_u16(_fq(dev_f32(W), dev_scales(sb, SDT[bits]), bits, "bf16"))
    assert np.array_equal(got, quant.fake_quant(W, sb, SDT[bits], bits, "bf16"))


@pytest.mark.parametrize("bits", [4, 8])
def test_equals_pack_then_dequant(bits):
    K, N = 2560, 3584
    W = workloads.weights(K, N, 77)
    Wd = dev_f32(W)
    s = q.rtn_scales(Wd, bits)
    fq = _fq(Wd, s, bits, "bf16")
    g = Guarded((K, N), torch.bfloat16)
    q.dequant(q.pack_to_grid(Wd, s, bits), s, bits, K, N, out=g.t)
    dq = g.check("dequant")
    assert torch.equal(fq.view(torch.int16), dq.view(torch.int16))


def test_full_size_gate_up():
    K, N = 2560, 19456
    W = workloads.weights(K, N, workloads.seed_for(2, 0, 0))
    sb = quant.rtn_scales(W, 4)
    got = host_u16(_fq(dev_f32(W), dev_scales(sb, "f16"), 4, "bf16"))
    assert np.array_equal(got, quant.fake_quant(W, sb, "f16", 4, "bf16"))


def test_straight_through_backward():
    K, N = 256, 48
    W = workloads.weights(K, N, 3)
    Wd = dev_f32(W).requires_grad_(True)
    s = q.rtn_scales(Wd.detach(), 4)
    y = q.FakeQuantSTE.apply(Wd, s, 4)
    G = torch.randn(K, N, device=DEV)
    (y * G).sum().backward()
    assert torch.equal(Wd.grad, G)
    assert torch.equal(y.detach().cpu(), torch.from_numpy(quant.fake_quant(W, host_u16(s), "f16", 4, "f32")))
