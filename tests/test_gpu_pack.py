"""GPU parity for the integer/byte side of the path: RTN scales, Q_s codes,
packed bytes, unpack and prepack. The bar is bit-exact against the oracle.

Every output is written into a buffer between canary bands, twice, under two
different poison bytes (float scales under NaN): both results must agree, so
no byte is left unwritten, and no store lands outside the buffer.

Cases: small shapes spanning several tiles with ragged tails (N not a
multiple of the 64- or 256-column spans the kernels use), fp32 and bf16
weights, crafted ties / clamp ends / zero groups / NaN / infinities /
subnormals, and the full-size shapes of the decode, verification and drafter
workloads (hidden 2560: gate/up 2560x19456, down 9728x2560, QKV 2560x3584).
"""

import numpy as np
import pytest
import torch

import int8_group_quantized_amd as q
from oracle import layout, numerics, quant
import workloads
from gpu_helpers import (Guarded, dev_bf16, dev_f32, dev_i8, dev_scales, host_i8, host_u16, host_u8,
                         written_twice)

pytestmark = pytest.mark.gpu

SDT = {4: "f16", 8: "bf16"}
SMALL = [(128, 16), (256, 512), (384, 48), (896, 592)]


def _weights_for(K, N, seed, wdt, dist="normal"):
    W = workloads.weights(K, N, seed, dist=dist)
    if wdt == "bf16":
        bits = workloads.to_bf16_bits(W)
        return dev_bf16(bits), numerics.bf16_to_f64(bits).astype(np.float32)
    return dev_f32(W), W


def _rtn(Wd, bits):
    K, N = Wd.shape
    g = Guarded((K // 128, N), torch.float16 if bits == 4 else torch.bfloat16)
    q.rtn_scales(Wd, bits, out=g.t)
    return g.check("rtn scales")


def _pack(Wd, sd, bits):
    K, N = Wd.shape
    return written_twice(lambda o: q.pack_to_grid(Wd, sd, bits, out=o),
                         (q.packed_bytes(bits, K, N),), torch.uint8, "pack_to_grid")


def _unpack(pg, K, N, bits):
    return written_twice(lambda o: q.unpack(pg, K, N, bits, out=o), (K, N), torch.int8, "unpack")


def _prepack(cd, bits):
    K, N = cd.shape
    return written_twice(lambda o: q.prepack(cd, bits, out=o), (q.packed_bytes(bits, K, N),),
                         torch.uint8, "prepack")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("K,N", SMALL)
@pytest.mark.parametrize("wdt", ["f32", "bf16"])
def test_rtn_pack_unpack_small(bits, K, N, wdt):
    Wd, Wf = _weights_for(K, N, 7 * K + N, wdt)
    sb = quant.rtn_scales(Wf, bits)
    codes = quant.q_s(Wf, numerics.scale_bits_to_f64(sb, SDT[bits]), bits)
    ref_packed = layout.pack(codes, bits)

    sg = _rtn(Wd, bits)
    assert np.array_equal(host_u16(sg), sb)
    pg = _pack(Wd, sg, bits)
    assert np.array_equal(host_u8(pg), ref_packed)
    cg = _unpack(pg, K, N, bits)
    assert np.array_equal(host_i8(cg), codes)
    assert np.array_equal(host_u8(_prepack(cg, bits)), ref_packed)


@pytest.mark.parametrize("bits", [4, 8])
def test_prepack_full_code_range(bits):
    K, N = 512, 80
    lo, hi = (-8, 7) if bits == 4 else (-128, 127)
    c = workloads.codes(K, N, bits, 5, lo=lo, hi=hi)
    pg = _prepack(dev_i8(c), bits)
    assert np.array_equal(host_u8(pg), layout.pack(c, bits))
    assert np.array_equal(host_i8(_unpack(pg, K, N, bits)), c)


def _crafted(bits):
    """Ties, clamp ends, zero scales, NaN/Inf and subnormal weights."""
    K, N = 256, 32
    lo, hi = quant.RANGE[bits]
    rng = np.random.default_rng(11 + bits)
    s = workloads.scales(K // 128, N, SDT[bits], 12 + bits)
    sv = numerics.scale_bits_to_f64(s, SDT[bits])
    t = rng.integers(2 * lo - 4, 2 * hi + 5, size=(K, N)) / 2.0     # many exact halves
    W = (t * np.repeat(sv, 128, axis=0)).astype(np.float32)
    W[0, :8] = [np.nan, np.inf, -np.inf, -0.0, 1e-40, -1e-45, 3e38, -3e38]
    W[1, :4] = (np.array([lo - 0.4, hi + 0.4, lo - 0.6, hi + 0.6]) * sv[0, :4]).astype(np.float32)
    s = s.copy()
    s[0, 5] = 0                          # a zero scale
    s[1, 6] = 0x0001                     # the smallest subnormal 16-bit scale
    W[128:, 7] = 0.0                     # an all-zero group
    return W, s


@pytest.mark.parametrize("bits", [4, 8])
def test_pack_crafted_cases(bits):
    W, s = _crafted(bits)
    K, N = W.shape
    codes = quant.q_s(W, numerics.scale_bits_to_f64(s, SDT[bits]), bits)
    assert codes.min() == quant.RANGE[bits][0]          # the clamp end is exercised
    pg = _pack(dev_f32(W), dev_scales(s, SDT[bits]), bits)
    got = host_i8(_unpack(pg, K, N, bits))
    bad = np.argwhere(got != codes)
    assert bad.size == 0, [(int(k), int(n), W[k, n], int(got[k, n]), int(codes[k, n]))
                           for k, n in bad[:10]]
    assert np.array_equal(host_u8(pg), layout.pack(codes, bits))


@pytest.mark.parametrize("bits", [4, 8])
def test_rtn_crafted(bits):
    K, N = 256, 48
    W = workloads.weights(K, N, 31, dist="student_t")
    W[:128, 3] = 0.0
    W[5, 4] = np.nan
    W[7, 9] = 1e-40
    sb = quant.rtn_scales(W, bits)
    assert np.array_equal(host_u16(_rtn(dev_f32(W), bits)), sb)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("K,N", [(1 << 20, 16), (128, 1 << 20)])
def test_maximum_extents(bits, K, N):
    """The largest K and N the boundary accepts (2^20): 8,192 groups of one
    column block, and 65,536 column blocks of one group; codes, scales and
    packed bytes bit-exact, unpack and prepack inverse."""
    Wd, Wf = _weights_for(K, N, 11 + (K >> 7), "f32")
    sb = quant.rtn_scales(Wf, bits)
    codes = quant.q_s(Wf, numerics.scale_bits_to_f64(sb, SDT[bits]), bits)
    sg = _rtn(Wd, bits)
    assert np.array_equal(host_u16(sg), sb)
    pg = _pack(Wd, sg, bits)
    assert np.array_equal(host_u8(pg), layout.pack(codes, bits))
    cg = _unpack(pg, K, N, bits)
    assert np.array_equal(host_i8(cg), codes)
    assert torch.equal(_prepack(cg, bits), pg)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("K,N", [(2560, 19456), (9728, 2560), (2560, 3584)])
def test_full_size_codes(bits, K, N):
    seed = workloads.seed_for(3 if bits == 4 else 4, [(2560, 19456), (9728, 2560),
                                                      (2560, 3584)].index((K, N)), 0)
    W = workloads.weights(K, N, seed)
    sb = quant.rtn_scales(W, bits)
    codes = quant.q_s(W, numerics.scale_bits_to_f64(sb, SDT[bits]), bits)
    Wd = dev_f32(W)
    sg = _rtn(Wd, bits)
    assert np.array_equal(host_u16(sg), sb)
    pg = _pack(Wd, sg, bits)
    assert np.array_equal(host_u8(pg), layout.pack(codes, bits))
    cg = _unpack(pg, K, N, bits)
    assert np.array_equal(host_i8(cg), codes)
    # prepack of the GPU's own unpacked codes reproduces its packed bytes
    assert torch.equal(_prepack(cg, bits), pg)
