"""GPU parity for the fp16-activation GEMMs and dense dequantization.

fp16 activations (the pages serve the INT4 target with FP16 activations:
adaptfm-quant-dflash README, Stage 2) run the same kernels with the fp16
matrix instruction; parity is the acceptance bound against the oracle's
float64 product with fp16-decoded x, bit-exact where the result is exact
(identity probe: x = I_K returns fp16(s * q)). Dequantization (the dense
s (.) W_q of the QAD paragraph) is bit-exact against the oracle.
"""

import numpy as np
import pytest
import torch

import int8_group_quantized_amd as q
from oracle import gemm, numerics, quant
import workloads
from gpu_helpers import Guarded, GuardedWorkspace, guarded_gemm as _call, dev_f16, dev_f32, dev_i8, dev_scales, host_u16

pytestmark = pytest.mark.gpu

SDT = {4: "f16", 8: "bf16"}


def _inputs(bits, M, K, N, seed, xstd=1.0):
    x = workloads.activations(M, K, seed, std=xstd, dtype="f16")
    c = workloads.codes(K, N, bits, seed + 1)
    s = workloads.scales(K // 128, N, SDT[bits], seed + 2)
    return x, c, s




def _run(bits, x, c, s, N, plan=None):
    pg = q.prepack(dev_i8(c), bits)
    return numerics.f16_to_f64(_call(dev_f16(x), pg, dev_scales(s, SDT[bits]), bits, N, plan=plan,
                                     what="plan %s" % (plan,)))


def _close(got, ref, what=""):
    ok = gemm.within_tolerance(got, ref)
    assert ok.all(), "%s: %d of %d outside tolerance" % (what, (~ok).sum(), ok.size)


def _ref(bits, x, c, s):
    return gemm.gemm_ref(x, c, s, SDT[bits], x_dtype="f16")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M,K,N", [(1, 256, 512), (3, 896, 592), (16, 1280, 272), (7, 384, 48)])
def test_small_shapes_plans(bits, M, K, N):
    x, c, s = _inputs(bits, M, K, N, 300 + M + K)
    ref = _ref(bits, x, c, s)
    first = None
    for plan in [None, (1, 1, 1), (1, 4, 1), (2, 4, 3), (4, 1, 2), (1, 8, 2)]:
        if plan is not None and plan[2] > K // 128:
            continue                      # more K-splits than groups: rejected by design
        got = _run(bits, x, c, s, N, plan)
        _close(got, ref, "M=%d K=%d N=%d plan %s" % (M, K, N, plan))
        if plan is None:
            first = got
    assert np.array_equal(first, _run(bits, x, c, s, N))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M,K,N", [(17, 128, 16), (129, 896, 592), (300, 384, 272),
                                   (8190, 256, 2080)])
def test_prefill_shapes(bits, M, K, N):
    x, c, s = _inputs(bits, M, K, N, 7 * M + N + 1)
    _close(_run(bits, x, c, s, N), _ref(bits, x, c, s), "prefill M=%d" % M)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("K", [256, 2560])
def test_identity_probe_bit_exact(bits, K):
    N = 64
    _, c, s = _inputs(bits, 1, K, N, 40 + K)
    eye = np.where(np.eye(K, dtype=bool), np.uint16(0x3C00), np.uint16(0))
    pg = q.prepack(dev_i8(c), bits)
    got = _call(dev_f16(eye), pg, dev_scales(s, SDT[bits]), bits, N)
    want = quant.dequant_bits(c, s, SDT[bits], "f16")
    assert np.array_equal(got, want), int((got != want).sum())


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M", [1, 5, 16, 200])
def test_zero_codes_scales_and_activations(bits, M):
    """Exact zeros for zero scales and zero x on every path, and for an
    all-zero code column at M <= 16 (the INT4 offset 1032 * sum x is the same
    matrix-core chain as the code product there) and for INT8 codes; at
    M > 16 an INT4 zero column keeps only the fp32 rounding of the offset."""
    K, N = 640, 320
    x, c, s = _inputs(bits, M, K, N, 61 + M)
    c[:, :16] = 0
    s = s.copy()
    s[:, 16:32] = 0
    got = _run(bits, x, c, s, N)
    assert np.all(got[:, 16:32] == 0)
    if bits == 8 or M <= 16:
        assert np.all(got[:, :16] == 0)
        for plan in ([(1, 1, 1), (1, 4, 1), (2, 4, 3), (1, 1, 5)] if M <= 16 else []):
            assert np.all(_run(bits, x, c, s, N, plan)[:, :16] == 0), plan
    else:
        xs = numerics.f16_to_f64(x)
        sv = numerics.scale_bits_to_f64(s, SDT[bits])
        gsum = np.abs(xs).reshape(M, K // 128, 128).sum(axis=2)
        bound = 8 * 2.0 ** -24 * 1032 * gsum @ np.abs(sv[:, :16])   # fp16 codes carry 1032 + q
        assert np.all(np.abs(got[:, :16]) <= bound)
    _close(got, _ref(bits, x, c, s))
    assert np.all(_run(bits, np.zeros_like(x), c, s, N) == 0)


CASES = [(2, 0), (2, 1), (3, 2), (4, 2), (5, 0), (5, 1)]


@pytest.mark.parametrize("cfg,si", CASES)
def test_workload_shapes_with_f16_activations(cfg, si):
    """The decode, verification, drafter and prefill shapes with fp16 x."""
    w = workloads.WORKLOADS[cfg]
    K, N = w["shapes"][si]
    bits, M = w["bits"], w["M"]
    W = workloads.weights(K, N, workloads.seed_for(cfg, si, 0))
    x = workloads.activations(M, K, workloads.seed_for(cfg, si, 1), dtype="f16")
    sb = quant.rtn_scales(W, bits)
    codes = quant.q_s(W, numerics.scale_bits_to_f64(sb, SDT[bits]), bits)
    print("fp16 workload config %d shape %d: M=%d K=%d N=%d" % (cfg, si, M, K, N), flush=True)
    pg = q.pack_to_grid(dev_f32(W), dev_scales(sb, SDT[bits]), bits)
    got_bits = _call(dev_f16(x), pg, dev_scales(sb, SDT[bits]), bits, N, what="cfg %d" % cfg)
    # every output, rms over the whole [M, N] output (M = 8192 included)
    _close(numerics.f16_to_f64(got_bits), _ref(bits, x, codes, sb), "cfg %d shape %d" % (cfg, si))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("s_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("K,N", [(128, 16), (384, 272), (256, 2000), (640, 4096)])
def test_dequant_bit_exact(bits, s_dtype, out_dtype, K, N):
    c = workloads.codes(K, N, bits, K + N)
    c[::5, ::3] = -8 if bits == 4 else -127
    s = workloads.scales(K // 128, N, s_dtype, K + N + 1)
    s[0, :3] = np.array([0x7BFF, 0x0001, 0], dtype=np.uint16) if s_dtype == "f16" \
        else np.array([0x7F7F, 0x0001, 0], dtype=np.uint16)
    pg = q.prepack(dev_i8(c), bits)
    dt = torch.bfloat16 if out_dtype == "bf16" else torch.float16
    out = Guarded((K, N), dt)                   # NaN-poisoned: s * q is never NaN here
    q.dequant(pg, dev_scales(s, s_dtype), bits, K, N, out=out.t)
    got = host_u16(out.check())
    want = quant.dequant_bits(c, s, s_dtype, out_dtype)
    assert np.array_equal(got, want), int((got != want).sum())


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("K,N", [(1 << 20, 16), (128, 1 << 20)])
def test_dequant_maximum_extents(bits, K, N):
    """The largest K and N the boundary accepts (2^20), bit-exact."""
    c = workloads.codes(K, N, bits, 17 + (K >> 7))
    s = workloads.scales(K // 128, N, SDT[bits], 18 + (K >> 7))
    pg = q.prepack(dev_i8(c), bits)
    out = Guarded((K, N), torch.bfloat16)
    q.dequant(pg, dev_scales(s, SDT[bits]), bits, K, N, out=out.t)
    got = host_u16(out.check())
    assert np.array_equal(got, quant.dequant_bits(c, s, SDT[bits], "bf16"))


@pytest.mark.parametrize("bits", [4, 8])
def test_dequant_full_size(bits):
    """The decode gate/up weight (2560 x 19456) through Q_s and back."""
    K, N = 2560, 19456
    W = workloads.weights(K, N, workloads.seed_for(2, 0, 0))
    sb = quant.rtn_scales(W, bits)
    codes = quant.q_s(W, numerics.scale_bits_to_f64(sb, SDT[bits]), bits)
    pg = q.pack_to_grid(dev_f32(W), dev_scales(sb, SDT[bits]), bits)
    out = Guarded((K, N), torch.bfloat16)
    q.dequant(pg, dev_scales(sb, SDT[bits]), bits, K, N, out=out.t)
    got = host_u16(out.check())
    assert np.array_equal(got, quant.dequant_bits(codes, sb, SDT[bits], "bf16"))
