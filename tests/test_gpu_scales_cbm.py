"""Column-block-major scales (qg_prepack_scales): the prepacked order equals
the oracle's element-by-element statement of it, every GEMM path gives
bit-identical outputs with the prepacked scales and with the logical ones
(the order changes where a scale is read, never the arithmetic), and each
prepacked-scale result also meets the acceptance bound against the oracle's
float64 product directly. Outputs and workspaces are NaN-poisoned between
canary bands."""

import numpy as np
import pytest
import torch

import int8_group_quantized_amd as q
from oracle import gemm, layout, numerics
import workloads
from gpu_helpers import Guarded, GuardedWorkspace, dev_bf16, dev_i8, dev_scales, guarded_gemm, host_u16

pytestmark = pytest.mark.gpu

SDT = {4: "f16", 8: "bf16"}


@pytest.mark.parametrize("sdt", ["f16", "bf16"])
@pytest.mark.parametrize("K,N", [(128, 16), (256, 512), (2560, 3584), (9728, 2560), (384, 48)])
def test_prepack_matches_oracle(sdt, K, N):
    print("prepack scales: K=%d N=%d %s" % (K, N, sdt), flush=True)
    s = workloads.scales(K // 128, N, sdt, K + N)
    sd = dev_scales(s, sdt)
    g = Guarded((N // 16, K // 128, 16), sd.dtype)
    q.prepack_scales(sd, out=g.t)
    got = host_u16(g.check("prepack scales")).reshape(-1)
    assert np.array_equal(got, layout.scales_cbm(s))


def _pair(bits, M, K, N, seed, plan=None, f16=False):
    x = workloads.activations(M, K, seed, dtype="f16" if f16 else "bf16")
    c = workloads.codes(K, N, bits, seed + 1)
    s = workloads.scales(K // 128, N, SDT[bits], seed + 2)
    pg = q.prepack(dev_i8(c), bits)
    xs = torch.from_numpy(x.view(np.int16)).view(torch.float16 if f16 else torch.bfloat16).cuda()
    sd = dev_scales(s, SDT[bits])
    ref = guarded_gemm(xs, pg, sd, bits, N, plan=plan, what="logical scales")
    got = guarded_gemm(xs, pg, q.prepack_scales(sd), bits, N, plan=plan, cbm=True,
                       what="column-block-major scales")
    act = "f16" if f16 else "bf16"
    exact = gemm.gemm_ref(x, c, s, SDT[bits], x_dtype=act)
    ok = gemm.within_tolerance(numerics.act_to_f64(got, act), exact)
    assert ok.all(), "%d of %d outside tolerance" % ((~ok).sum(), ok.size)
    return ref, got


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M,K,N", [(1, 256, 512), (1, 2560, 19456), (1, 9728, 2560), (5, 896, 592),
                                   (16, 2560, 3584), (16, 9728, 2560), (17, 640, 272),
                                   (300, 1280, 336)])
def test_gemm_bit_identical(bits, M, K, N):
    print("cbm gemm: bits=%d M=%d K=%d N=%d" % (bits, M, K, N), flush=True)
    ref, got = _pair(bits, M, K, N, 300 + M)
    assert np.array_equal(ref, got)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("plan", [(1, 1, 3), (2, 4, 1), (4, 1, 2), (1, 8, 2)])
def test_gemm_bit_identical_explicit_plans(bits, plan):
    print("cbm gemm plan %s bits=%d" % (plan, bits), flush=True)
    ref, got = _pair(bits, 3, 1152, 592, 400, plan=plan)
    assert np.array_equal(ref, got)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M", [1, 64])
def test_fp16_activations_bit_identical(bits, M):
    ref, got = _pair(bits, M, 768, 208, 500 + M, f16=True)
    assert np.array_equal(ref, got)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M", [16, 40])
def test_grouped_bit_identical(bits, M):
    K = 1280
    xh = workloads.activations(M, K, 600 + M)
    x = dev_bf16(xh)
    items, items_cbm, host = [], [], []
    for i, N in enumerate((1024, 512, 3584)):
        c = workloads.codes(K, N, bits, 610 + i)
        s = workloads.scales(K // 128, N, SDT[bits], 620 + i)
        host.append((c, s, N))
        sd = dev_scales(s, SDT[bits])
        pg = q.prepack(dev_i8(c), bits)
        items.append((pg, sd, N))
        items_cbm.append((pg, q.prepack_scales(sd), N))
    def run(its, cbm):
        outs = [Guarded((M, N), torch.bfloat16) for _, _, N in its]
        ws = GuardedWorkspace(q.grouped_workspace_bytes(bits, M, K, its))
        q.qgemm_grouped(x, its, bits, outs=[o.t for o in outs], ws=ws.t, scales_cbm=cbm)
        res = [host_u16(o.check()) for o in outs]
        ws.check()
        return res

    ref = run(items, False)
    got = run(items_cbm, True)
    for r, g, (c, s, N) in zip(ref, got, host):
        assert np.array_equal(r, g)
        ok = gemm.within_tolerance(numerics.bf16_to_f64(g), gemm.gemm_ref(xh, c, s, SDT[bits]))
        assert ok.all(), (N, int((~ok).sum()))
