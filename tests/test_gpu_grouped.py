"""GPU parity for the grouped launch: several GEMMs sharing x (the K/V
projections of every drafter layer computed from one input, Qwen3.5-4B-
DFlash-W8A16 model card, "Required vLLM patches": the fused K+V buffer
across the 5 layers) in one kernel launch. Each item must meet the
acceptance bound against the oracle's plain per-item product; a group of
one is bit-identical to the single call; repeated calls are bit-identical.
Every item's output is NaN-poisoned between canary bands and the shared
workspace's partials are NaN-poisoned before a canary band, so an item a
launch leaves unwritten, or a store into a neighbour, fails the test.
"""

import numpy as np
import pytest
import torch

import int8_group_quantized_amd as q
from oracle import gemm, numerics
import workloads
from gpu_helpers import Guarded, GuardedWorkspace, dev_bf16, dev_f16, dev_i8, dev_scales, host_u16

pytestmark = pytest.mark.gpu

SDT = {4: "f16", 8: "bf16"}


def _group(bits, M, K, Ns, seed, act="bf16"):
    x = workloads.activations(M, K, seed, dtype=act)
    items = []
    for i, N in enumerate(Ns):
        c = workloads.codes(K, N, bits, seed + 10 * i + 1)
        s = workloads.scales(K // 128, N, SDT[bits], seed + 10 * i + 2)
        items.append((c, s, N))
    return x, items


def _dev(bits, items):
    return [(q.prepack(dev_i8(c), bits), dev_scales(s, SDT[bits]), N) for c, s, N in items]


def _decode(t, act):
    return numerics.act_to_f64(host_u16(t), act)


def _grouped(xd, dw, bits, scales_cbm=False):
    """One grouped launch into guarded, poisoned outputs and workspace."""
    M, K = xd.shape
    outs = [Guarded((M, N), xd.dtype) for _, _, N in dw]
    ws = GuardedWorkspace(q.grouped_workspace_bytes(bits, M, K, dw))
    q.qgemm_grouped(xd, dw, bits, outs=[o.t for o in outs], ws=ws.t, scales_cbm=scales_cbm)
    res = [o.check("item %d" % i) for i, o in enumerate(outs)]
    ws.check("grouped")
    return res


# The cases reach every tiling the library's plans give a group: one row with
# narrow and with wide summed N (one or two column blocks per wavefront),
# 2-16 rows with wide N, long K (split across workgroups) and the rest, and
# more than 16 rows (the prefill kernel, one launch per item).
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("M,K,Ns", [(1, 2560, [1024] * 5), (16, 2560, [1024] * 5),
                                    (3, 896, [592, 16, 272]), (16, 9728, [2560, 512]),
                                    (7, 384, [48] * 16), (40, 512, [96, 208]),
                                    (1, 2560, [8192, 8192, 4096]), (16, 9728, [1024, 1536]),
                                    (4, 2560, [8192, 8192])])
def test_items_match_the_oracle(bits, act, M, K, Ns):
    x, items = _group(bits, M, K, Ns, 500 + M + len(Ns), act)
    xd = dev_bf16(x) if act == "bf16" else dev_f16(x)
    dw = _dev(bits, items)
    outs = _grouped(xd, dw, bits)
    for (c, s, N), o in zip(items, outs):
        ref = gemm.gemm_ref(x, c, s, SDT[bits], x_dtype=act)
        ok = gemm.within_tolerance(_decode(o, act), ref)
        assert ok.all(), (N, int((~ok).sum()))
    again = _grouped(xd, dw, bits)
    for o, a in zip(outs, again):
        assert torch.equal(o.view(torch.int16), a.view(torch.int16))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M,K,N", [(1, 2560, 19456), (16, 9728, 2560), (5, 640, 320),
                                   (16, 2560, 19456)])
def test_group_of_one_is_the_single_call(bits, M, K, N):
    x, items = _group(bits, M, K, [N], 900 + M)
    dw = _dev(bits, items)
    one = _grouped(dev_bf16(x), dw, bits)[0]
    out = Guarded((M, N), torch.bfloat16)
    q.qgemm(dev_bf16(x), dw[0][0], dw[0][1], bits, N, out=out.t)
    single = out.check("single")
    assert torch.equal(one.view(torch.int16), single.view(torch.int16))
