"""qgemm_w4a16_noalloc: the W4A16 GEMM for callers that cannot allocate
device memory, with its workspace in the library's fixed per-device scratch.

Called through the C ABI on two calls in a row, the second with a smaller
input, and checked against qgemm_w4a16 (same kernels and plan, its own
workspace) bit for bit, and against the oracle's float64 product within the
acceptance bound. The cases use the scratch for split-K partials (M <= 16
with long K), for the prefill INT4 offsets (M > 16), and not at all (decode
shapes whose plan needs no workspace).
"""

import numpy as np
import pytest
import torch

import int8_group_quantized_amd as q
from oracle import gemm, numerics
import workloads
from gpu_helpers import Guarded, GuardedWorkspace, dev_bf16, dev_i8, dev_scales, host_u16

pytestmark = pytest.mark.gpu

QG_F16 = 1

SEQUENCES = [
    [(16, 9728, 2560), (5, 6400, 256)],        # split-K partials, then fewer of them
    [(2048, 9728, 2560), (300, 1280, 336)],    # prefill offsets, then a smaller prefill
    [(300, 1280, 336), (1, 2560, 19456)],      # prefill, then a decode call (no scratch)
    [(1, 9728, 2560), (3, 896, 592)],          # small shapes
]


def _case(M, K, N, seed):
    x = workloads.activations(M, K, seed)
    c = workloads.codes(K, N, 4, seed + 1)
    s = workloads.scales(K // 128, N, "f16", seed + 2)
    return x, c, s


def _noalloc(xd, pg, sd, N):
    M, K = xd.shape
    out = Guarded((M, N), torch.bfloat16)
    st = torch.cuda.current_stream().cuda_stream
    code = q.lib().qgemm_w4a16_noalloc(xd.data_ptr(), pg.data_ptr(), sd.data_ptr(), QG_F16,
                                       out.t.data_ptr(), M, K, N, st)
    assert code == 0, code
    return host_u16(out.check("noalloc"))


def _with_workspace(xd, pg, sd, N):
    M, K = xd.shape
    out = Guarded((M, N), torch.bfloat16)
    ws = GuardedWorkspace(q.workspace_bytes(4, M, K, N))
    q.qgemm(xd, pg, sd, 4, N, out=out.t, ws=ws.t)
    ws.check()
    return host_u16(out.check("qgemm_w4a16"))


@pytest.mark.parametrize("seq", range(len(SEQUENCES)))
def test_two_calls_match_the_workspace_entry_point(seq):
    for i, (M, K, N) in enumerate(SEQUENCES[seq]):
        print("noalloc sequence %d call %d: M=%d K=%d N=%d" % (seq, i, M, K, N), flush=True)
        x, c, s = _case(M, K, N, 5000 + 100 * seq + 10 * i)
        xd, pg, sd = dev_bf16(x), q.prepack(dev_i8(c), 4), dev_scales(s, "f16")
        got = _noalloc(xd, pg, sd, N)
        want = _with_workspace(xd, pg, sd, N)
        assert np.array_equal(got, want), int((got != want).sum())
        ok = gemm.within_tolerance(numerics.bf16_to_f64(got), gemm.gemm_ref(x, c, s, "f16"))
        assert ok.all(), int((~ok).sum())
