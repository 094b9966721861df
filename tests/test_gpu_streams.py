"""Calls on different streams of one device, each stream with its own
workspace, may run at the same time: every entry point keeps its state
(split-K partials, arrival counters, chunk results) in the workspace it is
given, so concurrent calls must give the bits the same calls give one at a
time. Cases: two split-K GEMMs (INT4 and INT8 codes), the attention's
chunked merges (one-head kernel and shared K/V stream) and a grouped GEMM,
all interleaved on separate default-priority streams, each stream running
its calls back to back on one workspace (its counters left at zero after
every call). Every concurrent output is compared bit for bit with the same
call made alone on the current stream, and that one against the oracle.
"""

import numpy as np
import pytest
import torch

import int8_group_quantized_amd as q
from oracle import attention, gemm, numerics
import workloads
from gpu_helpers import DEV, Guarded, GuardedWorkspace, dev_bf16, dev_i8, dev_scales, host_u16

pytestmark = pytest.mark.gpu

SDT = {4: "f16", 8: "bf16"}
D = 128
REPEATS = 12


class _Gemm:
    def __init__(self, bits, M, K, N, plan, seed):
        self.bits, self.N, self.plan = bits, N, plan
        self.x = workloads.activations(M, K, seed)
        self.c = workloads.codes(K, N, bits, seed + 1)
        self.s = workloads.scales(K // 128, N, SDT[bits], seed + 2)
        self.xd = dev_bf16(self.x)
        self.pg = q.prepack(dev_i8(self.c), bits)
        self.sd = dev_scales(self.s, SDT[bits])
        self.shape, self.dtype = (M, N), torch.bfloat16
        self.ws_bytes = q.workspace_bytes(bits, M, K, N, plan)
        self.what = "gemm W%d M=%d K=%d N=%d plan %s" % (bits, M, K, N, plan)

    def launch(self, out, ws):
        q.qgemm(self.xd, self.pg, self.sd, self.bits, self.N, out=out, plan=self.plan, ws=ws)

    def check_ref(self, got_bits):
        ref = gemm.gemm_ref(self.x, self.c, self.s, SDT[self.bits])
        assert gemm.within_tolerance(numerics.bf16_to_f64(got_bits), ref).all(), self.what


class _Grouped:
    def __init__(self, bits, M, K, Ns, seed):
        self.bits = bits
        self.x = workloads.activations(M, K, seed)
        self.items = []
        for i, N in enumerate(Ns):
            c = workloads.codes(K, N, bits, seed + 10 * i + 1)
            s = workloads.scales(K // 128, N, SDT[bits], seed + 10 * i + 2)
            self.items.append((c, s, N))
        self.xd = dev_bf16(self.x)
        self.weights = [(q.prepack(dev_i8(c), bits), dev_scales(s, SDT[bits]), N)
                        for c, s, N in self.items]
        # the outputs one after another in one buffer, each [M, N_i] contiguous
        self.M, self.offs = M, M * np.cumsum([0] + list(Ns))
        self.shape, self.dtype = (int(self.offs[-1]),), torch.bfloat16
        self.ws_bytes = q.grouped_workspace_bytes(bits, M, K, self.weights)
        self.what = "grouped W%d M=%d K=%d N=%s" % (bits, M, K, Ns)

    def launch(self, out, ws):
        outs = [out[int(a):int(b)].view(self.M, -1) for a, b in zip(self.offs[:-1], self.offs[1:])]
        q.qgemm_grouped(self.xd, self.weights, self.bits, outs=outs, ws=ws)

    def check_ref(self, got_bits):
        for (c, s, N), a, b in zip(self.items, self.offs[:-1], self.offs[1:]):
            ref = gemm.gemm_ref(self.x, c, s, SDT[self.bits])
            got = numerics.bf16_to_f64(got_bits[int(a):int(b)].reshape(self.M, N))
            assert gemm.within_tolerance(got, ref).all(), self.what


class _Attention:
    def __init__(self, B, T, Hq, Hkv, S_max, lens, window, chunk, heads, seed):
        self.qb, self.kb, self.vb = workloads.attention_inputs(B, T, Hq, Hkv, D, S_max, seed)
        self.lens, self.T, self.S_max, self.window = lens, T, S_max, window
        self.chunk, self.heads, self.sc = chunk, heads, 1.0 / np.sqrt(D)
        self.qd, self.kd, self.vd = dev_bf16(self.qb), dev_bf16(self.kb), dev_bf16(self.vb)
        self.ld = torch.tensor(lens, dtype=torch.int32, device=DEV)
        self.shape, self.dtype = (B, T, Hq, D), torch.bfloat16
        self.ws_bytes = q.lib().qg_swa_workspace_bytes_plan(B, T, Hq, Hkv, D, S_max, window,
                                                            chunk, heads)
        self.what = "attention B=%d S=%s window=%d chunk=%d heads=%d" % (B, lens, window,
                                                                         chunk, heads)

    def launch(self, out, ws):
        q.swa_attention(self.qd, self.kd, self.vd, self.ld, self.window, self.sc,
                        chunk=self.chunk, heads=self.heads, out=out, ws=ws)

    def check_ref(self, got_bits):
        eff = [min(max(S, self.T), self.S_max) for S in self.lens]
        ref = attention.swa_attention(numerics.bf16_to_f64(self.qb), numerics.bf16_to_f64(self.kb),
                                      numerics.bf16_to_f64(self.vb), eff, self.window, self.sc)
        got = numerics.bf16_to_f64(got_bits)
        bound = 1e-2 * np.abs(ref) + 1e-3 * np.sqrt(np.mean(ref ** 2))
        assert (np.abs(got - ref) <= bound).all(), self.what


def _alone(case):
    out = Guarded(case.shape, case.dtype)
    ws = GuardedWorkspace(case.ws_bytes)
    case.launch(out.t, ws.t)
    got = host_u16(out.check(case.what))
    ws.check(case.what)
    return got


def _concurrent(cases):
    """Every case REPEATS times on a stream of its own, the launches
    interleaved across the streams; returns each case's outputs."""
    print("concurrent: " + "; ".join(c.what for c in cases), flush=True)
    streams = [torch.cuda.Stream(device=DEV) for _ in cases]
    wss = [GuardedWorkspace(c.ws_bytes) for c in cases]
    outs = [[Guarded(c.shape, c.dtype) for _ in range(REPEATS)] for c in cases]
    torch.cuda.synchronize()
    for r in range(REPEATS):
        for c, s, ws, o in zip(cases, streams, wss, outs):
            with torch.cuda.stream(s):
                c.launch(o[r].t, ws.t)
    torch.cuda.synchronize()
    for c, ws in zip(cases, wss):
        ws.check(c.what)
    return [[host_u16(g.check(c.what)) for g in o] for c, o in zip(cases, outs)]


def _same_as_alone(cases):
    alone = [_alone(c) for c in cases]
    for c, a in zip(cases, alone):
        c.check_ref(a)
    for c, a, got in zip(cases, alone, _concurrent(cases)):
        for r, g in enumerate(got):
            assert np.array_equal(g, a), "%s: call %d on its stream differs" % (c.what, r)


def test_split_gemms_on_two_streams():
    # K split across workgroups: partials and arrival counters in each
    # stream's own workspace
    _same_as_alone([_Gemm(4, 16, 4096, 1024, (1, 1, 8), 11000),
                    _Gemm(8, 9, 2560, 768, (2, 4, 4), 11100)])


def test_attention_kernels_on_two_streams():
    # chunk merges of the one-head kernel and of the shared K/V stream
    _same_as_alone([_Attention(2, 16, 20, 4, 3000, [3000, 1900], 0, 256, 1, 11200),
                    _Attention(2, 16, 20, 4, 3000, [2800, 3000], 0, 256, 5, 11300)])


def test_mixed_calls_on_four_streams():
    _same_as_alone([_Gemm(4, 16, 2560, 2048, (1, 1, 4), 11400),
                    _Grouped(4, 16, 2560, [512, 256, 256], 11500),
                    _Attention(1, 16, 20, 4, 8192, [8192], 0, 0, 0, 11600),
                    _Attention(3, 16, 20, 4, 2048, [2048, 1024, 77], 1024, 128, 1, 11700)])
