"""GPU parity for the drafter's sliding-window attention (Drafter SWA
paragraph of arXiv 2607.04244) against the oracle's float64 definition.

Acceptance, per output element of one call:
    |gpu - ref| <= 1e-2 |ref| + 1e-3 rms(ref),
ref in float64 before output rounding. The kernel's own error is far inside
it: scores are fp32 sums of exact bf16 products, the softmax runs in fp32,
probabilities enter the value product as a bf16 pair (~2^-18 relative), the
sums are fp32, and the one bf16 rounding of the output is 2^-9 relative.

Every output is NaN-poisoned between canary bands, and the workspace's
chunk results are NaN-poisoned before a canary band, so a query or head left
unwritten, a chunk result never stored, or a stray store fails the test.

Inputs: q, k, v ~ N(0, 1) rounded to bf16, seeded; the drafter's head layout
(20 query heads, 4 KV heads of 128) and a 16-token block over the 8,192-token
Long context, plus smaller ragged batches.
"""

import numpy as np
import pytest
import torch

import int8_group_quantized_amd as q
from oracle import attention, numerics
import workloads
from gpu_helpers import DEV, Guarded, GuardedWorkspace, dev_bf16, host_u16

pytestmark = pytest.mark.gpu

D = 128


def _run(B, T, Hq, Hkv, S_max, lens, window, seed, scale=None, chunk=0, heads=0, std=1.0,
         poison=False, ws=None):
    qb, kb, vb = workloads.attention_inputs(B, T, Hq, Hkv, D, S_max, seed, std=std)
    if poison:   # NaN past each sequence's end: must never be read
        for b, S in enumerate(lens):
            kb[b, min(max(S, T), S_max):] = 0x7FC0
            vb[b, min(max(S, T), S_max):] = 0x7FC0
    sc = 1.0 / np.sqrt(D) if scale is None else scale
    out = Guarded((B, T, Hq, D), torch.bfloat16)
    wsg = ws or GuardedWorkspace(q.lib().qg_swa_workspace_bytes_plan(B, T, Hq, Hkv, D, S_max,
                                                                      window, chunk, heads))
    q.swa_attention(dev_bf16(qb), dev_bf16(kb), dev_bf16(vb),
                    torch.tensor(lens, dtype=torch.int32, device=DEV), window, sc,
                    chunk=chunk, heads=heads, out=out.t, ws=wsg.t)
    got = out.check("attention")
    wsg.check("attention")
    return qb, kb, vb, sc, host_u16(got)


def _ref(qb, kb, vb, lens, T, S_max, window, sc):
    eff = [min(max(S, T), S_max) for S in lens]
    return attention.swa_attention(numerics.bf16_to_f64(qb), numerics.bf16_to_f64(kb),
                                   numerics.bf16_to_f64(vb), eff, window, sc)


def _check(got_bits, ref, what=""):
    got = numerics.bf16_to_f64(got_bits)
    assert np.isfinite(got).all(), what
    rms = np.sqrt(np.mean(ref ** 2))
    err = np.abs(got - ref)
    bound = 1e-2 * np.abs(ref) + 1e-3 * rms
    bad = np.argwhere(err > bound)
    assert bad.size == 0, "%s: %d bad, first %s got %r ref %r" % (
        what, len(bad), bad[0], got[tuple(bad[0])], ref[tuple(bad[0])])


def _parity(B, T, Hq, Hkv, S_max, lens, window, seed, **kw):
    print("swa case B=%d T=%d Hq=%d Hkv=%d S_max=%d lens=%s window=%d %s" %
          (B, T, Hq, Hkv, S_max, lens, window, kw), flush=True)
    qb, kb, vb, sc, got = _run(B, T, Hq, Hkv, S_max, lens, window, seed, **kw)
    ref = _ref(qb, kb, vb, lens, T, S_max, window, sc)
    _check(got, ref, "B%d T%d S%s W%d" % (B, T, lens, window))
    return got


@pytest.mark.parametrize("window", [1024, 2048, 0])
def test_drafter_long_context_full_size(window):
    # one 16-token block after the 8,192-token Long context, drafter heads
    A = workloads.ATTENTION
    S = A["context"] + A["T"]
    _parity(1, A["T"], A["Hq"], A["Hkv"], S, [S], window, 6000 + window)


@pytest.mark.parametrize("window", [1024, 2048, 0])
def test_batch8_long_context_plans(window):
    # eight sequences of the drafter's heads over the Long cache, ragged: the
    # library's plan runs windowed spans unsplit at 160 query heads, one head
    # per workgroup, and the full cache in eight chunks with the 5 query heads
    # of a KV head sharing one stream of its rows
    A = workloads.ATTENTION
    S = A["context"] + A["T"]
    lens = [S, 5000, 1000, 600, S, 3000, 100, 2048]
    _parity(8, A["T"], A["Hq"], A["Hkv"], S, lens, window, 6050 + window)


def test_batch4_full_cache_plan():
    # four sequences over the Long cache without a window: the library's plan
    # streams K/V once per KV head group in 16 chunks; one sequence is only
    # the block, one ends inside the first chunk
    A = workloads.ATTENTION
    S = A["context"] + A["T"]
    _parity(4, A["T"], A["Hq"], A["Hkv"], S, [S, 4100, 700, 16], 0, 6080)


@pytest.mark.parametrize("B", [16, 40])
def test_large_batch_full_cache_sampled(B):
    # the library's plan over the full Long cache at larger batches: the
    # shared K/V stream in four chunks (16 sequences) or in one chunk, stored
    # without a merge (40 sequences, 160 units); sequences are independent,
    # so four of them (a ragged one and one that is only the block among
    # them) are checked against the oracle
    A = workloads.ATTENTION
    T, S = A["T"], A["context"] + A["T"]
    lens = [S if b % 7 else 3000 for b in range(B)]
    lens[-1] = T
    qb, kb, vb, sc, got = _run(B, T, A["Hq"], A["Hkv"], S, lens, 0, 6090 + B)
    pick = [0, 7, B // 2 + 1, B - 1]
    ref = _ref(qb[pick], kb[pick], vb[pick], [lens[i] for i in pick], T, S, 0, sc)
    _check(got[pick], ref, "B%d sampled %s" % (B, pick))


@pytest.mark.parametrize("window", [0, 64, 256, 1024, 5, 1])
def test_ragged_batch(window):
    # a long sequence, a medium one, one that is only the block, and one
    # just past the window
    _parity(4, 16, 8, 2, 700, [700, 333, 16, 65], window, 6100 + window)


@pytest.mark.parametrize("T", [1, 7, 15])
def test_partial_blocks(T):
    _parity(2, T, 20, 4, 1500, [1500, 900], 1024, 6200 + T)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 1), (16, 2)])
def test_head_layouts(Hq, Hkv):
    _parity(2, 16, Hq, Hkv, 1200, [1200, 1037], 512, 6300 + Hq * 10 + Hkv)


@pytest.mark.parametrize("chunk", [32, 64, 96, 4096])
def test_explicit_chunks(chunk):
    # 32: one step per workgroup (three wavefronts idle, many chunks to merge);
    # 4096: the whole window in one workgroup (no cross-workgroup merge)
    _parity(2, 16, 20, 4, 3000, [3000, 2100], 2048, 6400 + chunk, chunk=chunk)


def test_seq_lens_are_clamped():
    # a length past the cache reads as S_max, one below the block as T
    _parity(2, 4, 4, 2, 300, [400, 2], 64, 6500)


def test_cache_past_sequence_end_is_not_read():
    lens = [900, 417, 16]
    _, _, _, _, clean = _run(3, 16, 20, 4, 1000, lens, 256, 6600)
    _, _, _, _, dirty = _run(3, 16, 20, 4, 1000, lens, 256, 6600, poison=True)
    np.testing.assert_array_equal(dirty, clean)


@pytest.mark.parametrize("scale,std", [(0.05, 1.0), (1.0, 1.0), (1.0 / np.sqrt(128), 4.0)])
def test_scales_and_sharp_softmax(scale, std):
    _parity(1, 16, 20, 4, 2000, [2000], 1024, 6700, scale=scale, std=std)


def test_deterministic_and_workspace_reusable():
    lens = [2500, 1800]
    a = _parity(2, 16, 20, 4, 2500, lens, 0, 6800)
    ws = GuardedWorkspace(q.lib().qg_swa_workspace_bytes_plan(2, 16, 20, 4, D, 2500, 0, 0, 0))
    for _ in range(3):     # one workspace reused: its counters are left at zero
        _, _, _, _, b = _run(2, 16, 20, 4, 2500, lens, 0, 6800, ws=ws)
        np.testing.assert_array_equal(a, b)


def test_most_chunks_one_head_merges():
    # 256 chunks of 32 keys (the most one (sequence, head) may have): the
    # last workgroup to arrive merges 256 partial results
    _parity(1, 16, 4, 1, 8192, [8192], 0, 6900, chunk=32)


def test_million_token_cache():
    # a 2^20-position cache per sequence (offsets past 2^28 elements), the
    # window at its end and in the middle of a shorter sequence
    _parity(2, 16, 4, 1, 1 << 20, [1 << 20, 600001], 1024, 7000)


def test_empty_batch_is_a_no_op():
    qt = torch.empty((0, 16, 20, D), dtype=torch.bfloat16, device=DEV)
    kt = torch.empty((0, 100, 4, D), dtype=torch.bfloat16, device=DEV)
    lens = torch.empty((0,), dtype=torch.int32, device=DEV)
    out = q.swa_attention(qt, kt, kt, lens, 0)
    assert out.shape == qt.shape


# ---- query heads of one KV head sharing one stream of its K/V rows ----

@pytest.mark.parametrize("heads,Hq,Hkv", [(2, 8, 2), (3, 6, 1), (4, 16, 2), (5, 20, 4), (6, 12, 2),
                                          (8, 8, 1)])
def test_shared_stream_head_counts(heads, Hq, Hkv):
    # every head count the kernel is built for, with two head groups per KV
    # head where Hq / Hkv allows, ragged lengths and a chunk that ends inside
    # a 64-key step
    _parity(3, 16, Hq, Hkv, 2100, [2100, 1333, 40], 0, 7100 + heads, chunk=416, heads=heads)


@pytest.mark.parametrize("window,chunk", [(1024, 96), (64, 32), (1, 32)])
def test_shared_stream_windows(window, chunk):
    _parity(2, 16, 20, 4, 3000, [3000, 1100], window, 7200 + window, chunk=chunk, heads=5)


@pytest.mark.parametrize("T", [1, 7])
def test_shared_stream_partial_blocks(T):
    _parity(2, T, 20, 4, 1500, [1500, 700], 0, 7300 + T, chunk=256, heads=5)


def test_shared_stream_one_chunk():
    # a chunk covering the whole span: no merge, outputs stored directly
    _parity(2, 16, 20, 4, 1000, [1000, 517], 0, 7400, chunk=1024, heads=5)


def test_shared_stream_most_chunks():
    # 16 chunks (the most this kernel merges), several of them past the end
    # of the shorter sequences
    _parity(3, 16, 20, 4, 4096, [4096, 900, 16], 0, 7500, chunk=256, heads=5)


def test_shared_stream_cache_past_sequence_end_is_not_read():
    lens = [900, 417, 16]
    _, _, _, _, clean = _run(3, 16, 20, 4, 1000, lens, 0, 7600, chunk=128, heads=5)
    _, _, _, _, dirty = _run(3, 16, 20, 4, 1000, lens, 0, 7600, chunk=128, heads=5, poison=True)
    np.testing.assert_array_equal(dirty, clean)


def test_shared_stream_deterministic_and_workspace_shared():
    # one workspace serves both kernels in turn: each leaves its arrival
    # counters at zero
    lens = [2500, 1800]
    need = max(q.lib().qg_swa_workspace_bytes_plan(2, 16, 20, 4, D, 2500, 0, 320, h)
               for h in (1, 5))
    ws = GuardedWorkspace(need)
    a = _parity(2, 16, 20, 4, 2500, lens, 0, 7700, chunk=320, heads=5, ws=ws)
    for h in (1, 5, 5, 1, 5):
        _, _, _, _, b = _run(2, 16, 20, 4, 2500, lens, 0, 7700, chunk=320, heads=h, ws=ws)
        if h == 5:
            np.testing.assert_array_equal(a, b)
