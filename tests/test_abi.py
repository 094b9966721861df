"""The C-ABI library loads, exports every symbol include/qgemm.h declares, and
rejects bad arguments on the host with the documented status codes.

No call here reaches the GPU: every case fails validation, which the library
performs before any HIP call. Pointers are fake but aligned addresses that are
never dereferenced.
"""

import ctypes
import os
import re

import pytest

import int8_group_quantized_amd as q
from int8_group_quantized_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemm.h")

OK, NULL, SHAPE, ALIGN, DTYPE, WS, HIP, PLAN = range(8)
FAKE = 0x10000          # aligned, never dereferenced
MIS = 0x10008           # 8-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:qg_status|size_t|const char\*)\s+(\w+)\(", text, re.M)))


def test_library_exists_and_loads():
    assert os.path.exists(q.library_path()), "build the library first"
    assert q.lib() is not None


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 17
    L = ctypes.CDLL(q.library_path())
    for n in names:
        assert hasattr(L, n), n
    # and the binding describes every one of them
    assert set(names) == set(b._SIGNATURES)


def test_status_strings():
    L = q.lib()
    for code in range(8):
        assert L.qg_status_str(code).decode().startswith(b.STATUS[code])


def test_sizes():
    L = q.lib()
    assert L.qg_packed_bytes(4, 2560, 19456) == 24903680
    assert L.qg_packed_bytes(8, 2560, 19456) == 49807360
    assert L.qg_packed_bytes(4, 100, 16) == 0
    assert L.qg_packed_bytes(3, 128, 16) == 0
    assert L.qg_scale_bytes(9728, 2560) == 76 * 2560 * 2
    assert L.qg_workspace_bytes(4, 0, 128, 16) == 0
    # a split-K plan needs the counter block plus fp32 partials: whole 16-row
    # blocks per split
    ws = L.qg_workspace_bytes_plan(4, 3, 1024, 64, 1, 1, 4)
    assert ws == 65536 + 4 * 16 * 64 * 4
    assert L.qg_workspace_bytes_plan(4, 17, 1024, 64, 1, 1, 4) == 65536 + 4 * 32 * 64 * 4
    assert L.qg_workspace_bytes_plan(4, 3, 1024, 64, 1, 1, 1) == 0
    assert L.qg_workspace_bytes_plan(4, 3, 1024, 64, 3, 1, 1) == 0   # bad plan -> 0
    # the library's own plans: the decode GEMV and the 2-16-row GEMV (at most
    # 40 groups and 512 column blocks) need none; the M = 16 down shape
    # splits K and does
    assert L.qg_workspace_bytes(4, 1, 9728, 2560) == 0
    assert L.qg_workspace_bytes(8, 16, 2560, 3584) == 0
    assert L.qg_workspace_bytes(4, 16, 5120, 8192) == 0
    assert L.qg_workspace_bytes(4, 16, 9728, 2560) > 65536


def _gemm(M=1, K=256, N=512, x=FAKE, w=FAKE, s=FAKE, sdt=1, out=FAKE, ws=0, wsb=0, bits=4):
    f = q.lib().qgemm_w4a16 if bits == 4 else q.lib().qgemm_w8a16
    return f(x, w, s, sdt, out, M, K, N, ws, wsb, None)


@pytest.mark.parametrize("M,K,N", [(1, 100, 512), (1, 0, 512), (1, 256, 0), (1, 256, 24),
                                   (-1, 256, 512), (1, 2**21, 16), (2**25, 128, 16),
                                   (70000, 32768, 16)])
def test_gemm_bad_shapes(M, K, N):
    assert _gemm(M=M, K=K, N=N) == SHAPE
    assert _gemm(M=M, K=K, N=N, bits=8) == SHAPE


def test_gemm_bad_pointers_and_dtypes():
    assert _gemm(w=0) == NULL
    assert _gemm(s=0) == NULL
    assert _gemm(x=0) == NULL
    assert _gemm(out=0) == NULL
    assert _gemm(w=MIS) == ALIGN
    assert _gemm(x=MIS) == ALIGN
    assert _gemm(out=MIS + 2) == ALIGN
    assert _gemm(sdt=2) == DTYPE
    assert _gemm(sdt=7) == DTYPE
    # M == 0 is a valid empty call that enqueues nothing
    assert _gemm(M=0, x=0, out=0) == OK


def test_gemm_workspace_rules():
    L = q.lib()
    need = L.qg_workspace_bytes_plan(4, 1, 1024, 64, 1, 1, 4)
    f = L.qgemm_w4a16_plan
    assert f(FAKE, FAKE, FAKE, 1, FAKE, 1, 1024, 64, 0, 0, 1, 1, 4, None) == WS
    assert f(FAKE, FAKE, FAKE, 1, FAKE, 1, 1024, 64, FAKE, need - 1, 1, 1, 4, None) == WS
    assert f(FAKE, FAKE, FAKE, 1, FAKE, 1, 1024, 64, MIS, need, 1, 1, 4, None) == ALIGN
    assert f(FAKE, FAKE, FAKE, 1, FAKE, 1, 1024, 64, 0, 0, 3, 1, 1, None) == PLAN
    assert f(FAKE, FAKE, FAKE, 1, FAKE, 1, 1024, 64, 0, 0, 1, 3, 1, None) == PLAN
    assert f(FAKE, FAKE, FAKE, 1, FAKE, 1, 1024, 64, 0, 0, 1, 1, 9, None) == PLAN


def test_pack_entry_points_validate():
    L = q.lib()
    assert L.qg_pack_to_grid_w4(FAKE, 2, FAKE, 1, 100, 16, FAKE, None) == SHAPE
    assert L.qg_pack_to_grid_w4(FAKE, 1, FAKE, 1, 128, 16, FAKE, None) == DTYPE   # fp16 W
    assert L.qg_pack_to_grid_w8(FAKE, 2, FAKE, 2, 128, 16, FAKE, None) == DTYPE   # fp32 scales
    assert L.qg_pack_to_grid_w8(FAKE, 2, 0, 0, 128, 16, FAKE, None) == NULL
    assert L.qg_pack_to_grid_w8(FAKE, 2, FAKE, 0, 128, 16, MIS, None) == ALIGN
    assert L.qg_rtn_scales_w4(FAKE, 1, 128, 16, FAKE, None) == DTYPE
    assert L.qg_rtn_scales_w8(0, 2, 128, 16, FAKE, None) == NULL
    assert L.qg_rtn_scales_w8(FAKE, 2, 128, 8, FAKE, None) == SHAPE
    for fn in (L.qg_prepack_w4, L.qg_prepack_w8, L.qg_unpack_w4, L.qg_unpack_w8):
        assert fn(FAKE, 96, 16, FAKE, None) == SHAPE
        assert fn(0, 128, 16, FAKE, None) == NULL
        assert fn(FAKE, 128, 16, MIS, None) == ALIGN


def test_f16_gemm_entry_points_validate():
    L = q.lib()
    for f in (L.qgemm_w4f16, L.qgemm_w8f16):
        assert f(FAKE, FAKE, FAKE, 1, FAKE, 1, 100, 512, 0, 0, None) == SHAPE
        assert f(0, FAKE, FAKE, 1, FAKE, 1, 256, 512, 0, 0, None) == NULL
        assert f(FAKE, FAKE, FAKE, 2, FAKE, 1, 256, 512, 0, 0, None) == DTYPE
        assert f(FAKE, FAKE, FAKE, 1, MIS, 1, 256, 512, 0, 0, None) == ALIGN
        assert f(0, FAKE, FAKE, 1, 0, 0, 256, 512, 0, 0, None) == OK      # M = 0
    f = L.qgemm_w4f16_plan
    need = L.qg_workspace_bytes_plan(4, 1, 1024, 64, 1, 1, 4)
    assert f(FAKE, FAKE, FAKE, 1, FAKE, 1, 1024, 64, FAKE, need - 1, 1, 1, 4, None) == WS
    assert L.qgemm_w8f16_plan(FAKE, FAKE, FAKE, 0, FAKE, 1, 1024, 64, 0, 0, 3, 1, 1, None) == PLAN
    # an INT4 prefill call needs the offset workspace
    need = L.qg_workspace_bytes(4, 100, 256, 64)
    assert need == 65536 + 128 * 2 * 4
    assert L.qgemm_w4f16(FAKE, FAKE, FAKE, 1, FAKE, 100, 256, 64, 0, 0, None) == WS
    assert L.qg_workspace_bytes(8, 100, 256, 64) == 0


def test_dequant_entry_points_validate():
    L = q.lib()
    for f in (L.qg_dequant_w4, L.qg_dequant_w8):
        assert f(FAKE, FAKE, 1, 100, 16, FAKE, 0, None) == SHAPE
        assert f(FAKE, FAKE, 1, 128, 8, FAKE, 0, None) == SHAPE
        assert f(FAKE, FAKE, 2, 128, 16, FAKE, 0, None) == DTYPE       # fp32 scales
        assert f(FAKE, FAKE, 1, 128, 16, FAKE, 2, None) == DTYPE       # fp32 output
        assert f(0, FAKE, 1, 128, 16, FAKE, 0, None) == NULL
        assert f(FAKE, FAKE, 1, 128, 16, 0, 1, None) == NULL
        assert f(FAKE, MIS, 1, 128, 16, FAKE, 1, None) == ALIGN


def test_fake_quant_entry_points_validate():
    L = q.lib()
    for f in (L.qg_fake_quant_w4, L.qg_fake_quant_w8):
        assert f(FAKE, 2, FAKE, 1, 100, 16, FAKE, 0, None) == SHAPE
        assert f(FAKE, 1, FAKE, 1, 128, 16, FAKE, 0, None) == DTYPE      # fp16 W
        assert f(FAKE, 2, FAKE, 2, 128, 16, FAKE, 0, None) == DTYPE      # fp32 scales
        assert f(FAKE, 2, FAKE, 1, 128, 16, FAKE, 7, None) == DTYPE      # bad output dtype
        assert f(0, 2, FAKE, 1, 128, 16, FAKE, 2, None) == NULL
        assert f(FAKE, 0, FAKE, 0, 128, 16, MIS, 0, None) == ALIGN


def _items(*ns, p=FAKE):
    return (b.GroupItem * len(ns))(*[b.GroupItem(p, FAKE, FAKE, n) for n in ns])


def test_grouped_entry_points_validate():
    L = q.lib()
    for f in (L.qgemm_w4a16_grouped, L.qgemm_w8a16_grouped, L.qgemm_w4f16_grouped,
              L.qgemm_w8f16_grouped):
        assert f(FAKE, None, 1, 1, 1, 256, 0, 0, None) == NULL
        assert f(FAKE, _items(512), 0, 1, 1, 256, 0, 0, None) == SHAPE
        assert f(FAKE, _items(*([512] * 17)), 17, 1, 1, 256, 0, 0, None) == SHAPE
        assert f(FAKE, _items(512, 24), 2, 1, 1, 256, 0, 0, None) == SHAPE     # N % 16
        assert f(FAKE, _items(512), 1, 1, 1, 100, 0, 0, None) == SHAPE       # K % 128
        # each N within limits, their sum past 2^20
        assert f(FAKE, _items(1 << 19, 1 << 19, 16), 3, 1, 1, 128, 0, 0, None) == SHAPE
        assert f(FAKE, _items(512, 512, p=0), 2, 1, 1, 256, 0, 0, None) == NULL
        assert f(FAKE, _items(512), 1, 2, 1, 256, 0, 0, None) == DTYPE
        assert f(MIS, _items(512), 1, 1, 1, 256, 0, 0, None) == ALIGN
        assert f(0, _items(512), 1, 1, 0, 256, 0, 0, None) == OK             # M = 0
    # a group needs no more workspace than its plan; one item matches the single call
    assert L.qg_workspace_bytes_grouped(4, 16, 9728, _items(2560), 1) == \
        L.qg_workspace_bytes(4, 16, 9728, 2560)
    assert L.qg_workspace_bytes_grouped(4, 16, 9728, None, 1) == 0


def _swa(L, B=1, T=16, Hq=20, Hkv=4, D=128, S_max=8208, window=1024, scale=0.088, chunk=0,
         heads=0, q=FAKE, k=FAKE, v=FAKE, lens=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return L.qg_swa_attention_plan(q, k, v, lens, out, B, T, Hq, Hkv, D, S_max, window, scale,
                                   chunk, heads, ws, ws_bytes, None)


def test_swa_attention_validates():
    L = q.lib()
    # shapes
    assert _swa(L, D=64) == SHAPE
    assert _swa(L, T=0) == SHAPE
    assert _swa(L, T=17) == SHAPE
    assert _swa(L, Hq=20, Hkv=3) == SHAPE
    assert _swa(L, Hkv=0) == SHAPE
    assert _swa(L, T=1, Hq=4104, Hkv=4) == SHAPE      # more than 4096 query heads
    assert _swa(L, S_max=8) == SHAPE                # shorter than the block
    assert _swa(L, window=-1) == SHAPE
    assert _swa(L, chunk=48) == SHAPE               # not a multiple of 32
    # query heads per workgroup: 2-6 or 8, dividing Hq / Hkv (5 here)
    for heads in (-1, 7, 9, 2, 3, 4, 6, 8):
        assert _swa(L, heads=heads) == SHAPE, heads
    assert _swa(L, Hq=24, Hkv=4, heads=4) == SHAPE  # 6 heads per KV head
    # the shared-ring kernel merges at most 16 chunks
    assert _swa(L, window=0, heads=5, chunk=512) == SHAPE      # 17 chunks
    assert L.qg_swa_workspace_bytes_plan(1, 16, 20, 4, 128, 8208, 0, 512, 5) == 0
    assert L.qg_swa_workspace_bytes_plan(1, 16, 20, 4, 128, 8208, 0, 512, 1) > 0   # one head each
    assert _swa(L, B=-1) == SHAPE
    assert _swa(L, S_max=1 << 22, Hkv=16) == SHAPE  # a sequence's cache past 2^31 bytes
    assert _swa(L, scale=float("nan")) == SHAPE
    assert _swa(L, scale=float("inf")) == SHAPE
    # pointers
    assert _swa(L, q=0) == NULL
    assert _swa(L, lens=0) == NULL
    assert _swa(L, out=MIS) == ALIGN
    assert _swa(L, lens=FAKE + 2) == ALIGN
    # workspace (the library plan splits S = 8208 into chunks)
    need = L.qg_swa_workspace_bytes(1, 16, 20, 4, 128, 8208, 1024)
    assert need > 65536
    assert _swa(L, ws=0, ws_bytes=0) == WS
    assert _swa(L, ws_bytes=need - 1) == WS
    assert _swa(L, ws=MIS) == ALIGN
    # an empty batch is a no-op that touches nothing
    assert _swa(L, B=0, q=0, k=0, v=0, lens=0, out=0, ws=0, ws_bytes=0) == OK


def test_swa_workspace_sizes():
    L = q.lib()
    # one chunk (a short cache, or a chunk covering the whole window) needs none
    assert L.qg_swa_workspace_bytes(1, 16, 20, 4, 128, 100, 0) == 0
    assert L.qg_swa_workspace_bytes_plan(1, 16, 20, 4, 128, 8208, 1024, 2048, 0) == 0
    assert L.qg_swa_workspace_bytes_plan(1, 16, 20, 4, 128, 8208, 1024, 2048, 5) == 0
    # otherwise the counter block plus per-chunk partials (16 x 128 outputs,
    # 16 maxima, 16 sums, fp32) for each (sequence, query head)
    n = L.qg_swa_workspace_bytes_plan(2, 16, 8, 2, 128, 1000, 0, 256, 0)
    assert n == 65536 + 2 * 8 * 4 * (16 * 128 + 32) * 4
    # the shared-ring kernel keeps the same record per (sequence, query head, chunk)
    assert L.qg_swa_workspace_bytes_plan(2, 16, 8, 2, 128, 1000, 0, 256, 2) == n
    assert L.qg_swa_workspace_bytes_plan(2, 16, 8, 2, 128, 1000, 0, 256, 3) == 0   # 3 does not divide 4
    # the library's own split: batch 4 and 8 of the drafter's heads over the
    # full 8,208-token cache stream K/V once per 5 query heads in 16 and 8
    # chunks; batch 1 and windowed spans keep one head per workgroup (12 and
    # 5 chunks here)
    rec = (16 * 128 + 32) * 4
    assert L.qg_swa_workspace_bytes(8, 16, 20, 4, 128, 8208, 0) == 65536 + 8 * 20 * 8 * rec
    assert L.qg_swa_workspace_bytes(4, 16, 20, 4, 128, 8208, 0) == 65536 + 4 * 20 * 16 * rec
    assert L.qg_swa_workspace_bytes(1, 16, 20, 4, 128, 8208, 0) == 65536 + 20 * 12 * rec
    assert L.qg_swa_workspace_bytes(1, 16, 20, 4, 128, 8208, 1024) == 65536 + 20 * 5 * rec
    # a window wider than the cache is no window
    assert L.qg_swa_workspace_bytes(1, 16, 20, 4, 128, 1000, 5000) == \
        L.qg_swa_workspace_bytes(1, 16, 20, 4, 128, 1000, 0)


@pytest.mark.parametrize("nbytes,wgs", [(0, 1), (17, 1), (8, 1), (1 << 40, 1), (16, 0), (16, 65537),
                                        (16, -1)])
def test_read_stream_bad_sizes(nbytes, wgs):
    assert q.lib().qg_read_stream(FAKE, nbytes, wgs, FAKE, None) == SHAPE


def test_read_stream_bad_pointers():
    L = q.lib()
    assert L.qg_read_stream(0, 16, 1, FAKE, None) == NULL
    assert L.qg_read_stream(FAKE, 16, 1, 0, None) == NULL
    assert L.qg_read_stream(MIS, 16, 1, FAKE, None) == ALIGN
    assert L.qg_read_stream(FAKE, 16, 1, MIS, None) == ALIGN


def test_prepack_scales_rejects_bad_arguments():
    L = q.lib()
    assert L.qg_prepack_scales(FAKE, 1, 100, 16, FAKE, None) == SHAPE
    assert L.qg_prepack_scales(FAKE, 1, 128, 24, FAKE, None) == SHAPE
    assert L.qg_prepack_scales(FAKE, 2, 128, 16, FAKE, None) == DTYPE      # fp32 scales
    assert L.qg_prepack_scales(FAKE, 3, 128, 16, FAKE, None) == DTYPE      # already prepacked
    assert L.qg_prepack_scales(0, 1, 128, 16, FAKE, None) == NULL
    assert L.qg_prepack_scales(FAKE, 1, 128, 16, MIS, None) == ALIGN


@pytest.mark.parametrize("cbm", [3, 4])
def test_prepacked_scales_only_for_gemms(cbm):
    """Only the GEMM entry points take column-block-major scales."""
    L = q.lib()
    assert L.qg_pack_to_grid_w4(FAKE, 2, FAKE, cbm, 128, 16, FAKE, None) == DTYPE
    assert L.qg_dequant_w4(FAKE, FAKE, cbm, 128, 16, FAKE, 0, None) == DTYPE
    assert L.qg_fake_quant_w4(FAKE, 2, FAKE, cbm, 128, 16, FAKE, 0, None) == DTYPE
    assert _gemm(M=1, K=100, N=512, sdt=cbm) == SHAPE          # accepted dtype, shape checked
    assert L.qgemm_w4a16(FAKE, FAKE, FAKE, 5, FAKE, 1, 256, 512, 0, 0, None) == DTYPE


def test_noalloc_gemm_validates_before_any_device_call():
    """The no-allocation W4A16 GEMM: the checks of qgemm_w4a16, then the
    workspace the call would need against the fixed scratch, all on the
    host (these calls reach no device)."""
    L = q.lib()
    assert L.qg_noalloc_scratch_bytes() == 8 << 20
    f = L.qgemm_w4a16_noalloc
    assert f(FAKE, FAKE, FAKE, 1, FAKE, 1, 100, 512, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, 1, FAKE, 1, 256, 24, None) == SHAPE
    assert f(0, FAKE, FAKE, 1, FAKE, 1, 256, 512, None) == NULL
    assert f(FAKE, FAKE, 0, 1, FAKE, 1, 256, 512, None) == NULL
    assert f(MIS, FAKE, FAKE, 1, FAKE, 1, 256, 512, None) == ALIGN
    assert f(FAKE, FAKE, FAKE, 2, FAKE, 1, 256, 512, None) == DTYPE
    assert f(0, FAKE, FAKE, 1, 0, 0, 256, 512, None) == OK          # M = 0: nothing to do
    # a prefill whose INT4 offsets (30016 rows x 76 groups x 4 B) exceed 8 MiB
    assert L.qg_workspace_bytes(4, 30000, 9728, 16) > L.qg_noalloc_scratch_bytes()
    assert f(FAKE, FAKE, FAKE, 1, FAKE, 30000, 9728, 16, None) == WS
