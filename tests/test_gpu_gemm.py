"""GPU parity for the GEMM: the HIP path against the oracle's float64
reference with the acceptance bound
    |gpu - ref| <= 1e-2 |ref| + 1e-3 rms(ref),
bit-exact where the result is exact (identity probe, zero scales, zero x),
and bit-identical across repeated calls (determinism).

Small shapes span several tiles with ragged tails and run every tiling plan
(columns per wave, K-splitting waves, K-splitting workgroups); the five
workloads run at full size with the library's own plan, every output
compared (the M = 8192 prefill ones included, with rms over the whole
output).

Every call writes into a NaN-poisoned output between two canary bands, and
uses a workspace whose split-K partials / prefill offsets are NaN-poisoned
and followed by a canary band: an output element a plan leaves unwritten, a
partial a split never stores, or a store outside either buffer fails the
test (the caching allocator can no longer hand back a block that still holds
an earlier plan's correct result).
"""

import numpy as np
import pytest
import torch

import int8_group_quantized_amd as q
from oracle import gemm, numerics, quant
import workloads
from gpu_helpers import Guarded, GuardedWorkspace, guarded_gemm as _call, dev_bf16, dev_f32, dev_i8, dev_scales, host_u16

pytestmark = pytest.mark.gpu

SDT = {4: "f16", 8: "bf16"}


def _inputs(bits, M, K, N, seed, xstd=1.0):
    x = workloads.activations(M, K, seed, std=xstd)
    c = workloads.codes(K, N, bits, seed + 1)
    s = workloads.scales(K // 128, N, SDT[bits], seed + 2)
    return x, c, s




def _run(bits, x, c, s, N, plan=None):
    pg = q.prepack(dev_i8(c), bits)
    return numerics.bf16_to_f64(_call(dev_bf16(x), pg, dev_scales(s, SDT[bits]), bits, N, plan=plan,
                                      what="plan %s" % (plan,)))


def _assert_close(got, ref, what=""):
    ok = gemm.within_tolerance(got, ref)
    if not ok.all():
        bad = np.argwhere(~ok)[:8]
        detail = [(tuple(int(i) for i in b), float(got[tuple(b)]), float(ref[tuple(b)])) for b in bad]
        raise AssertionError("%s: %d of %d outside tolerance (rms %.4g): %s"
                             % (what, (~ok).sum(), ok.size, gemm.rms(ref), detail))


PLANS = [None, (1, 1, 1), (1, 4, 1), (2, 4, 3), (4, 1, 2), (4, 4, 5), (1, 2, 7), (2, 1, 2),
         (1, 8, 2), (2, 2, 1), (2, 2, 3)]
SHAPES = [(1, 256, 512), (3, 896, 592), (16, 1280, 272), (7, 384, 48), (16, 128, 16)]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_small_shapes_every_plan(bits, M, K, N):
    x, c, s = _inputs(bits, M, K, N, 100 * M + K + N)
    ref = gemm.gemm_ref(x, c, s, SDT[bits])
    G = K // 128
    first = None
    for plan in PLANS:
        if plan is not None and plan[2] > G:
            continue
        got = _run(bits, x, c, s, N, plan)
        _assert_close(got, ref, "plan %s" % (plan,))
        if plan is not None and plan[2] == 1 and first is None:
            first = got
    # every plan is a valid summation order; repeated calls are bit-identical
    a = _run(bits, x, c, s, N, (2, 4, min(3, G)))
    b = _run(bits, x, c, s, N, (2, 4, min(3, G)))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M", [17, 33, 64])
def test_multi_row_blocks(bits, M):
    """M > 16: the library's plan (prefill kernel) and the small-M kernel
    over 16-row blocks (explicit plans, K unsplit and split across
    workgroups, whose partials are kept per row block) all match the
    oracle; a split plan repeats bit for bit."""
    K, N = 512, 96
    x, c, s = _inputs(bits, M, K, N, 900 + M)
    ref = gemm.gemm_ref(x, c, s, SDT[bits])
    _assert_close(_run(bits, x, c, s, N), ref, "M=%d prefill" % M)
    for plan in [(1, 1, 1), (1, 1, 4), (2, 4, 2), (4, 1, 3)]:
        _assert_close(_run(bits, x, c, s, N, plan=plan), ref, "M=%d row blocks %s" % (M, plan))
    a = _run(bits, x, c, s, N, plan=(1, 1, 4))
    assert np.array_equal(a, _run(bits, x, c, s, N, plan=(1, 1, 4)))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M,K,N", [(17, 128, 16), (129, 896, 592), (256, 1280, 2048),
                                   (300, 384, 272), (1000, 256, 4096),
                                   (8190, 256, 2080), (4097, 384, 4112)])
def test_prefill_shapes(bits, M, K, N):
    """Prefill kernel: ragged tiles in M and N, one-group K; the last two
    shapes have enough 128 x 256 tiles for the large-tile plan (ragged in
    both M and N there too)."""
    x, c, s = _inputs(bits, M, K, N, 7 * M + N)
    ref = gemm.gemm_ref(x, c, s, SDT[bits])
    got = _run(bits, x, c, s, N)
    _assert_close(got, ref, "prefill M=%d K=%d N=%d" % (M, K, N))
    assert np.array_equal(got, _run(bits, x, c, s, N))      # deterministic


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M,K,N", [(1, 1 << 20, 16), (16, 1 << 20, 16), (17, 1 << 20, 16),
                                   (1, 128, 1 << 20), (16, 128, 1 << 20), (17, 128, 1 << 20)])
def test_maximum_extents(bits, M, K, N):
    """The largest K and N the boundary accepts (2^20 each): 8,192 groups in
    one column block (hundreds of K splits at M = 16, a 8,192-group K loop
    in the prefill kernel) and 65,536 column blocks in one group (the widest
    grids), on each kernel."""
    x, c, s = _inputs(bits, M, K, N, 31 + M + (K >> 7))
    ref = gemm.gemm_ref(x, c, s, SDT[bits])
    _assert_close(_run(bits, x, c, s, N), ref, "M=%d K=%d N=%d" % (M, K, N))


@pytest.mark.parametrize("bits", [4, 8])
def test_prefill_other_scale_dtype(bits):
    """fp16 and bf16 scales are both accepted (configs use fp16 for INT4,
    bf16 for INT8; the other pairing goes through the same kernels)."""
    M, K, N = 200, 640, 320
    other = "bf16" if bits == 4 else "f16"
    x = workloads.activations(M, K, 5)
    c = workloads.codes(K, N, bits, 6)
    sb = workloads.scales(K // 128, N, other, 7)
    pg = q.prepack(dev_i8(c), bits)
    for m in (M, 1, 16):
        got = numerics.bf16_to_f64(_call(dev_bf16(x[:m]), pg, dev_scales(sb, other), bits, N))
        _assert_close(got, gemm.gemm_ref(x[:m], c, sb, other), "M=%d" % m)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("K", [256, 2560])
def test_identity_probe_bit_exact(bits, K):
    """x = I_K reads back the effective weight: out = bf16(s * q) exactly
    (the identity probe of the W8A16 model card's vLLM patch notes)."""
    N = 64
    _, c, s = _inputs(bits, 1, K, N, 40 + K)
    eye = np.where(np.eye(K, dtype=bool), np.uint16(0x3F80), np.uint16(0))
    ref = gemm.gemm_ref(eye, c, s, SDT[bits])
    want = numerics.f64_exact_to_bf16(ref)
    pg = q.prepack(dev_i8(c), bits)
    got = _call(dev_bf16(eye), pg, dev_scales(s, SDT[bits]), bits, N)
    bad = np.argwhere(got != want)
    assert bad.size == 0, [(int(k), int(n), int(c[k, n]), hex(got[k, n]), hex(want[k, n]))
                           for k, n in bad[:10]]


def _zero_code_bound(bits, x, s):
    """|out| bound for an all-zero code column: INT8 codes give exact zeros;
    INT4 codes 0 expand to 136 and cancel against the 136 * sum x offset that
    seeds the chain, leaving the fp32 rounding of a few partial sums of size
    136 * sum |x| per group."""
    M, K = x.shape
    if bits == 8:
        return np.zeros((M, 1))
    xs = numerics.bf16_to_f64(x)
    sv = numerics.scale_bits_to_f64(s, SDT[bits])
    gsum = np.abs(xs).reshape(M, K // 128, 128).sum(axis=2)          # [M, G]
    return 8 * 2.0 ** -24 * 136 * gsum @ np.abs(sv[:, :16])           # [M, 16]


ZERO_PLANS = [None, (1, 1, 1), (1, 4, 1), (2, 4, 3), (4, 1, 2), (1, 1, 5)]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M", [1, 5, 16, 200])
def test_zero_codes_scales_and_activations(bits, M):
    """Zero scales and zero activations give exact zeros on every path. An
    all-zero code column gives exactly 0 at M <= 16 on every small-M plan
    (INT8 codes are exact zeros; INT4 zero codes expand to 136 and cancel
    against the 136 * sum x offset, which is the same matrix-core chain over
    the same operands), and at M > 16 exactly 0 for INT8 and only the fp32
    rounding of the INT4 offset it cancels (the prefill pre-pass seeds the
    chain with the negated offset)."""
    K, N = 640, 320
    x, c, s = _inputs(bits, M, K, N, 61 + M)
    c[:, :16] = 0                     # first column block: all-zero codes
    s = s.copy()
    s[:, 16:32] = 0                   # second block: zero scales
    z = np.zeros_like(c)
    plans = ZERO_PLANS if M <= 16 else [None]
    for plan in plans:
        got = _run(bits, x, c, s, N, plan)
        assert np.all(got[:, 16:32] == 0), plan
        if M <= 16 or bits == 8:
            assert np.all(got[:, :16] == 0), plan
            assert np.all(_run(bits, x, z, s, N, plan) == 0), plan
        else:
            assert np.all(np.abs(got[:, :16]) <= _zero_code_bound(bits, x, s))
            assert np.all(np.abs(_run(bits, x, z, s, N, plan)[:, :16]) <= _zero_code_bound(bits, x, s))
        _assert_close(got, gemm.gemm_ref(x, c, s, SDT[bits]), "plan %s" % (plan,))
        assert np.all(_run(bits, np.zeros_like(x), c, s, N, plan) == 0), plan


@pytest.mark.parametrize("bits", [4, 8])
def test_range_ends_and_large_activations(bits):
    M, K, N = 16, 1024, 128
    x, c, s = _inputs(bits, M, K, N, 71, xstd=3e3)
    lo = -8 if bits == 4 else -127
    c[:, ::3] = lo                    # the asymmetric INT4 end, never produced by RTN
    c[::5, :] = -lo if bits == 8 else 7
    _assert_close(_run(bits, x, c, s, N), gemm.gemm_ref(x, c, s, SDT[bits]))


@pytest.mark.parametrize("bits", [4, 8])
def test_constant_codes_and_ones(bits):
    M, K, N = 2, 768, 48
    x, c, s = _inputs(bits, M, K, N, 81)
    c[:] = 3
    ones = np.full((M, K), 0x3F80, dtype=np.uint16)
    _assert_close(_run(bits, ones, c, s, N), gemm.gemm_ref(ones, c, s, SDT[bits]))
    _assert_close(_run(bits, x, c, s, N), gemm.gemm_ref(x, c, s, SDT[bits]))


def test_empty_m_is_a_noop():
    K, N = 256, 32
    c = workloads.codes(K, N, 4, 1)
    pg = q.prepack(dev_i8(c), 4)
    x = torch.empty((0, K), dtype=torch.bfloat16, device="cuda:0")
    out = q.qgemm_w4a16(x, pg, dev_scales(workloads.scales(2, N, "f16", 2), "f16"), N)
    assert out.shape == (0, N)


def test_workspace_reuse_across_plans():
    """Counters are left at zero: alternating split plans on one workspace."""
    M, K, N = 4, 1280, 80
    x, c, s = _inputs(4, M, K, N, 91)
    ref = gemm.gemm_ref(x, c, s, "f16")
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda:0")
    pg = q.prepack(dev_i8(c), 4)
    xd, sd = dev_bf16(x), dev_scales(s, "f16")
    for plan in [(1, 1, 10), (2, 4, 3), (1, 1, 10), (4, 4, 2), (1, 1, 1), (2, 1, 5), (2, 2, 4)]:
        out = Guarded((M, N), torch.bfloat16)
        q.qgemm_w4a16(xd, pg, sd, N, out=out.t, plan=plan, ws=ws)
        _assert_close(numerics.bf16_to_f64(host_u16(out.check(str(plan)))), ref, str(plan))
    assert torch.count_nonzero(ws[:65536]) == 0


def _workload_case(cfg, shape_index):
    w = workloads.WORKLOADS[cfg]
    K, N = w["shapes"][shape_index]
    bits, M = w["bits"], w["M"]
    W = workloads.weights(K, N, workloads.seed_for(cfg, shape_index, 0))
    x = workloads.activations(M, K, workloads.seed_for(cfg, shape_index, 1))
    return bits, M, K, N, W, x


WORKLOAD_CASES = [(cfg, i) for cfg in (1, 2, 3, 4, 5)
                  for i in range(len(workloads.WORKLOADS[cfg]["shapes"]))]


@pytest.mark.parametrize("cfg,shape_index", WORKLOAD_CASES)
def test_workloads_full_size(cfg, shape_index):
    """Full pipeline on the GPU (RTN scales -> Q_s pack -> GEMM) against the
    oracle's RTN -> Q_s -> float64 product on the same seeded W and x."""
    bits, M, K, N, W, x = _workload_case(cfg, shape_index)
    sdt = SDT[bits]
    sb = quant.rtn_scales(W, bits)
    codes = quant.q_s(W, numerics.scale_bits_to_f64(sb, sdt), bits)
    print("workload config %d shape %d: M=%d K=%d N=%d" % (cfg, shape_index, M, K, N), flush=True)
    Wd = dev_f32(W)
    sg = q.rtn_scales(Wd, bits)
    assert np.array_equal(host_u16(sg), sb)
    pg = q.pack_to_grid(Wd, sg, bits)
    del Wd
    got_bits = _call(dev_bf16(x), pg, sg, bits, N, what="config %d shape %d" % (cfg, shape_index))
    # every output, rms over the whole [M, N] output (M = 8192 included)
    ref = gemm.gemm_ref(x, codes, sb, sdt)
    _assert_close(numerics.bf16_to_f64(got_bits), ref, "config %d shape %d" % (cfg, shape_index))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M", [1, 16, 300])
def test_heavy_tailed_weights_through_rtn(bits, M):
    """Heavy-tailed weights (Student-t, 3 dof, x 0.02): the oracle's RTN scales
    and Q_s codes, whose scales then spread over a wide range across groups,
    through the decode, verification and prefill paths."""
    K, N = 1280, 336
    W = workloads.weights(K, N, 90 + M, dist="student_t")
    sb = quant.rtn_scales(W, bits)
    c = quant.q_s(W, numerics.scale_bits_to_f64(sb, SDT[bits]), bits)
    x = workloads.activations(M, K, 91 + M)
    sv = numerics.scale_bits_to_f64(sb, SDT[bits])
    assert sv.max() / sv[sv > 0].min() > 8        # the scales do spread
    _assert_close(_run(bits, x, c, sb, N), gemm.gemm_ref(x, c, sb, SDT[bits]), "M=%d" % M)


def _prefill_walk(M, N):
    """Host mirror of the prefill plan's tile-width choice and of the
    condition under which its tile walk goes panel by panel (each XCD's
    share of tiles is whole tile rows); returns (wn, tiles_n, panel walk,
    width of the last panel). Used only to document what a case covers."""
    tiles_m, NB = -(-M // 64), N // 16
    best, pick = -1.0, None
    for wn in (4, 2):
        tn = -(-NB // (4 * wn))
        tiles = tiles_m * tn
        slots = 256 * (2 if wn == 4 else 3)
        eff = tiles / (-(-tiles // slots) * slots) * (1.0 if wn == 4 else 0.85)
        if eff > best + 1e-9:
            best, pick = eff, (wn, tn, tiles)
    wn, tn, tiles = pick
    per = tiles // 8
    return wn, tn, per % tn == 0, tn % 8


PANEL_CASES = [(4096, 256, 19456), (1024, 384, 2560)]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("cbm", [False, True])
@pytest.mark.parametrize("M,K,N", PANEL_CASES)
def test_prefill_panel_walk_full_output(bits, act, cbm, M, K, N):
    """The production prefill tile walk (the one the M = 8192 calls take:
    64-row tiles dealt to XCDs in whole tile rows, walked in panels of eight
    column tiles with a narrower last panel), every output compared. The
    first case uses 64 x 256 tiles (76 tile columns: nine panels of eight and
    one of four), the second 64 x 128 tiles (20 tile columns: two panels of
    eight and one of four); with fp16 activations and column-block-major
    scales as well."""
    wn, tn, panel, last = _prefill_walk(M, N)
    assert panel and last, (wn, tn)
    print("panel walk: bits=%d act=%s cbm=%s M=%d K=%d N=%d wn=%d tiles_n=%d"
          % (bits, act, cbm, M, K, N, wn, tn), flush=True)
    x = workloads.activations(M, K, 1300 + M, dtype=act)
    c = workloads.codes(K, N, bits, 1301 + M)
    s = workloads.scales(K // 128, N, SDT[bits], 1302 + M)
    xd = dev_bf16(x) if act == "bf16" else torch.from_numpy(x.view(np.int16)).view(
        torch.float16).to("cuda:0")
    sd = dev_scales(s, SDT[bits])
    if cbm:
        sd = q.prepack_scales(sd)
    pg = q.prepack(dev_i8(c), bits)
    got = numerics.act_to_f64(_call(xd, pg, sd, bits, N, cbm=cbm, what="panel walk"), act)
    _assert_close(got, gemm.gemm_ref(x, c, s, SDT[bits], x_dtype=act), "panel walk")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("K,N", [(128, 16), (384, 48), (896, 592), (2688, 1040), (10368, 48),
                                 (10624, 208), (20608, 16)])
def test_decode_gemv_k_waves_and_rounds(bits, K, N):
    """M = 1, the decode GEMV: K of 1, 3, 7, 21, 81, 83 and 161 groups, so the
    number of K-wavefronts runs 1, 1, 2, 8, 16, 16, 16 with ragged (or
    empty) last wavefronts and one, two or three rounds of five groups per
    wavefront; the first column block has all-zero codes and must come out
    exactly 0."""
    x, c, s = _inputs(bits, 1, K, N, 1700 + K + N)
    c[:, :16] = 0
    got = _run(bits, x, c, s, N)
    assert np.all(got[:, :16] == 0)
    _assert_close(got, gemm.gemm_ref(x, c, s, SDT[bits]), "K=%d N=%d" % (K, N))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M", [2, 5, 9, 16])
@pytest.mark.parametrize("K,N", [(128, 16), (640, 48), (768, 32), (2560, 8192), (5120, 64),
                                 (5248, 64), (2560, 8208)])
def test_rows_gemv_rows_groups_and_limits(bits, M, K, N):
    """2-16 rows on the library's own plan: 1, 5, 6, 20, 40 groups take the
    rows GEMV (one to eight K-wavefronts, ragged last wavefronts), 41 groups
    or 513 column blocks the staged kernel; rows past M are never written
    (NaN-poisoned output), the first column block has all-zero codes and
    must come out exactly 0."""
    x, c, s = _inputs(bits, M, K, N, 1900 + 31 * M + K + N)
    c[:, :16] = 0
    got = _run(bits, x, c, s, N)
    assert np.all(got[:, :16] == 0)
    _assert_close(got, gemm.gemm_ref(x, c, s, SDT[bits]), "M=%d K=%d N=%d" % (M, K, N))
