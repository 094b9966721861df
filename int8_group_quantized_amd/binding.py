"""Thin Python binding over libqgemm.so (the C ABI in include/qgemm.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library. Tensors are PyTorch CUDA (HIP) tensors; work is
enqueued on the current PyTorch stream of the tensor's device. If the
library has not been built this module raises at first use -- there is no
fallback path.
"""

import ctypes
import math
import os
import threading

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqgemm.so")
_lib = None
_lock = threading.Lock()

QG_BF16, QG_F16, QG_F32 = 0, 1, 2
QG_F16_CBM, QG_BF16_CBM = 3, 4           # column-block-major scales (prepack_scales)
_CBM = {QG_F16: QG_F16_CBM, QG_BF16: QG_BF16_CBM}
STATUS = {0: "QG_OK", 1: "QG_ERR_NULL", 2: "QG_ERR_SHAPE", 3: "QG_ERR_ALIGN",
          4: "QG_ERR_DTYPE", 5: "QG_ERR_WORKSPACE", 6: "QG_ERR_HIP", 7: "QG_ERR_PLAN"}

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_SZ = ctypes.c_size_t

class GroupItem(ctypes.Structure):
    """qg_group_item of the C ABI."""
    _fields_ = [("packed_w", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("N", ctypes.c_int64)]


_ITEMS = ctypes.POINTER(GroupItem)

_SIGNATURES = {
    "qg_status_str": ([_INT], ctypes.c_char_p),
    "qg_packed_bytes": ([_INT, _I64, _I64], _SZ),
    "qg_scale_bytes": ([_I64, _I64], _SZ),
    "qg_workspace_bytes": ([_INT, _I64, _I64, _I64], _SZ),
    "qg_workspace_bytes_plan": ([_INT, _I64, _I64, _I64, _INT, _INT, _INT], _SZ),
    "qg_rtn_scales_w4": ([_P, _INT, _I64, _I64, _P, _P], _INT),
    "qg_rtn_scales_w8": ([_P, _INT, _I64, _I64, _P, _P], _INT),
    "qg_pack_to_grid_w4": ([_P, _INT, _P, _INT, _I64, _I64, _P, _P], _INT),
    "qg_pack_to_grid_w8": ([_P, _INT, _P, _INT, _I64, _I64, _P, _P], _INT),
    "qg_prepack_w4": ([_P, _I64, _I64, _P, _P], _INT),
    "qg_unpack_w4": ([_P, _I64, _I64, _P, _P], _INT),
    "qg_prepack_w8": ([_P, _I64, _I64, _P, _P], _INT),
    "qg_unpack_w8": ([_P, _I64, _I64, _P, _P], _INT),
    "qgemm_w4a16": ([_P, _P, _P, _INT, _P, _I64, _I64, _I64, _P, _SZ, _P], _INT),
    "qgemm_w8a16": ([_P, _P, _P, _INT, _P, _I64, _I64, _I64, _P, _SZ, _P], _INT),
    "qgemm_w4a16_plan": ([_P, _P, _P, _INT, _P, _I64, _I64, _I64, _P, _SZ, _INT, _INT, _INT, _P],
                         _INT),
    "qgemm_w8a16_plan": ([_P, _P, _P, _INT, _P, _I64, _I64, _I64, _P, _SZ, _INT, _INT, _INT, _P],
                         _INT),
    "qgemm_w4f16": ([_P, _P, _P, _INT, _P, _I64, _I64, _I64, _P, _SZ, _P], _INT),
    "qgemm_w8f16": ([_P, _P, _P, _INT, _P, _I64, _I64, _I64, _P, _SZ, _P], _INT),
    "qgemm_w4f16_plan": ([_P, _P, _P, _INT, _P, _I64, _I64, _I64, _P, _SZ, _INT, _INT, _INT, _P],
                         _INT),
    "qgemm_w8f16_plan": ([_P, _P, _P, _INT, _P, _I64, _I64, _I64, _P, _SZ, _INT, _INT, _INT, _P],
                         _INT),
    "qg_fake_quant_w4": ([_P, _INT, _P, _INT, _I64, _I64, _P, _INT, _P], _INT),
    "qg_fake_quant_w8": ([_P, _INT, _P, _INT, _I64, _I64, _P, _INT, _P], _INT),
    "qg_dequant_w4": ([_P, _P, _INT, _I64, _I64, _P, _INT, _P], _INT),
    "qg_workspace_bytes_grouped": ([_INT, _I64, _I64, _ITEMS, _INT], _SZ),
    "qgemm_w4a16_grouped": ([_P, _ITEMS, _INT, _INT, _I64, _I64, _P, _SZ, _P], _INT),
    "qgemm_w8a16_grouped": ([_P, _ITEMS, _INT, _INT, _I64, _I64, _P, _SZ, _P], _INT),
    "qgemm_w4f16_grouped": ([_P, _ITEMS, _INT, _INT, _I64, _I64, _P, _SZ, _P], _INT),
    "qgemm_w8f16_grouped": ([_P, _ITEMS, _INT, _INT, _I64, _I64, _P, _SZ, _P], _INT),
    "qg_dequant_w8": ([_P, _P, _INT, _I64, _I64, _P, _INT, _P], _INT),
    "qg_swa_workspace_bytes": ([_I64] * 7, _SZ),
    "qg_swa_workspace_bytes_plan": ([_I64] * 9, _SZ),
    "qg_swa_attention": ([_P, _P, _P, _P, _P] + [_I64] * 7 + [ctypes.c_float, _P, _SZ, _P], _INT),
    "qg_swa_attention_plan": ([_P, _P, _P, _P, _P] + [_I64] * 7 + [ctypes.c_float, _I64, _I64, _P,
                                                                    _SZ, _P], _INT),
    "qg_read_stream": ([_P, _SZ, _INT, _P, _P], _INT),
    "qg_prepack_scales": ([_P, _INT, _I64, _I64, _P, _P], _INT),
    "qg_noalloc_scratch_bytes": ([], _SZ),
    "qgemm_w4a16_noalloc": ([_P, _P, _P, _INT, _P, _I64, _I64, _I64, _P], _INT),
}


class QGError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__("%s failed: %s" % (fn, STATUS.get(code, code)))
        self.code = code


def lib():
    """Load libqgemm.so (once). Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError(
                    "libqgemm.so is not built; run `python -m int8_group_quantized_amd.build`")
            L = ctypes.CDLL(_LIB_PATH)
            for name, (args, res) in _SIGNATURES.items():
                f = getattr(L, name)
                f.argtypes = args
                f.restype = res
            _lib = L
    return _lib


def library_path():
    return _LIB_PATH


def _check(fn, code):
    if code != 0:
        raise QGError(fn, code)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dt(t):
    if t.dtype == torch.bfloat16:
        return QG_BF16
    if t.dtype == torch.float16:
        return QG_F16
    if t.dtype == torch.float32:
        return QG_F32
    raise TypeError("unsupported dtype %s" % t.dtype)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous GPU tensors")


def packed_bytes(bits, K, N):
    return int(lib().qg_packed_bytes(bits, K, N))


def workspace_bytes(bits, M, K, N, plan=None):
    if plan is None:
        return int(lib().qg_workspace_bytes(bits, M, K, N))
    return int(lib().qg_workspace_bytes_plan(bits, M, K, N, *plan))


# Zero-initialised workspace per device, grown on demand. The library leaves
# its arrival counters at zero after every call, so the buffer is reusable on
# one stream.
_workspaces = {}


def workspace(device, nbytes):
    device = torch.device(device)
    key = device.index if device.index is not None else torch.cuda.current_device()
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _out_bytes(out, nbytes, what):
    if out.numel() * out.element_size() != nbytes:
        raise ValueError("%s must hold %d bytes" % (what, nbytes))


def _check_scales(scales, K, N):
    """Logical scales must be [K/128, N] (left to the library's status when
    K or N is not a valid shape)."""
    if K > 0 and N > 0 and K % 128 == 0 and N % 16 == 0 and tuple(scales.shape) != (K // 128, N):
        raise ValueError("scales must be [K/128, N] = %s, got %s" % ((K // 128, N),
                                                                     tuple(scales.shape)))


def rtn_scales(W, bits, out=None):
    """RTN scales [K/128, N]: fp16 (bits=4) or bf16 (bits=8), into out if given."""
    _need_cuda(W, out)
    K, N = W.shape
    sdt = torch.float16 if bits == 4 else torch.bfloat16
    if out is None:
        s = torch.empty((K // 128, N), dtype=sdt, device=W.device)
    else:
        if out.dtype != sdt:
            raise TypeError("out must be %s" % sdt)
        _out_bytes(out, (K // 128) * N * 2, "out")
        s = out
    fn = "qg_rtn_scales_w%d" % bits
    _check(fn, getattr(lib(), fn)(_ptr(W), _dt(W), K, N, _ptr(s), _stream(W)))
    return s


def pack_to_grid(W, scales, bits, out=None):
    """Q_s(W) under the given scales, packed; returns a uint8 tensor (out, if
    given: a contiguous GPU tensor of packed_bytes(bits, K, N) bytes)."""
    _need_cuda(W, scales, out)
    K, N = W.shape
    _check_scales(scales, K, N)
    if out is None:
        out = torch.empty(packed_bytes(bits, K, N), dtype=torch.uint8, device=W.device)
    elif out.numel() * out.element_size() != packed_bytes(bits, K, N):
        raise ValueError("out must hold packed_bytes(bits, K, N) bytes")
    fn = "qg_pack_to_grid_w%d" % bits
    _check(fn, getattr(lib(), fn)(_ptr(W), _dt(W), _ptr(scales), _dt(scales), K, N, _ptr(out),
                                  _stream(W)))
    return out


def pack_to_grid_w4(W, scales):
    return pack_to_grid(W, scales, 4)


def pack_to_grid_w8(W, scales):
    return pack_to_grid(W, scales, 8)


def prepack(codes, bits, out=None):
    _need_cuda(codes, out)
    if codes.dtype != torch.int8:
        raise TypeError("codes must be int8")
    K, N = codes.shape
    if out is None:
        out = torch.empty(packed_bytes(bits, K, N), dtype=torch.uint8, device=codes.device)
    else:
        _out_bytes(out, packed_bytes(bits, K, N), "out")
    fn = "qg_prepack_w%d" % bits
    _check(fn, getattr(lib(), fn)(_ptr(codes), K, N, _ptr(out), _stream(codes)))
    return out


def unpack(packed, K, N, bits, out=None):
    _need_cuda(packed, out)
    if packed_bytes(bits, K, N):
        _out_bytes(packed, packed_bytes(bits, K, N), "packed")
    if out is None:
        codes = torch.empty((K, N), dtype=torch.int8, device=packed.device)
    else:
        if out.dtype != torch.int8:
            raise TypeError("out must be int8")
        _out_bytes(out, K * N, "out")
        codes = out
    fn = "qg_unpack_w%d" % bits
    _check(fn, getattr(lib(), fn)(_ptr(packed), K, N, _ptr(codes), _stream(packed)))
    return codes


def _sdt(scales, cbm):
    d = _dt(scales)
    if d not in _CBM:
        raise TypeError("scales must be fp16 or bf16")
    return _CBM[d] if cbm else d


def check_weight(packed_w, scales, bits, K, N, scales_cbm=False):
    """Host-side agreement of a quantized weight with (bits, K, N): the packed
    bytes are qg_packed_bytes(bits, K, N), and the scales are [K/128, N]
    (logical order) or [N/16, K/128, 16] (column-block-major, from
    prepack_scales, which must then be passed with scales_cbm=True). Shapes
    the library rejects anyway (K not a multiple of 128, N of 16) are left
    to its status code."""
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    _sdt(scales, scales_cbm)
    nb = packed_bytes(bits, K, N)
    if nb == 0:
        return
    _out_bytes(packed_w, nb, "packed_w")
    G = K // 128
    if scales_cbm:
        if tuple(scales.shape) != (N // 16, G, 16):
            raise ValueError("column-block-major scales must be [N/16, K/128, 16] = %s, got %s"
                             % ((N // 16, G, 16), tuple(scales.shape)))
    else:
        if scales.dim() == 3:
            raise ValueError("3-D scales are the column-block-major order: pass scales_cbm=True")
        if tuple(scales.shape) != (G, N):
            raise ValueError("scales must be [K/128, N] = %s, got %s" % ((G, N), tuple(scales.shape)))


def prepack_scales(scales, out=None):
    """Column-block-major copy of scales [K/128, N] (qg_prepack_scales),
    shaped [N/16, K/128, 16]; pass it with scales_cbm=True to qgemm or
    qgemm_grouped, whose outputs equal those with the logical scales."""
    _need_cuda(scales, out)
    G, N = scales.shape
    if out is None:
        out = torch.empty((N // 16, G, 16), dtype=scales.dtype, device=scales.device)
    else:
        if out.dtype != scales.dtype:
            raise TypeError("out must have the dtype of scales")
        _out_bytes(out, G * N * 2, "out")
    _check("qg_prepack_scales", lib().qg_prepack_scales(_ptr(scales), _dt(scales), G * 128, N,
                                                        _ptr(out), _stream(scales)))
    return out


def qgemm(x, packed_w, scales, bits, N, out=None, plan=None, ws=None, scales_cbm=False):
    """out[M,N] = x[M,K] . (s (.) W_q) with fp32 accumulation; x and out are
    both bf16 or both fp16 (qgemm_w*a16 / qgemm_w*f16 in the C ABI).

    plan: optional (cols_per_wave, k_waves, splits) for the small-M kernel.
    ws: optional workspace tensor (zeroed before first use). Without it the
    call uses the device's shared workspace, which is safe for calls in
    order on one stream; calls that may run concurrently on different
    streams must each pass their own ws.
    scales_cbm: scales come from prepack_scales (column-block-major).
    """
    _need_cuda(x, packed_w, scales, out, ws)
    if x.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("x must be bf16 or fp16")
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    act = "a16" if x.dtype == torch.bfloat16 else "f16"
    M, K = x.shape
    check_weight(packed_w, scales, bits, K, N, scales_cbm)
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    elif out.dtype != x.dtype:
        raise TypeError("out must have the dtype of x")
    elif tuple(out.shape) != (M, N):
        raise ValueError("out must be [M, N] = %s" % ((M, N),))
    need = workspace_bytes(bits, M, K, N, plan)
    if ws is None and need > 0:
        ws = workspace(x.device, need)
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    if plan is None:
        fn = "qgemm_w%d%s" % (bits, act)
        code = getattr(lib(), fn)(_ptr(x), _ptr(packed_w), _ptr(scales), _sdt(scales, scales_cbm),
                                  _ptr(out), M, K, N, _ptr(ws), ws_bytes, _stream(x))
    else:
        fn = "qgemm_w%d%s_plan" % (bits, act)
        code = getattr(lib(), fn)(_ptr(x), _ptr(packed_w), _ptr(scales), _sdt(scales, scales_cbm),
                                  _ptr(out), M, K, N, _ptr(ws), ws_bytes, plan[0], plan[1],
                                  plan[2], _stream(x))
    _check(fn, code)
    return out


def qgemm_w4a16(x, packed_w, scales, N, out=None, plan=None, ws=None, scales_cbm=False):
    return qgemm(x, packed_w, scales, 4, N, out=out, plan=plan, ws=ws, scales_cbm=scales_cbm)


def qgemm_w8a16(x, packed_w, scales, N, out=None, plan=None, ws=None, scales_cbm=False):
    return qgemm(x, packed_w, scales, 8, N, out=out, plan=plan, ws=ws, scales_cbm=scales_cbm)


def dequant(packed_w, scales, bits, K, N, dtype=torch.bfloat16, out=None):
    """Dense W[K,N] = s (.) W_q, rounded once to dtype (bf16 or fp16)."""
    _need_cuda(packed_w, scales, out)
    check_weight(packed_w, scales, bits, K, N)
    if out is None:
        out = torch.empty((K, N), dtype=dtype, device=packed_w.device)
    elif tuple(out.shape) != (K, N):
        raise ValueError("out must be [K, N]")
    fn = "qg_dequant_w%d" % bits
    _check(fn, getattr(lib(), fn)(_ptr(packed_w), _ptr(scales), _dt(scales), K, N, _ptr(out),
                                  _dt(out), _stream(packed_w)))
    return out


def fake_quant(W, scales, bits, dtype=None, out=None):
    """s (.) Q_s(W) rounded once to dtype (bf16, fp16 or fp32; default W's)."""
    _need_cuda(W, scales, out)
    K, N = W.shape
    _check_scales(scales, K, N)
    if out is None:
        out = torch.empty((K, N), dtype=dtype or W.dtype, device=W.device)
    elif tuple(out.shape) != (K, N):
        raise ValueError("out must be [K, N]")
    fn = "qg_fake_quant_w%d" % bits
    _check(fn, getattr(lib(), fn)(_ptr(W), _dt(W), _ptr(scales), _dt(scales), K, N, _ptr(out),
                                  _dt(out), _stream(W)))
    return out


class FakeQuantSTE(torch.autograd.Function):
    """Forward: the fixed-grid fake quantizer on the GPU. Backward: the
    straight-through estimator, i.e. the incoming gradient unchanged (with
    respect to W; the frozen scales get none)."""

    @staticmethod
    def forward(ctx, W, scales, bits):
        return fake_quant(W, scales, bits)

    @staticmethod
    def backward(ctx, grad):
        return grad, None, None


def _items(weights, outs=None):
    return (GroupItem * len(weights))(*[
        GroupItem(p.data_ptr(), sc.data_ptr(), outs[i].data_ptr() if outs is not None else 0, n)
        for i, (p, sc, n) in enumerate(weights)])


def grouped_workspace_bytes(bits, M, K, weights):
    """Workspace bytes of a grouped call over weights [(packed_w, scales, N)]."""
    items = _items(weights)
    return int(lib().qg_workspace_bytes_grouped(bits, M, K, items, len(weights)))


def qgemm_grouped(x, weights, bits, outs=None, ws=None, scales_cbm=False):
    """One launch of several GEMMs sharing x: weights is a list of
    (packed_w, scales, N); returns the list of outputs [M, N_i]."""
    _need_cuda(x, ws)
    if x.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("x must be bf16 or fp16")
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    if not weights:
        raise ValueError("weights is empty")
    if outs is None:
        outs = [torch.empty((M, n), dtype=x.dtype, device=x.device) for _, _, n in weights]
    if len(outs) != len(weights):
        raise ValueError("one output per weight")
    sdt = weights[0][1].dtype
    for (p, sc, n), o in zip(weights, outs):
        _need_cuda(p, sc, o)
        if sc.dtype != sdt:
            raise TypeError("every item's scales must have one dtype (the ABI takes one)")
        check_weight(p, sc, bits, K, n, scales_cbm)
        if o.dtype != x.dtype or tuple(o.shape) != (M, n):
            raise ValueError("each output must be [M, N_i] in the dtype of x")
    items = _items(weights, outs)
    need = int(lib().qg_workspace_bytes_grouped(bits, M, K, items, len(weights)))
    if ws is None and need > 0:
        ws = workspace(x.device, need)
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    fn = "qgemm_w%d%s_grouped" % (bits, "a16" if x.dtype == torch.bfloat16 else "f16")
    _check(fn, getattr(lib(), fn)(_ptr(x), items, len(weights), _sdt(weights[0][1], scales_cbm), M, K,
                                  _ptr(ws), ws_bytes, _stream(x)))
    return outs


def swa_attention(q, k_cache, v_cache, seq_lens, window, scale=None, out=None, ws=None, chunk=0,
                  heads=0):
    """Drafter attention with a symmetric sliding window over a full KV cache.

    q [B, T, Hq, 128] bf16; k_cache, v_cache [B, S_max, Hkv, 128] bf16;
    seq_lens int32 [B] on the device (cache entries per sequence, the block's
    T included); window 0 for full attention. Returns out [B, T, Hq, 128].
    chunk (keys per workgroup) and heads (query heads per workgroup: 1, or
    2-6 / 8 for the shared K/V stream) override the library's split; 0 keeps
    its choice.
    """
    _need_cuda(q, k_cache, v_cache, seq_lens)
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16 or v_cache.dtype != torch.bfloat16:
        raise TypeError("q, k_cache and v_cache must be bf16")
    if seq_lens.dtype != torch.int32:
        raise TypeError("seq_lens must be int32")
    if not (q.is_contiguous() and k_cache.is_contiguous() and v_cache.is_contiguous()
            and seq_lens.is_contiguous()):
        raise ValueError("tensors must be contiguous")
    B, T, Hq, D = q.shape
    S_max, Hkv = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, S_max, Hkv, D) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache / v_cache must both be [B, S_max, Hkv, D]")
    if seq_lens.shape != (B,):
        raise ValueError("seq_lens must be [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    need = int(lib().qg_swa_workspace_bytes_plan(B, T, Hq, Hkv, D, S_max, window, chunk, heads))
    if ws is None and need > 0:
        ws = workspace(q.device, need)
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check("qg_swa_attention", lib().qg_swa_attention_plan(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(out), B, T, Hq, Hkv, D, S_max,
        window, scale, chunk, heads, _ptr(ws), ws_bytes, _stream(q)))
    return out


READ_PROBE_MARK = 0x9E3779B9


def read_stream(buf, workgroups, sink):
    """Measurement aid: read the bytes of the contiguous GPU tensor buf once
    (qg_read_stream). sink is a GPU tensor of at least 4 bytes; it receives
    READ_PROBE_MARK only when one thread's XOR of its words equals it."""
    _need_cuda(buf, sink)
    nbytes = buf.numel() * buf.element_size()
    _check("qg_read_stream", lib().qg_read_stream(_ptr(buf), nbytes, workgroups, _ptr(sink),
                                                  _stream(buf)))
