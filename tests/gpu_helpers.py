"""Helpers for the GPU parity tests: host <-> device conversions of the
seeded inputs. No arithmetic of the method lives here."""

import numpy as np
import torch

DEV = "cuda:0"


def dev_bf16(bits):
    """uint16 bf16 patterns -> bf16 tensor on the GPU (bit-preserving)."""
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).view(torch.bfloat16).to(DEV)


def dev_f16(bits):
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).view(torch.float16).to(DEV)


def dev_scales(bits, dtype):
    return dev_f16(bits) if dtype == "f16" else dev_bf16(bits)


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dev_i8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int8)).to(DEV)


def host_u16(t):
    """bf16 / fp16 tensor -> uint16 bit patterns on the host."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def host_u8(t):
    return t.detach().cpu().contiguous().numpy().view(np.uint8).copy()


def host_i8(t):
    return t.detach().cpu().contiguous().numpy().astype(np.int8)


# ---------------------------------------------------------------------------
# Poisoned outputs and guard bands. Every output a GPU test hands to the
# library sits inside a larger allocation: GUARD bytes of a canary pattern on
# each side, and the output itself pre-filled with a poison value. A kernel
# that leaves an element unwritten then shows the poison (a NaN for float
# outputs, which no tolerance test accepts; for bit-exact outputs the case is
# run under two different poison bytes, which no single expected value can
# match twice), and a kernel that writes outside its output breaks a canary.

GUARD = 4096
CANARY = 0xC5
NAN16 = {torch.bfloat16: 0x7FC0, torch.float16: 0x7E00}
NAN32 = 0x7FC00000


class Guarded:
    """A contiguous GPU tensor of `shape` and `dtype` with canary bands of
    GUARD bytes before and after it. `poison` is a byte value (int) or "nan"
    (16-bit or 32-bit float NaN for float dtypes)."""

    def __init__(self, shape, dtype, poison="nan"):
        self.shape, self.dtype = tuple(shape), dtype
        n = int(np.prod(self.shape)) if self.shape else 1
        self.nbytes = n * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((GUARD + self.nbytes + GUARD,), CANARY, dtype=torch.uint8, device=DEV)
        body = self.buf[GUARD:GUARD + self.nbytes]
        if poison == "nan":
            if dtype in NAN16:
                body.view(torch.int16).fill_(NAN16[dtype])
            elif dtype == torch.float32:
                body.view(torch.int32).fill_(NAN32)
            else:
                raise ValueError("nan poison needs a float dtype")
        else:
            body.fill_(int(poison))
        self.t = body.view(dtype).view(self.shape)

    def guards_intact(self):
        torch.cuda.synchronize()
        front = self.buf[:GUARD]
        back = self.buf[GUARD + self.nbytes:]
        return bool((front == CANARY).all()) and bool((back == CANARY).all())

    def check(self, what=""):
        assert self.guards_intact(), "write outside the output %s" % what
        return self.t


class GuardedWorkspace:
    """A workspace of `need` bytes for the GEMM / attention entry points: the
    64 KiB of arrival counters zeroed (as the library requires before first
    use), everything after them (split-K partials, prefill offsets, attention
    chunk results, all written before they are read) poisoned with fp32 NaN,
    and a canary band after it. After a call the counters must be back at
    zero and the canary intact."""

    COUNTERS = 65536

    def __init__(self, need):
        self.need = int(need)
        self.buf = torch.full((self.need + GUARD,), CANARY, dtype=torch.uint8, device=DEV)
        body = self.buf[:self.need]
        if self.need:
            c = min(self.COUNTERS, self.need)
            body[:c].zero_()
            if self.need > c:
                body[c:].view(torch.int32).fill_(NAN32)
        # the library sees exactly `need` bytes (a view of the front)
        self.t = body if self.need else None

    def check(self, what=""):
        torch.cuda.synchronize()
        assert bool((self.buf[self.need:] == CANARY).all()), "write past the workspace %s" % what
        c = min(self.COUNTERS, self.need)
        if c:
            assert int(torch.count_nonzero(self.buf[:c])) == 0, "counters not left at zero %s" % what


def written_twice(fn, shape, dtype, what=""):
    """Run fn(out) into an output poisoned with 0xA5 bytes, then into one
    poisoned with 0x5A bytes, both between canary bands. The two results must
    be identical, so every byte was written (an unwritten byte would keep two
    different poisons), and the canaries intact. Returns the output."""
    res = []
    for poison in (0xA5, 0x5A):
        g = Guarded(shape, dtype, poison=poison)
        fn(g.t)
        res.append(g.check(what).clone())
    assert torch.equal(res[0].view(torch.uint8), res[1].view(torch.uint8)), \
        "output bytes left unwritten %s" % what
    return res[0]


def guarded_gemm(x_dev, pg, sd, bits, N, *, plan=None, cbm=False, what=""):
    """One GEMM call into a NaN-poisoned output between canary bands, with a
    workspace whose data part is NaN-poisoned and followed by a canary band;
    returns the output's 16-bit patterns on the host after both checks."""
    import int8_group_quantized_amd as q
    M, K = x_dev.shape
    out = Guarded((M, N), x_dev.dtype)
    ws = GuardedWorkspace(q.workspace_bytes(bits, M, K, N, plan))
    q.qgemm(x_dev, pg, sd, bits, N, out=out.t, plan=plan, ws=ws.t, scales_cbm=cbm)
    got = out.check(what)
    ws.check(what)
    return host_u16(got)
