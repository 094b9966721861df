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
