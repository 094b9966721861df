"""The packed-weight layout, element by element.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the container ("compressed-tensors pack-quantized", W8A16
model card table; "W4A16 compressed-tensors format", QAD paragraph of arXiv
2607.04244) but give no bit layout, so the library defines its own. This
module states it as a map from a logical code position (k, n) of the
row-major [K, N] code matrix to a byte and bit position, and applies that map
one element at a time. The map is:

  nb = n // 16, g = k // 128, r = k % 128
  j  = r // 32            (which 32-deep K step inside the group)
  h  = (r % 32) // 8      (which 8-deep slice of that step)
  i  = r % 8              (element inside the slice)
  lane l = 16*h + n % 16
  tile t = nb * (K/128) + g

  INT4 (tile = 1024 bytes):
    byte  = 1024*t + 16*l + 4*j + p // 2,  with p = i // 2 + 4*(i % 2)
    bits  = low nibble if p is even, high nibble if p is odd
    value = q + 8 (offset binary, 0..15)
  INT8 (tile = 2048 bytes):
    byte  = 2048*t + 32*l + 8*j + i
    value = q as an 8-bit two's complement byte
"""

import numpy as np

from .quant import GROUP

TILE_COLS = 16


def packed_bytes(bits, K, N):
    """Bytes of packed codes: K*N/2 for INT4, K*N for INT8."""
    return K * N // 2 if bits == 4 else K * N


def _check(K, N):
    if K <= 0 or N <= 0 or K % GROUP or N % TILE_COLS:
        raise ValueError("K must be a positive multiple of 128, N of 16")


def position(bits, K, k, n):
    """(byte offset, shift in bits) of code (k, n); k, n may be arrays."""
    k = np.asarray(k, dtype=np.int64)
    n = np.asarray(n, dtype=np.int64)
    G = K // GROUP
    nb, g, r = n // TILE_COLS, k // GROUP, k % GROUP
    j, h, i = r // 32, (r % 32) // 8, r % 8
    lane = 16 * h + n % TILE_COLS
    tile = nb * G + g
    if bits == 4:
        p = i // 2 + 4 * (i % 2)
        return 1024 * tile + 16 * lane + 4 * j + p // 2, 4 * (p % 2)
    if bits == 8:
        return 2048 * tile + 32 * lane + 8 * j + i, np.zeros_like(k)
    raise ValueError(bits)


def pack(codes, bits):
    """Logical int8 codes [K, N] -> packed uint8 bytes (flat)."""
    codes = np.asarray(codes, dtype=np.int8)
    K, N = codes.shape
    _check(K, N)
    kk, nn = np.meshgrid(np.arange(K), np.arange(N), indexing="ij")
    byte, shift = position(bits, K, kk.ravel(), nn.ravel())
    out = np.zeros(packed_bytes(bits, K, N), dtype=np.uint16)
    if bits == 4:
        lo, hi = -8, 7
        c = codes.ravel().astype(np.int64)
        if c.min() < lo or c.max() > hi:
            raise ValueError("INT4 code out of [-8, 7]")
        u = (c + 8).astype(np.uint16) << shift.astype(np.uint16)
        np.add.at(out, byte, u)          # the two nibbles of a byte never overlap
    else:
        out[byte] = codes.ravel().view(np.uint8)
    return out.astype(np.uint8)


def unpack(packed, bits, K, N):
    """Packed uint8 bytes -> logical int8 codes [K, N]."""
    _check(K, N)
    packed = np.asarray(packed, dtype=np.uint8).ravel()
    if packed.size != packed_bytes(bits, K, N):
        raise ValueError("packed size does not match K, N")
    kk, nn = np.meshgrid(np.arange(K), np.arange(N), indexing="ij")
    byte, shift = position(bits, K, kk.ravel(), nn.ravel())
    if bits == 4:
        u = (packed[byte].astype(np.int64) >> shift) & 0xF
        return (u - 8).astype(np.int8).reshape(K, N)
    return packed[byte].view(np.int8).reshape(K, N)


def storage_bytes(bits, n_params, scale_bytes=2):
    """Bytes for n_params weights: the codes plus one 2-byte scale per 128."""
    return n_params * bits / 8 + n_params / GROUP * scale_bytes


def scales_cbm(scales):
    """Column-block-major order of scales [G, N] (the library's own storage
    order for qg_prepack_scales; the pages fix none): element (g, n) moves to
    flat position ((n // 16) * G + g) * 16 + n % 16, written out one element
    at a time. Returns a flat array of the same dtype."""
    G, N = scales.shape
    if N % 16:
        raise ValueError("N must be a multiple of 16")
    out = np.empty(G * N, dtype=scales.dtype)
    for g in range(G):
        for n in range(N):
            out[((n // 16) * G + g) * 16 + n % 16] = scales[g, n]
    return out
