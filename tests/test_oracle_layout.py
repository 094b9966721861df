"""Pins for oracle.layout: the packed tile layout and the storage model.

The layout is this library's own (the pages name only the container format:
"compressed-tensors pack-quantized" in the W8A16 model card table). It is
pinned by hand-derived byte positions, by one-hot patterns showing that every
code lands in exactly one distinct nibble or byte, by round trips in both
directions, and by the storage sizes the pages print.
"""

import json
import os

import numpy as np
import pytest

from oracle import layout

GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("bits", [4, 8])
def test_hand_derived_positions(bits):
    gold = json.load(open(os.path.join(GOLD, "layout_positions.json")))
    K, N = gold["K"], gold["N"]
    lo = -8 if bits == 4 else -127
    for e in gold["int%d" % bits]:
        codes = np.zeros((K, N), dtype=np.int8)
        if bits == 4:
            codes[:] = -8                  # offset-binary nibble 0 everywhere
            codes[e["k"], e["n"]] = 7      # nibble 15 at one place
            p = layout.pack(codes, 4)
            nz = np.flatnonzero(p)
            assert nz.tolist() == [e["byte"]], e
            assert int(p[e["byte"]]) == 0xF << e["shift"], e
        else:
            codes[e["k"], e["n"]] = lo
            p = layout.pack(codes, 8)
            nz = np.flatnonzero(p)
            assert nz.tolist() == [e["byte"]], e
            assert int(p[e["byte"]]) == (lo & 0xFF)


@pytest.mark.parametrize("bits", [4, 8])
def test_one_hot_positions_are_distinct_and_complete(bits):
    """Every code of a 2-group x 2-block shape owns one distinct nibble/byte."""
    K, N = 256, 32
    base = -8 if bits == 4 else 0
    seen = set()
    for k in range(K):
        codes = np.full((K, N), base, dtype=np.int8)
        # row k gets a non-zero stored value in every column
        codes[k, :] = np.arange(N) % 7 + 1 + base
        p = layout.pack(codes, bits)
        if bits == 4:
            nib = np.stack([p & 0xF, p >> 4], axis=1).ravel()
            idx = np.flatnonzero(nib)
        else:
            idx = np.flatnonzero(p)
        assert idx.size == N
        for i in idx.tolist():
            assert i not in seen
            seen.add(i)
    total = layout.packed_bytes(bits, K, N) * (2 if bits == 4 else 1)
    assert len(seen) == total


@pytest.mark.parametrize("bits", [4, 8])
def test_round_trips(bits):
    rng = np.random.default_rng(3)
    K, N = 384, 48
    lo, hi = (-8, 7) if bits == 4 else (-128, 127)
    c = rng.integers(lo, hi + 1, size=(K, N)).astype(np.int8)
    assert np.array_equal(layout.unpack(layout.pack(c, bits), bits, K, N), c)
    # every byte value, every position: pack(unpack(p)) == p
    nbytes = layout.packed_bytes(bits, K, N)
    p = (np.arange(nbytes) * 37 % 256).astype(np.uint8)
    assert np.array_equal(layout.pack(layout.unpack(p, bits, K, N), bits), p)


def test_int4_all_values_each_position_of_a_tile():
    """Every nibble value at every position of one 1 KiB tile."""
    K, N = 128, 16
    for v in range(-8, 8):
        c = np.full((K, N), v, dtype=np.int8)
        p = layout.pack(c, 4)
        assert np.all(p == ((v + 8) | ((v + 8) << 4)))
        assert np.array_equal(layout.unpack(p, 4, K, N), c)


def test_bad_shapes_rejected():
    with pytest.raises(ValueError):
        layout.pack(np.zeros((100, 16), dtype=np.int8), 4)
    with pytest.raises(ValueError):
        layout.pack(np.zeros((128, 10), dtype=np.int8), 8)
    with pytest.raises(ValueError):
        layout.pack(np.full((128, 16), 9, dtype=np.int8), 4)


def test_storage_model_matches_printed_sizes():
    g = json.load(open(os.path.join(GOLD, "storage_w8a16_drafter.json")))
    n = g["params"]
    bf16_gib = n * 2 / 2**30
    w8_mib = layout.storage_bytes(8, n) / 2**20
    assert abs(bf16_gib - g["bf16_on_disk_GB"]) < 0.005
    # codes + scales come to 520.1 MiB; the printed 521 MB also holds the
    # unquantized norms, so the model must land just below it
    assert g["w8a16_on_disk_MB"] - 2 < w8_mib <= g["w8a16_on_disk_MB"]
    # a layout with 4-byte scales or per-64 groups would not fit the print
    assert (n + n / 128 * 4) / 2**20 > g["w8a16_on_disk_MB"] + 2
    assert (n + n / 64 * 2) / 2**20 > g["w8a16_on_disk_MB"] + 2
    # INT4 costs 0.515625 bytes per weight
    assert layout.storage_bytes(4, 128) == 66


def test_scales_cbm_hand_derived_and_a_permutation():
    """Hand-worked positions of the column-block-major scale order for G = 3,
    N = 32: (g, n) -> ((n // 16) * 3 + g) * 16 + n % 16."""
    G, N = 3, 32
    s = np.arange(G * N, dtype=np.uint16).reshape(G, N)       # value = g * 32 + n
    flat = layout.scales_cbm(s)
    assert flat[0] == 0            # (0, 0)
    assert flat[15] == 15          # (0, 15)
    assert flat[16] == 32          # (1, 0): block 0, group 1
    assert flat[47] == 79          # (2, 15)
    assert flat[48] == 16          # (0, 16): block 1 starts after 3 groups of block 0
    assert flat[95] == 95          # (2, 31)
    assert sorted(flat.tolist()) == list(range(G * N))         # a permutation
    with pytest.raises(ValueError):
        layout.scales_cbm(np.zeros((2, 24), dtype=np.uint16))
