"""Pins for the oracle's sliding-window attention (attention.swa_attention).

Pinned by a table of visible key ranges worked by hand from the Drafter SWA
paragraph of arXiv 2607.04244 (tests/golden/swa_windows.json), by the closed
form of attention with equal scores (the plain mean of the visible values,
which with v[j] = j is the window's midpoint), by torch's own
scaled_dot_product_attention in float64 (with masks taken from the hand
table, and with its grouped-query head mapping), by the cache rows past the
sequence end never being read, and by a dominant key taking all the weight.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import attention

HERE = os.path.dirname(os.path.abspath(__file__))
CASES = json.load(open(os.path.join(HERE, "golden", "swa_windows.json")))["cases"]


def _sdpa(q, k, v, mask, scale):
    """torch SDPA in float64 for one sequence: q [T, Hq, D], k/v [S, Hkv, D],
    mask [T, S] bool or None."""
    qt = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0)
    kt = torch.from_numpy(k).permute(1, 0, 2).unsqueeze(0)
    vt = torch.from_numpy(v).permute(1, 0, 2).unsqueeze(0)
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale,
                                                          enable_gqa=True)
    return o.squeeze(0).permute(1, 0, 2).numpy()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "S%d_T%d_W%d" % (c["seq_len"], c["T"], c["window"]))
def test_windows_match_hand_table(case):
    for t, (lo, hi) in enumerate(case["ranges"]):
        assert attention.visible_range(case["seq_len"], case["T"], t, case["window"]) == (lo, hi)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "S%d_T%d_W%d" % (c["seq_len"], c["T"], c["window"]))
def test_equal_scores_average_the_window(case):
    S, T, W = case["seq_len"], case["T"], case["window"]
    Hq, Hkv, D = 2, 1, 3
    q = np.zeros((1, T, Hq, D))
    k = np.random.default_rng(1).standard_normal((1, S, Hkv, D))
    v = np.broadcast_to(np.arange(S, dtype=np.float64)[None, :, None, None], (1, S, Hkv, D)).copy()
    out = attention.swa_attention(q, k, v, [S], W, 0.125)
    for t, (lo, hi) in enumerate(case["ranges"]):
        np.testing.assert_allclose(out[0, t], (lo + hi - 1) / 2.0, rtol=1e-12)


@pytest.mark.parametrize("case", [c for c in CASES if c["seq_len"] <= 3000],
                         ids=lambda c: "S%d_T%d_W%d" % (c["seq_len"], c["T"], c["window"]))
def test_matches_torch_with_hand_masks(case):
    S, T, W = case["seq_len"], case["T"], case["window"]
    Hq, Hkv, D = 6, 2, 16
    rng = np.random.default_rng(S * 31 + W)
    q = rng.standard_normal((1, T, Hq, D))
    k = rng.standard_normal((1, S, Hkv, D))
    v = rng.standard_normal((1, S, Hkv, D))
    mask = np.zeros((T, S), dtype=bool)
    for t, (lo, hi) in enumerate(case["ranges"]):
        mask[t, lo:hi] = True
    ref = _sdpa(q[0], k[0], v[0], mask, 0.3)
    out = attention.swa_attention(q, k, v, [S], W, 0.3)
    np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("window", [0, 64, 1000])
def test_full_attention_matches_torch_ragged_batch(window):
    # window 0, or a window at least as long as every sequence: plain
    # attention over each sequence's own cache prefix.
    B, T, Hq, Hkv, D, S_max = 3, 5, 8, 2, 16, 64
    rng = np.random.default_rng(7)
    q = rng.standard_normal((B, T, Hq, D))
    k = rng.standard_normal((B, S_max, Hkv, D))
    v = rng.standard_normal((B, S_max, Hkv, D))
    lens = [37, 64, 5]
    out = attention.swa_attention(q, k, v, lens, window, 1 / np.sqrt(D))
    for b, S in enumerate(lens):
        ref = _sdpa(q[b], k[b, :S], v[b, :S], None, 1 / np.sqrt(D))
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-13)


def test_cache_past_sequence_end_is_not_read():
    B, T, Hq, Hkv, D, S_max = 2, 4, 4, 2, 8, 40
    rng = np.random.default_rng(3)
    q = rng.standard_normal((B, T, Hq, D))
    k = rng.standard_normal((B, S_max, Hkv, D))
    v = rng.standard_normal((B, S_max, Hkv, D))
    lens = [23, 31]
    clean = attention.swa_attention(q, k, v, lens, 8, 0.5)
    for b, S in enumerate(lens):
        k[b, S:] = np.nan
        v[b, S:] = np.nan
    dirty = attention.swa_attention(q, k, v, lens, 8, 0.5)
    assert np.isfinite(dirty).all()
    np.testing.assert_array_equal(dirty, clean)


def test_dominant_key_takes_all_weight():
    T, Hq, Hkv, D, S = 1, 1, 1, 4, 50
    rng = np.random.default_rng(5)
    k = rng.standard_normal((1, S, Hkv, D)) * 0.01
    v = rng.standard_normal((1, S, Hkv, D))
    j = 45                              # inside the window of the query at 49 (half = 8)
    k[0, j, 0] = [10.0, 0, 0, 0]
    q = np.zeros((1, T, Hq, D))
    q[0, 0, 0, 0] = 10.0                # score 100 * scale against key j, ~0 elsewhere
    out = attention.swa_attention(q, k, v, [S], 16, 1.0)
    np.testing.assert_allclose(out[0, 0, 0], v[0, j, 0], rtol=0, atol=1e-30 + 1e-40 + np.exp(-90) * 10)
    # the same key outside the window (position 30 < 49 - 8) has no effect
    k2 = k.copy()
    k2[0, j, 0] = k[0, 0, 0]
    k2[0, 30, 0] = [10.0, 0, 0, 0]
    out2 = attention.swa_attention(q, k2, v, [S], 16, 1.0)
    assert np.abs(out2[0, 0, 0] - v[0, 30, 0]).max() > 0.1
