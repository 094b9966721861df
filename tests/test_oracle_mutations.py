"""Planted mistakes in the oracle must trip its pins.

Each case swaps one oracle function for a plausibly wrong variant (on the CPU,
for the duration of one test) and runs the pins that should catch it. A
mutation that every pin let through would mean the oracle is not pinned
where it matters.
"""

import numpy as np
import pytest

from oracle import attention, gemm, layout, numerics, quant
import test_oracle_attention as ta
import test_oracle_dequant as td
import test_oracle_gemm as tg
import test_oracle_layout as tl
import test_oracle_numerics as tn
import test_oracle_quant as tq


def _q_s_variant(kind):
    orig = quant.q_s

    def q_s(W, scale_values, bits):
        W = np.asarray(W, dtype=np.float32)
        s = quant.expand_groups(np.asarray(scale_values, dtype=np.float64),
                                W.shape[0]).astype(np.float32)
        lo, hi = quant.RANGE[bits]
        with np.errstate(all="ignore"):
            if kind == "reciprocal":
                t = W * (np.float32(1.0) / s)
            else:
                t = W / s
        if kind == "half_away":
            q = np.sign(t) * np.floor(np.abs(t) + 0.5)
        elif kind == "truncate":
            q = np.trunc(t)
        else:
            q = np.rint(t)
        if kind == "symmetric7":
            lo = -hi
        q = np.clip(q, lo, hi)
        q = np.where((s == 0) | np.isnan(t), 0.0, q)
        return q.astype(np.int8)
    return q_s


def _expect_failure(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


@pytest.mark.parametrize("kind", ["half_away", "truncate", "symmetric7"])
def test_rounding_mutations_caught(monkeypatch, kind):
    monkeypatch.setattr(quant, "q_s", _q_s_variant(kind))
    _expect_failure(tq.test_ties_follow_hand_table, 4)


def test_reciprocal_multiply_caught(monkeypatch):
    monkeypatch.setattr(quant, "q_s", _q_s_variant("reciprocal"))
    _expect_failure(tq.test_ties_many_scales_need_true_division)


def test_wrong_rtn_divisor_caught(monkeypatch):
    monkeypatch.setattr(quant, "RTN_DIVISOR", {4: 8.0, 8: 128.0})
    _expect_failure(tq.test_rtn_largest_code_hits_range_end, 4)
    _expect_failure(tq.test_rtn_scales_brute_force, 8)


def test_nibble_order_mutation_caught(monkeypatch):
    orig = layout.position

    def position(bits, K, k, n):
        byte, shift = orig(bits, K, k, n)
        if bits == 4:   # straight nibble order inside each dword
            k = np.asarray(k)
            i = k % 8
            j = (k % 128) // 32
            base = byte - (np.where(i % 2 == 0, i // 2, 4 + i // 2) // 2)
            return base + i // 2, 4 * (i % 2)
        return byte, shift
    monkeypatch.setattr(layout, "position", position)
    _expect_failure(tl.test_hand_derived_positions, 4)


def test_lane_map_mutation_caught(monkeypatch):
    orig = layout.position

    def position(bits, K, k, n):
        # columns and 8-deep slices swapped in the lane index
        k = np.asarray(k)
        n = np.asarray(n)
        h = (k % 32) // 8
        byte, shift = orig(bits, K, k, n)
        stride = 16 if bits == 4 else 32
        lane = 16 * h + n % 16
        lane2 = 4 * (n % 16) + h
        return byte + (lane2 - lane) * stride, shift
    monkeypatch.setattr(layout, "position", position)
    _expect_failure(tl.test_hand_derived_positions, 8)


def test_scale_axis_mutations_caught(monkeypatch):
    orig = quant.expand_groups

    def reversed_groups(s, K):
        return orig(np.asarray(s)[::-1], K)
    monkeypatch.setattr(quant, "expand_groups", reversed_groups)
    _expect_failure(tg.test_one_hot_power_of_two_rows)


def test_dropped_scale_caught(monkeypatch):
    def dequant(codes, scale_values):
        return np.asarray(codes).astype(np.float64)
    monkeypatch.setattr(gemm, "dequant", dequant)
    _expect_failure(tg.test_identity_probe, 4)


def test_transposed_activation_caught(monkeypatch):
    orig = gemm.gemm_ref

    def gemm_ref(x_bits, codes, scale_bits, scale_dtype):
        x = numerics.bf16_to_f64(x_bits)
        w = quant.dequant(codes, numerics.scale_bits_to_f64(scale_bits, scale_dtype))
        return (x[::-1] @ w)             # rows of x taken in the wrong order
    monkeypatch.setattr(gemm, "gemm_ref", gemm_ref)
    _expect_failure(tg.test_one_hot_power_of_two_rows)


def test_bf16_truncation_caught(monkeypatch):
    def f32_to_bf16(x):
        x = np.asarray(x, dtype=np.float32)
        return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    monkeypatch.setattr(numerics, "f32_to_bf16", f32_to_bf16)
    _expect_failure(tn.test_bf16_ties_by_hand)


def test_f16_rounding_toward_zero_caught(monkeypatch):
    def f32_to_f16(x):
        x = np.asarray(x, dtype=np.float32)
        with np.errstate(over="ignore"):
            h = x.astype(np.float16)
        over = np.abs(h.astype(np.float32)) > np.abs(x)
        return np.where(over, np.nextafter(h, np.float16(0)), h).astype(np.float16).view(np.uint16)
    monkeypatch.setattr(numerics, "f32_to_f16", f32_to_f16)
    _expect_failure(td.test_golden_cases)


def test_f16_activations_decoded_as_bf16_caught(monkeypatch):
    monkeypatch.setattr(numerics, "act_to_f64", lambda bits, dtype: numerics.bf16_to_f64(bits))
    _expect_failure(td.test_f16_one_hot_rows)


def test_dequant_truncated_to_bf16_caught(monkeypatch):
    def f64_exact_to_bf16(x):
        x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
        return (x32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    monkeypatch.setattr(numerics, "f64_exact_to_bf16", f64_exact_to_bf16)
    _expect_failure(td.test_golden_cases)


def _window_variant(kind):
    def visible_range(seq_len, T, t, window):
        p = seq_len - T + t
        full = window == 0 if kind == "no_fallback" else (window == 0 or seq_len <= window)
        if full:
            return 0, seq_len
        half = window // 2
        if kind == "exclusive":
            return max(0, p - half + 1), min(seq_len, p + half)
        if kind == "causal":
            return max(0, p - window + 1), p + 1
        if kind == "whole_window_each_side":
            return max(0, p - window), min(seq_len, p + window + 1)
        return max(0, p - half), min(seq_len, p + half + 1)
    return visible_range


@pytest.mark.parametrize("kind", ["exclusive", "causal", "no_fallback", "whole_window_each_side"])
def test_window_mutations_caught(monkeypatch, kind):
    monkeypatch.setattr(attention, "visible_range", _window_variant(kind))
    case = {"exclusive": 0, "causal": 0, "no_fallback": 3, "whole_window_each_side": 5}[kind]
    _expect_failure(ta.test_equal_scores_average_the_window, ta.CASES[case])


def _attention_variant(kind):
    def swa_attention(q, k, v, seq_lens, window, scale):
        q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
        B, T, Hq, D = q.shape
        Hkv = k.shape[2]
        out = np.zeros((B, T, Hq, D))
        for b in range(B):
            S = int(seq_lens[b])
            for t in range(T):
                lo, hi = attention.visible_range(S, T, t, window)
                for h in range(Hq):
                    kv = h % Hkv if kind == "head_modulo" else h // (Hq // Hkv)
                    sc = 1.0 if kind == "no_scale" else scale
                    s_ = (k[b, lo:hi, kv] @ q[b, t, h]) * sc
                    w = np.exp(s_ - s_.max())
                    out[b, t, h] = (w / w.sum()) @ v[b, lo:hi, kv]
        return out
    return swa_attention


@pytest.mark.parametrize("kind", ["head_modulo", "no_scale"])
def test_attention_mutations_caught(monkeypatch, kind):
    monkeypatch.setattr(attention, "swa_attention", _attention_variant(kind))
    _expect_failure(ta.test_full_attention_matches_torch_ragged_batch, 0)
