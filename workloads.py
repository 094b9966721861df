"""Seeded synthetic inputs and the workload shapes.

This module draws random inputs and nothing else: it holds none of the
quantization or GEMM arithmetic, so both the CPU oracle and the GPU library
can consume what it produces without sharing code. Conversions to 16-bit
floats use library casts (torch for bf16, numpy for fp16).

Shapes stand in for the pages' workloads (the inputs are synthetic; no
checkpoint or dataset is used):
  * hidden size 2560 of the Qwen3.5-4B target and its 5-layer DFlash drafter
    ("Quantize the Target, Quantize the Drafter", key contributions; drafter
    setup paragraph of arXiv 2607.04244);
  * M = 1 for plain decode, M = 16 for one anchor plus 15 drafted tokens
    (num_speculative_tokens 15 in the quickstart of the GPTQ-W4A16 model
    card; one 16-token draft block in the drafter-PTQ paragraph);
  * M = 8192 for the Long setting's 8,192-token prefill (speed paragraph);
  * fused gate/up N = 19456 with K = 2560, down K = 9728 with N = 2560, fused
    QKV N = 2560 + 2*512 = 3584.

Seeds: 1000*config + 10*shape_index + {0: weights, 1: activations}.

The drafter's sliding-window attention (Drafter SWA paragraph) runs one
16-token block of queries against a KV cache of the 8,192-token Long context
plus the block, with a window of 1,024 or 2,048 tokens or none. The head
layout follows the fused QKV width: 2560 = 20 query heads and 512 = 4 KV heads
of 128. Seeds: 6000 + 10*case + {0: q, 1: k, 2: v}.
"""

import numpy as np

WORKLOADS = {
    1: dict(name="tiny_w4a16", M=1, bits=4, shapes=[(256, 512)]),
    2: dict(name="decode_w4a16_m1", M=1, bits=4,
            shapes=[(2560, 19456), (9728, 2560)]),
    3: dict(name="verify_w4a16_m16", M=16, bits=4,
            shapes=[(2560, 19456), (9728, 2560), (2560, 3584)]),
    4: dict(name="drafter_w8a16_m16", M=16, bits=8,
            shapes=[(2560, 19456), (9728, 2560), (2560, 3584)]),
    5: dict(name="prefill_w4a16_m8192", M=8192, bits=4,
            shapes=[(2560, 19456), (9728, 2560)]),
}

ATTENTION = dict(name="drafter_swa_attention", T=16, Hq=20, Hkv=4, D=128, context=8192,
                 windows=(1024, 2048, 0))

SHAPE_NAMES = {(2560, 19456): "gate_up", (9728, 2560): "down",
               (2560, 3584): "qkv", (256, 512): "tiny"}


def seed_for(config, shape_index, which):
    return 1000 * config + 10 * shape_index + which


def weights(K, N, seed, dist="normal", std=0.02):
    """W ~ N(0, std) as float32 [K, N] (or Student-t with 3 dof times std)."""
    rng = np.random.default_rng(seed)
    if dist == "normal":
        w = rng.standard_normal((K, N), dtype=np.float32) * np.float32(std)
    elif dist == "student_t":
        w = (rng.standard_t(3, size=(K, N)) * std).astype(np.float32)
    else:
        raise ValueError(dist)
    return w


def to_bf16_bits(a):
    """float32 array -> bf16 bit patterns (uint16) via torch's cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def to_f16_bits(a):
    """float32 array -> fp16 bit patterns (uint16) via torch's cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def activations(M, K, seed, std=1.0, dtype="bf16"):
    """x ~ N(0, std) rounded to bf16 (or fp16 with dtype="f16"); returns
    uint16 bit patterns [M, K]."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32) * np.float32(std)
    return to_bf16_bits(x) if dtype == "bf16" else to_f16_bits(x)


def codes(K, N, bits, seed, lo=None, hi=None):
    """Uniform random integer codes as int8 [K, N] (full range by default)."""
    rng = np.random.default_rng(seed)
    if lo is None:
        lo, hi = (-8, 7) if bits == 4 else (-127, 127)
    return rng.integers(lo, hi + 1, size=(K, N), dtype=np.int64).astype(np.int8)


def scales(G, N, dtype, seed, center=0.0074, spread=0.3):
    """Positive log-normal scales around ``center`` as 16-bit patterns.

    The default centre is the typical max|w|/7 of N(0, 0.02) groups of 128.
    """
    rng = np.random.default_rng(seed)
    s = (center * np.exp(spread * rng.standard_normal((G, N)))).astype(np.float32)
    if dtype == "f16":
        return s.astype(np.float16).view(np.uint16)
    return to_bf16_bits(s)


def attention_inputs(B, T, Hq, Hkv, D, S_max, seed, std=1.0):
    """q [B, T, Hq, D] and k, v [B, S_max, Hkv, D], each ~ N(0, std) rounded
    to bf16; returns three uint16 bit-pattern arrays (seeds seed, seed+1,
    seed+2)."""
    out = []
    for i, shape in enumerate(((B, T, Hq, D), (B, S_max, Hkv, D), (B, S_max, Hkv, D))):
        rng = np.random.default_rng(seed + i)
        out.append(to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std)))
    return tuple(out)
