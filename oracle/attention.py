"""Reference for the drafter's sliding-window attention over a full KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: arXiv 2607.04244 ("Quantize the Target, Quantize the Drafter"), the
"Drafter SWA" paragraph of the experimental setup, with the drafter
optimisation paragraph of the method section that introduces SWA (after
Beltagy et al., 2020):
  * the window has a fixed size of 1,024 or 2,048 tokens;
  * the drafter's mask-token queries attend bidirectionally, so the window is
    symmetric around each query, not a causal left-only window;
  * the window exists only inside the attention kernel: the KV cache keeps
    every position (nothing evicted or rotated);
  * a sequence no longer than the window falls back to full attention.
The drafter setup paragraph fixes one draft block at 16 tokens.

Readings taken where the page is silent (each is listed with the others in
the design notes):
  * a window of W tokens reaches W // 2 positions to each side of the query
    (|p - j| <= W // 2), the Longformer convention the page cites;
  * "sequence" means every cache position of the request, the block's own T
    entries included, and the block's queries sit at the last T positions;
  * W = 0 means no window (full attention);
  * query head h reads KV head h // (Hq / Hkv) (grouped-query attention);
  * scores are q . k times the caller's softmax scale, then a plain softmax.

The computation is the definition written out in float64: for each query, the
dot products with its visible keys, the softmax, and the weighted sum of the
visible values. Inputs arrive as float arrays already decoded exactly from
bf16; the result is float64, before any output rounding.
"""

import numpy as np


def visible_range(seq_len, T, t, window):
    """[lo, hi): the cache positions query t (0 <= t < T) of the block sees.

    The block occupies positions seq_len - T .. seq_len - 1.
    """
    p = seq_len - T + t
    if window == 0 or seq_len <= window:
        return 0, seq_len
    half = window // 2
    return max(0, p - half), min(seq_len, p + half + 1)


def swa_attention(q, k, v, seq_lens, window, scale):
    """q: [B, T, Hq, D]; k, v: [B, S_max, Hkv, D]; seq_lens: B ints with
    T <= seq_lens[b] <= S_max. Returns float64 [B, T, Hq, D].

    Cache rows at or beyond seq_lens[b] are never read.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    assert Hq % Hkv == 0
    group = Hq // Hkv
    out = np.zeros((B, T, Hq, D), dtype=np.float64)
    for b in range(B):
        S = int(seq_lens[b])
        assert T <= S <= k.shape[1]
        for t in range(T):
            lo, hi = visible_range(S, T, t, window)
            for h in range(Hq):
                kv = h // group
                scores = (k[b, lo:hi, kv, :] @ q[b, t, h, :]) * scale
                w = np.exp(scores - scores.max())
                out[b, t, h, :] = (w / w.sum()) @ v[b, lo:hi, kv, :]
    return out
