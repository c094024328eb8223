"""fp64 definition of sliding-window decode attention (GQA family).

TEST INFRASTRUCTURE ONLY -- see the package docstring. The product path never
imports this module.

Sources (page title -- section):

* "Grouped-Query Attention: Fewer KV Heads, Same Quality" -- "GQA and Related
  KV-Head Choices in Modern Architectures": Mistral 7B combines grouped KV heads
  with sliding-window attention of width w = 4096, so the cache it keeps is
  bounded by w positions whatever the sequence length.
* "Attention variants: MQA, GQA, and MLA" -- "Traps and misconceptions": the
  window is an axis independent of KV-head sharing (Mistral uses both).

Reading of what the pages leave open: a decode token at
sequence length n attends over the last ``window`` cached positions,
t in [max(0, n - window), n); ``window >= n`` is the full decode. Everything
else (group map, scale, clamping of n, padding never read) is as in
``attention.decode_gqa``.
"""

from __future__ import annotations

import numpy as np

from .attention import _f64, _lens, _softmax_1d, clamp_len


def window_start(n: int, window: int) -> int:
    """First attended position for a row of length n."""
    return max(0, int(n) - int(window))


def decode_gqa_window(q, k_cache, v_cache, seq_lens, scale: float, window: int) -> np.ndarray:
    """decode_gqa restricted to the positions [max(0, n - window), n) of each row."""
    if int(window) < 1:
        raise ValueError("window must be at least 1")
    B, h_q, D = q.shape
    _, h_kv, T_max, _ = k_cache.shape
    Dv = v_cache.shape[-1]
    g = h_q // h_kv
    lens = _lens(seq_lens, B)
    out = np.zeros((B, h_q, Dv), dtype=np.float64)
    for b in range(B):
        n = clamp_len(lens[b], T_max)
        lo = window_start(n, window)
        if n == 0:
            continue
        for j in range(h_kv):
            K = _f64(k_cache[b, j, lo:n])
            V = _f64(v_cache[b, j, lo:n])
            Q = _f64(q[b, j * g:(j + 1) * g])
            W = _softmax_1d(scale * (Q @ K.T))
            out[b, j * g:(j + 1) * g] = W @ V
    return out
