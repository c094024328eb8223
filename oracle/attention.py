"""fp64 definition of single-token decode attention (GQA family and absorbed MLA).

TEST INFRASTRUCTURE ONLY -- see the package docstring. The product path never
imports this module.

Sources (page title -- section):

* "Attention variants: MQA, GQA, and MLA" -- "MQA: one KV head for everyone"
  (each query head softmaxes its own scores against one shared K and V, scaled
  by the inverse square root of the head dimension) and "GQA: interpolating
  with groups" (query head i, 1-indexed, reads KV head ceil(i*n_kv/h); the
  module broadcasts each KV head to a consecutive block of query heads).
* "Grouped-Query Attention: Fewer KV Heads, Same Quality" -- "Writing the
  formula explicitly" (query heads are split into consecutive groups, each
  group sharing one K/V head) and "The Unified View".
* "Attention variants: MQA, GQA, and MLA" -- "MLA: cache a latent, not the keys
  and values" (after absorbing the key up-projection into the query, every
  head scores directly against the cached latent; the output is the weighted
  average of latents; a small decoupled rotary key is cached beside the
  latent and enters only the score).

Readings of points the pages leave open:

* Decode attends over every cached position t < n with no mask: the newest
  token is already in the cache (append-then-attend, as in the MLA decode
  step on the first page).
* ``n = seq_lens[b]`` is clamped to ``[0, T_max]``; ``n == 0`` gives an
  all-zero output row.
* Positions ``t >= n`` are never read: they may hold anything, NaN included.
* MLA: the value vector is the first ``d_c`` entries of the cached row (keys
  and values are the same latent); the rotary part contributes to the score
  only; no up-projection is applied to the output.

Inputs may be numpy arrays or CPU torch tensors of any float dtype; each
slice is widened to float64 before any arithmetic (exact for bf16/fp32).
"""

from __future__ import annotations

import numpy as np

try:  # torch is only needed to widen bf16 tensors, numpy has no bf16
    import torch
except Exception:  # pragma: no cover - torch is present in this image
    torch = None


def _f64(x) -> np.ndarray:
    """Widen a slice to float64 exactly (bf16 and fp32 values are exact in fp64)."""
    if torch is not None and isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _lens(seq_lens, B: int) -> np.ndarray:
    if torch is not None and isinstance(seq_lens, torch.Tensor):
        seq_lens = seq_lens.detach().cpu().numpy()
    return np.asarray(seq_lens, dtype=np.int64).reshape(B)


def clamp_len(n: int, T_max: int) -> int:
    """Number of cached positions a row attends over: seq_len clamped to [0, T_max]."""
    return int(min(max(int(n), 0), int(T_max)))


def _softmax_1d(s: np.ndarray) -> np.ndarray:
    """softmax over the last axis, shifted by the row maximum before exp."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def decode_gqa(q, k_cache, v_cache, seq_lens, scale: float) -> np.ndarray:
    """Decode attention for the MHA / GQA / MQA family.

    q        [B, h_q, D]          one new query token per head
    k_cache  [B, h_kv, T_max, D]  cached keys
    v_cache  [B, h_kv, T_max, Dv] cached values
    seq_lens [B]                  valid cached positions per sequence
    scale    score multiplier (1/sqrt(D) on the pages)

    For each sequence b and query head i: group size g = h_q / h_kv, KV head
    j = i // g (0-indexed form of the pages' ceil(i*h_kv/h_q)), scores
    s_t = scale * <q[b,i], K[b,j,t]> for t < n, weights softmax(s), and
    out[b,i] = sum_t w_t V[b,j,t]. Returns float64 [B, h_q, Dv].
    """
    B, h_q, D = q.shape
    Bk, h_kv, T_max, Dk = k_cache.shape
    Dv = v_cache.shape[-1]
    if Bk != B or Dk != D or tuple(v_cache.shape[:3]) != (B, h_kv, T_max):
        raise ValueError("shape mismatch between q, k_cache and v_cache")
    if h_kv < 1 or h_q % h_kv != 0:
        raise ValueError("h_q must be a multiple of h_kv")
    g = h_q // h_kv
    lens = _lens(seq_lens, B)
    out = np.zeros((B, h_q, Dv), dtype=np.float64)
    for b in range(B):
        n = clamp_len(lens[b], T_max)
        if n == 0:
            continue
        for j in range(h_kv):
            K = _f64(k_cache[b, j, :n])            # [n, D]
            V = _f64(v_cache[b, j, :n])            # [n, Dv]
            Q = _f64(q[b, j * g:(j + 1) * g])      # [g, D], the heads of group j
            S = scale * (Q @ K.T)                  # [g, n]
            W = _softmax_1d(S)
            out[b, j * g:(j + 1) * g] = W @ V
    return out


def decode_gqa_weights(q, k_cache, seq_lens, scale: float) -> list:
    """The softmax weights of ``decode_gqa``: a list over b of float64 [h_q, n_b]."""
    B, h_q, D = q.shape
    _, h_kv, T_max, _ = k_cache.shape
    g = h_q // h_kv
    lens = _lens(seq_lens, B)
    res = []
    for b in range(B):
        n = clamp_len(lens[b], T_max)
        W = np.zeros((h_q, n), dtype=np.float64)
        if n:
            for j in range(h_kv):
                K = _f64(k_cache[b, j, :n])
                Q = _f64(q[b, j * g:(j + 1) * g])
                W[j * g:(j + 1) * g] = _softmax_1d(scale * (Q @ K.T))
        res.append(W)
    return res


def decode_gqa_lse(q, k_cache, seq_lens, scale: float) -> np.ndarray:
    """Natural log of sum_t exp(s_t) per row, s_t the scaled scores of ``decode_gqa``.

    float64 [B, h_q]; rows with n == 0 hold -inf (an empty sum). This is the
    normaliser of the softmax, the quantity by which split partial results
    are weighted when they are combined.
    """
    B, h_q, D = q.shape
    _, h_kv, T_max, _ = k_cache.shape
    g = h_q // h_kv
    lens = _lens(seq_lens, B)
    res = np.full((B, h_q), -np.inf)
    for b in range(B):
        n = clamp_len(lens[b], T_max)
        if n == 0:
            continue
        for j in range(h_kv):
            S = scale * (_f64(q[b, j * g:(j + 1) * g]) @ _f64(k_cache[b, j, :n]).T)
            m = S.max(axis=1)
            res[b, j * g:(j + 1) * g] = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
    return res


def decode_mla(q_nope, q_rope, latent, seq_lens, scale: float, d_c: int) -> np.ndarray:
    """Absorbed multi-head latent attention, one decode step.

    q_nope  [B, H, d_c]          query already multiplied by the key up-projection
    q_rope  [B, H, d_r]          query part for the decoupled rotary key
    latent  [B, T_max, d_c+d_r]  cached row per token: [latent c | rotary key]
    seq_lens [B]

    For each b and head h, over t < n:
      s_t = scale * (<q_nope[b,h], c_t> + <q_rope[b,h], k_rope_t>)
      out[b,h] = sum_t softmax(s)_t * c_t        (value = the latent itself)
    Returns float64 [B, H, d_c]. Written independently of ``decode_gqa`` so
    that the two can check each other (MLA is structurally MQA with one
    shared head whose key is the whole row and whose value is its latent).
    """
    B, H, dc = q_nope.shape
    Bl, T_max, W = latent.shape
    if dc != d_c or Bl != B or q_rope.shape[:2] != (B, H) or W != d_c + q_rope.shape[2]:
        raise ValueError("shape mismatch between q_nope, q_rope and latent")
    lens = _lens(seq_lens, B)
    out = np.zeros((B, H, d_c), dtype=np.float64)
    for b in range(B):
        n = clamp_len(lens[b], T_max)
        if n == 0:
            continue
        row = _f64(latent[b, :n])                 # [n, d_c + d_r]
        c, kr = row[:, :d_c], row[:, d_c:]
        qn, qr = _f64(q_nope[b]), _f64(q_rope[b])  # [H, d_c], [H, d_r]
        S = scale * (qn @ c.T + qr @ kr.T)         # [H, n]
        out[b] = _softmax_1d(S) @ c
    return out
