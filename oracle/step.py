"""fp64 definition of one decode step: append the new token, then attend.

TEST INFRASTRUCTURE ONLY -- see the package docstring. The product path never
imports this module.

Sources (page title -- section):

* "Attention Variants: MHA, MQA, GQA — Speed vs Quality at Scale" -- "The KV
  Cache Problem": each generated token's K and V are computed once and stored
  in the cache; the token then attends to every cached pair, its own included.
* "Attention variants: MQA, GQA, and MLA" -- "MLA: cache a latent, not the keys
  and values" (decode sketch): the new token's latent is concatenated to the
  latent cache, and the scores and the average run over the extended cache.

Readings of points the pages leave open:

* ``seq_lens[b]`` holds the number of cached positions *before* the step;
  the new row goes to position ``pos = max(seq_lens[b], 0)`` and the step
  attends over ``pos + 1`` positions. Advancing ``seq_lens`` is the caller's
  business (the arrays passed in are not modified).
* A sequence whose cache is full (``pos >= T_max``) is not appended to; it
  attends over its ``T_max`` cached positions.
* Only row ``pos`` of each written head changes; every other byte of the
  caches is left as it was.
"""

from __future__ import annotations

import numpy as np

from .attention import decode_gqa, decode_mla, _lens

try:
    import torch
except Exception:  # pragma: no cover - torch is present in this image
    torch = None


def _copy(x):
    if torch is not None and isinstance(x, torch.Tensor):
        return x.detach().clone()
    return np.array(x, copy=True)


def _step_lengths(seq_lens, B: int, T_max: int):
    """(write position or -1 when the cache is full, attended length) per sequence."""
    pos = np.maximum(_lens(seq_lens, B), 0)
    write = np.where(pos < T_max, pos, -1)
    n = np.minimum(pos + 1, T_max)
    return write, n


def append_kv(k_cache, v_cache, k_new, v_new, seq_lens):
    """Caches after writing k_new[b, j] / v_new[b, j] into row seq_lens[b] of head j.

    k_cache, v_cache: [B, h_kv, T_max, D]; k_new, v_new: [B, h_kv, D]. Returns
    new arrays (same type and dtype as the caches); the stored values are the
    new rows' values unchanged (a copy, no arithmetic).
    """
    B, _, T_max, _ = k_cache.shape
    write, _ = _step_lengths(seq_lens, B, T_max)
    k_out, v_out = _copy(k_cache), _copy(v_cache)
    for b in range(B):
        if write[b] >= 0:
            k_out[b, :, int(write[b]), :] = k_new[b]
            v_out[b, :, int(write[b]), :] = v_new[b]
    return k_out, v_out


def decode_gqa_step(q, k_new, v_new, k_cache, v_cache, seq_lens, scale: float):
    """One decode step of the GQA family: append, then attend over pos + 1 rows.

    Returns (out float64 [B, h_q, D], k_cache after, v_cache after).
    """
    B, _, T_max, _ = k_cache.shape
    k_out, v_out = append_kv(k_cache, v_cache, k_new, v_new, seq_lens)
    _, n = _step_lengths(seq_lens, B, T_max)
    return decode_gqa(q, k_out, v_out, n, scale), k_out, v_out


def append_latent(latent, latent_new, seq_lens):
    """Latent cache [B, T_max, d_c + d_r] after writing latent_new[b] into row seq_lens[b]."""
    B, T_max, _ = latent.shape
    write, _ = _step_lengths(seq_lens, B, T_max)
    out = _copy(latent)
    for b in range(B):
        if write[b] >= 0:
            out[b, int(write[b]), :] = latent_new[b]
    return out


def decode_mla_step(q_nope, q_rope, latent_new, latent, seq_lens, scale: float, d_c: int):
    """One absorbed-MLA decode step: append the new latent row, then attend.

    Returns (out float64 [B, H, d_c], latent cache after).
    """
    B, T_max, _ = latent.shape
    lat_out = append_latent(latent, latent_new, seq_lens)
    _, n = _step_lengths(seq_lens, B, T_max)
    return decode_mla(q_nope, q_rope, lat_out, n, scale, d_c), lat_out
