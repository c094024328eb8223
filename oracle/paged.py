"""fp64 definition of decode attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY -- see the package docstring. The product path never
imports this module.

Source (page title -- section): "Attention variants: MQA, GQA, and MLA" --
"Against the real libraries": serving engines keep the KV cache in fixed-size
pages that are allocated like virtual memory and may be shared between
sequences with a common prefix.

Layout (a reading: the pages name no layout):

* GQA: ``k_pages``, ``v_pages`` [num_pages, h_kv, page_size, D]; logical
  position t of sequence b lives in physical page ``block_table[b, t //
  page_size]`` at row ``t % page_size`` of each KV head.
* MLA: ``latent_pages`` [num_pages, page_size, d_c + d_r], same mapping.
* ``block_table`` [B, max_pages] int32; a sequence holds at most
  ``T_max = max_pages * page_size`` positions and ``seq_lens`` is clamped to
  ``[0, T_max]``. Entries past a sequence's last page are never read, and
  neither are rows past its length inside its last page.

Attention itself is exactly ``attention.decode_gqa`` / ``decode_mla`` on the
positions gathered in logical order.
"""

from __future__ import annotations

import numpy as np

from .attention import _f64, _lens, clamp_len, decode_gqa, decode_mla

try:
    import torch
except Exception:  # pragma: no cover - torch is present in this image
    torch = None


def _table(block_table) -> np.ndarray:
    if torch is not None and isinstance(block_table, torch.Tensor):
        block_table = block_table.detach().cpu().numpy()
    return np.asarray(block_table, dtype=np.int64)


def _rows(block_table, b: int, n: int, page_size: int):
    """(physical page, row inside it) of logical positions 0..n-1 of sequence b."""
    t = np.arange(n)
    return _table(block_table)[b, t // page_size], t % page_size


def _index(pages, page, row):
    """pages[page[i], ..., row[i], ...] for GQA ([P, H, ps, D]) or MLA ([P, ps, W]) pages,
    gathered in the pages' own dtype and then widened."""
    if torch is not None and isinstance(pages, torch.Tensor):
        pi, ri = torch.as_tensor(page), torch.as_tensor(row)
        return _f64(pages[pi, :, ri] if pages.dim() == 4 else pages[pi, ri])
    x = np.asarray(pages)
    return _f64(x[page, :, row] if x.ndim == 4 else x[page, row])


def gather_kv(pages, block_table, b: int, n: int, page_size: int) -> np.ndarray:
    """Positions 0..n-1 of sequence b, in logical order: float64 [h_kv, n, D] (GQA pages)."""
    page, row = _rows(block_table, b, n, page_size)
    return _index(pages, page, row).transpose(1, 0, 2)   # [n, h_kv, D] -> [h_kv, n, D]


def gather_latent(pages, block_table, b: int, n: int, page_size: int) -> np.ndarray:
    """Positions 0..n-1 of sequence b, in logical order: float64 [n, d_c + d_r] (MLA pages)."""
    page, row = _rows(block_table, b, n, page_size)
    return _index(pages, page, row)


def decode_gqa_paged(q, k_pages, v_pages, block_table, seq_lens, scale: float, page_size: int):
    """decode_gqa over the positions the block table maps, one sequence at a time."""
    B = q.shape[0]
    T_max = _table(block_table).shape[1] * page_size
    lens = _lens(seq_lens, B)
    out = np.zeros((B, q.shape[1], v_pages.shape[3]), dtype=np.float64)
    for b in range(B):
        n = clamp_len(lens[b], T_max)
        if n == 0:
            continue
        K = gather_kv(k_pages, block_table, b, n, page_size)[None]   # [1, h_kv, n, D]
        V = gather_kv(v_pages, block_table, b, n, page_size)[None]
        out[b] = decode_gqa(_f64(q[b:b + 1]), K, V, [n], scale)[0]
    return out


def decode_mla_paged(q_nope, q_rope, latent_pages, block_table, seq_lens, scale: float, d_c: int,
                     page_size: int):
    """decode_mla over the positions the block table maps."""
    B = q_nope.shape[0]
    T_max = _table(block_table).shape[1] * page_size
    lens = _lens(seq_lens, B)
    out = np.zeros((B, q_nope.shape[1], d_c), dtype=np.float64)
    for b in range(B):
        n = clamp_len(lens[b], T_max)
        if n == 0:
            continue
        lat = gather_latent(latent_pages, block_table, b, n, page_size)[None]   # [1, n, d_c + d_r]
        out[b] = decode_mla(_f64(q_nope[b:b + 1]), _f64(q_rope[b:b + 1]), lat, [n], scale, d_c)[0]
    return out


def append_kv_paged(k_pages, v_pages, block_table, k_new, v_new, seq_lens, page_size: int):
    """Pages after writing k_new[b] / v_new[b] ([h_kv, D]) at logical position seq_lens[b]
    (clamped below at 0; a sequence whose pages are full, or whose table entry for that
    position names no page, is not written)."""
    table = _table(block_table)
    T_max = table.shape[1] * page_size
    B = table.shape[0]
    lens = _lens(seq_lens, B)
    k_out = k_pages.clone() if torch is not None and isinstance(k_pages, torch.Tensor) else np.array(k_pages)
    v_out = v_pages.clone() if torch is not None and isinstance(v_pages, torch.Tensor) else np.array(v_pages)
    num_pages = k_pages.shape[0]
    for b in range(B):
        pos = max(int(lens[b]), 0)
        if pos >= T_max:
            continue
        page = int(table[b, pos // page_size])
        if not 0 <= page < num_pages:      # an entry that names no page: nothing is written
            continue
        k_out[page, :, pos % page_size] = k_new[b]
        v_out[page, :, pos % page_size] = v_new[b]
    return k_out, v_out
