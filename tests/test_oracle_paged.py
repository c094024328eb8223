"""Pins for the oracle's paged-cache decode.

* A linear cache cut into pages with torch's own reshape and scattered over a
  random permutation of physical slots (the block table is the inverse
  permutation) must reproduce PyTorch's float64 scaled-dot-product attention
  on the linear cache (a library routine; the page mapping is built without
  the oracle's index arithmetic);
* prefix sharing (two sequences whose tables point at the same first pages)
  equals the linear caches with the prefix duplicated;
* pages nobody references, table entries past a sequence's last page and
  rows past its length hold NaN or garbage indices and are never read;
* the paged append writes one row, byte for byte, where plain indexing puts it;
* MLA: the same permutation check against the page's absorbed-MLA formula
  written in torch.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _rand(shape, seed, dtype=torch.float64):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64).to(dtype)


def _paginate(cache, page_size, perm):
    """[B, h_kv, T, D] linear cache -> pages [B*T/ps, h_kv, ps, D] placed at slots perm[logical]."""
    B, H, T, D = cache.shape
    npg = T // page_size
    logical = cache.reshape(B, H, npg, page_size, D).permute(0, 2, 1, 3, 4).reshape(B * npg, H, page_size, D)
    pages = torch.empty_like(logical)
    pages[perm] = logical
    table = perm.reshape(B, npg).to(torch.int32)
    return pages, table


@pytest.mark.parametrize("page_size", [1, 4, 16])
def test_paged_matches_sdpa_on_the_linear_cache(page_size):
    B, h_q, h_kv, T, d = 3, 8, 2, 32, 8
    q = _rand((B, h_q, d), 1)
    k = _rand((B, h_kv, T, d), 2)
    v = _rand((B, h_kv, T, d), 3)
    perm = torch.randperm(B * T // page_size, generator=torch.Generator().manual_seed(4))
    kp, table = _paginate(k, page_size, perm)
    vp, _ = _paginate(v, page_size, perm)
    lens = [32, 17, 1]
    got = oracle.decode_gqa_paged(q, kp, vp, table, lens, 0.3, page_size)
    for b, n in enumerate(lens):
        ref = F.scaled_dot_product_attention(q[b:b + 1, :, None], k[b:b + 1, :, :n], v[b:b + 1, :, :n],
                                             enable_gqa=True, scale=0.3)[0, :, 0]
        assert np.abs(got[b] - ref.numpy()).max() <= 1e-12


def test_prefix_sharing_and_unread_pages():
    page_size, h_q, h_kv, d = 4, 4, 1, 8
    shared = _rand((2, h_kv, page_size, d), 5)            # two physical pages of common prefix
    own = _rand((4, h_kv, page_size, d), 6)               # two private pages per sequence
    junk = torch.full((3, h_kv, page_size, d), float("nan"), dtype=torch.float64)
    kp = torch.cat([shared, own, junk])                   # pages 0-1 shared, 2-5 private, 6-8 never read
    vp = torch.cat([shared * 0.5, own * -1.0, junk])
    table = torch.tensor([[0, 1, 2, 3, 999], [0, 1, 4, 5, -7]], dtype=torch.int32)   # entries past the end: garbage
    lens = [14, 16]
    q = _rand((2, h_q, d), 7)
    got = oracle.decode_gqa_paged(q, kp, vp, table, lens, 0.5, page_size)
    assert np.isfinite(got).all()
    for b, pages in enumerate([[0, 1, 2, 3], [0, 1, 4, 5]]):
        kl = torch.cat([kp[p] for p in pages], dim=1)[None]   # [1, h_kv, 16, d]
        vl = torch.cat([vp[p] for p in pages], dim=1)[None]
        ref = oracle.decode_gqa(q[b:b + 1], kl, vl, [lens[b]], 0.5)[0]
        assert np.array_equal(got[b], ref)


def test_paged_append_writes_one_row():
    page_size, h_kv, d = 4, 2, 8
    kp = _rand((6, h_kv, page_size, d), 8, torch.bfloat16)
    vp = _rand((6, h_kv, page_size, d), 9, torch.bfloat16)
    table = torch.tensor([[3, 0, 5], [1, 2, 4]], dtype=torch.int32)
    kn = _rand((2, h_kv, d), 10, torch.bfloat16)
    vn = _rand((2, h_kv, d), 11, torch.bfloat16)
    lens = torch.tensor([5, 12], dtype=torch.int32)       # row 1 of page 0; sequence 1 is full
    k2, v2 = oracle.append_kv_paged(kp, vp, table, kn, vn, lens, page_size)
    ek, ev = kp.clone(), vp.clone()
    ek[0, :, 1] = kn[0]
    ev[0, :, 1] = vn[0]
    assert torch.equal(k2.view(torch.int16), ek.view(torch.int16))
    assert torch.equal(v2.view(torch.int16), ev.view(torch.int16))


def test_mla_paged_matches_the_formula_on_the_linear_cache():
    B, H, T, d_c, d_r, page_size = 2, 4, 24, 16, 8, 8
    qn = _rand((B, H, d_c), 12)
    qr = _rand((B, H, d_r), 13)
    lat = _rand((B, T, d_c + d_r), 14)
    npg = T // page_size
    perm = torch.randperm(B * npg, generator=torch.Generator().manual_seed(15))
    logical = lat.reshape(B * npg, page_size, d_c + d_r)
    pages = torch.empty_like(logical)
    pages[perm] = logical
    table = perm.reshape(B, npg).to(torch.int32)
    lens = [24, 9]
    got = oracle.decode_mla_paged(qn, qr, pages, table, lens, 0.2, d_c, page_size)
    for b, n in enumerate(lens):
        c = lat[b, :n]
        s = (qn[b] @ c[:, :d_c].T + qr[b] @ c[:, d_c:].T) * 0.2
        ref = torch.softmax(s, dim=-1) @ c[:, :d_c]
        assert np.abs(got[b] - ref.numpy()).max() <= 1e-12
