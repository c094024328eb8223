"""Pins for the oracle's decode step (append the new token, then attend).

Each test checks ``oracle.step`` against something other than itself:

* the token-by-token walk of "Attention Variants: MHA, MQA, GQA — Speed vs
  Quality at Scale" ("The KV Cache Problem"), driven from an empty cache,
  against PyTorch's causal scaled-dot-product attention (float64, native GQA
  head sharing): step t must reproduce row t of causal attention over the
  whole sequence, and the cache must end up holding every token's K and V;
* the cache writes against plain tensor indexing (a library copy), byte for
  byte, with every other byte unchanged;
* the MLA step against the first page's decode sketch written with torch
  (concatenate the new latent, then score and average over the extended
  cache), plus the rotary key, as causal SDPA with one shared 576-wide key;
* closed forms: an empty cache returns the new value exactly; a full cache is
  left unchanged.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _rand(shape, seed, dtype=torch.float64):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64).to(dtype)


@pytest.mark.parametrize("h_q,h_kv", [(8, 2), (4, 4), (6, 1)])
def test_token_by_token_walk_matches_causal_attention(h_q, h_kv):
    B, T, d = 2, 9, 8
    q = _rand((B, h_q, T, d), 1)
    k = _rand((B, h_kv, T, d), 2)
    v = _rand((B, h_kv, T, d), 3)
    ref = F.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=True)
    T_max = 12
    kc = torch.full((B, h_kv, T_max, d), float("nan"), dtype=torch.float64)
    vc = torch.full((B, h_kv, T_max, d), float("nan"), dtype=torch.float64)
    for t in range(T):
        lens = torch.full((B,), t, dtype=torch.int32)
        out, kc, vc = oracle.decode_gqa_step(q[:, :, t], k[:, :, t], v[:, :, t], kc, vc, lens,
                                             1.0 / math.sqrt(d))
        assert np.abs(out - ref[:, :, t].numpy()).max() <= 1e-12
    assert torch.equal(kc[:, :, :T], k) and torch.equal(vc[:, :, :T], v)
    assert torch.isnan(kc[:, :, T:]).all() and torch.isnan(vc[:, :, T:]).all()


def test_cache_write_is_a_byte_exact_copy():
    B, h_kv, T_max, D = 3, 2, 10, 16
    kc = _rand((B, h_kv, T_max, D), 4, torch.bfloat16)
    vc = _rand((B, h_kv, T_max, D), 5, torch.bfloat16)
    kn = _rand((B, h_kv, D), 6, torch.bfloat16)
    vn = _rand((B, h_kv, D), 7, torch.bfloat16)
    lens = torch.tensor([0, 7, 10], dtype=torch.int32)       # empty, middle, full
    k2, v2 = oracle.append_kv(kc, vc, kn, vn, lens)
    ek, ev = kc.clone(), vc.clone()
    for b, p in enumerate([0, 7]):
        ek[b, :, p] = kn[b]
        ev[b, :, p] = vn[b]
    assert torch.equal(k2.view(torch.int16), ek.view(torch.int16))
    assert torch.equal(v2.view(torch.int16), ev.view(torch.int16))
    assert torch.equal(kc, _rand((B, h_kv, T_max, D), 4, torch.bfloat16))   # inputs untouched


def test_empty_cache_returns_the_new_value_and_full_cache_is_unchanged():
    B, h_q, h_kv, T_max, D = 2, 4, 2, 6, 8
    q = _rand((B, h_q, D), 8)
    kc = _rand((B, h_kv, T_max, D), 9)
    vc = _rand((B, h_kv, T_max, D), 10)
    kn = _rand((B, h_kv, D), 11)
    vn = _rand((B, h_kv, D), 12)
    lens = torch.tensor([-3, T_max + 4], dtype=torch.int32)   # negative reads as 0; past the end is full
    out, k2, v2 = oracle.decode_gqa_step(q, kn, vn, kc, vc, lens, 0.3)
    g = h_q // h_kv
    for i in range(h_q):   # one position: the weight is exactly 1
        assert np.array_equal(out[0, i], vn[0, i // g].numpy())
    assert torch.equal(k2[1], kc[1]) and torch.equal(v2[1], vc[1])
    assert np.abs(out[1] - oracle.decode_gqa(q[1:], kc[1:], vc[1:], [T_max], 0.3)[0]).max() == 0


def test_mla_step_matches_the_pages_decode_sketch():
    B, H, T_past, d_c, d_r = 2, 4, 5, 16, 8
    T_max = 8
    qn = _rand((B, H, d_c), 13)
    qr = _rand((B, H, d_r), 14)
    lat = _rand((B, T_max, d_c + d_r), 15)
    new = _rand((B, d_c + d_r), 16)
    scale = 0.21
    lens = torch.tensor([T_past, 2], dtype=torch.int32)
    out, lat2 = oracle.decode_mla_step(qn, qr, new, lat, lens, scale, d_c)
    for b in range(B):
        n = int(lens[b])
        cache = torch.cat([lat[b, :n], new[b:b + 1]], dim=0)           # (n + 1, d_c + d_r)
        s = (qn[b] @ cache[:, :d_c].T + qr[b] @ cache[:, d_c:].T) * scale
        o = torch.softmax(s, dim=-1) @ cache[:, :d_c]
        assert np.abs(out[b] - o.numpy()).max() <= 1e-12
        # the same as SDPA with one shared 576-wide key and the latent as value
        kq = torch.cat([qn[b], qr[b]], dim=-1)[None, :, None]          # (1, H, 1, d_c + d_r)
        ref = F.scaled_dot_product_attention(kq, cache[None, None], cache[None, None, :, :d_c],
                                             enable_gqa=True, scale=scale)[0, :, 0]
        assert np.abs(out[b] - ref.numpy()).max() <= 1e-12
        assert torch.equal(lat2[b, n], new[b])
        assert torch.equal(torch.cat([lat2[b, :n], lat2[b, n + 1:]]), torch.cat([lat[b, :n], lat[b, n + 1:]]))
