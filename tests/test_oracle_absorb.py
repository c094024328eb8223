"""Pins for the oracle's MLA absorption products.

* the page's own einsum subscripts ('bhd,hcd->bhc' for the query, 'bhc,hcd->bhd'
  for the output), evaluated by torch.einsum in float64 (a library routine);
* the whole absorbed layer against the un-absorbed one: per-head keys and
  values materialised from the latent (c @ W_UK[h], c @ W_UV[h]) and plain
  softmax attention, in float64 -- absorb, decode over the latent, up-project
  must give the same outputs;
* transposition check: with W_UK = identity (d_c = d_h) the absorbed query is
  the query itself.
"""

import math

import numpy as np
import torch

import oracle


def _rand(shape, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64)


def test_absorb_and_up_match_the_pages_einsums():
    B, H, d_h, d_c, d_v = 3, 5, 8, 12, 7
    q = _rand((B, H, d_h), 1)
    w_uk = _rand((H, d_c, d_h), 2)
    o_lat = _rand((B, H, d_c), 3)
    w_uv = _rand((H, d_c, d_v), 4)
    assert np.abs(oracle.absorb_q(q, w_uk) - torch.einsum("bhd,hcd->bhc", q, w_uk).numpy()).max() <= 1e-12
    assert np.abs(oracle.up_v(o_lat, w_uv) - torch.einsum("bhc,hcd->bhd", o_lat, w_uv).numpy()).max() <= 1e-12


def test_absorbed_layer_equals_unabsorbed_attention():
    B, H, T, d_c, d_r, d_h, d_v = 2, 4, 10, 16, 4, 6, 5
    c = _rand((B, T, d_c), 10)
    kr = _rand((B, T, d_r), 11)
    w_uk = _rand((H, d_c, d_h), 12)
    w_uv = _rand((H, d_c, d_v), 13)
    q = _rand((B, H, d_h), 14)
    qr = _rand((B, H, d_r), 15)
    lens = [10, 3]
    scale = 1.0 / math.sqrt(d_h + d_r)
    ref = np.zeros((B, H, d_v))
    for b in range(B):
        n = lens[b]
        for h in range(H):
            k = c[b, :n] @ w_uk[h]                     # [n, d_h] materialised keys
            v = c[b, :n] @ w_uv[h]                     # [n, d_v] materialised values
            s = scale * (k @ q[b, h] + kr[b, :n] @ qr[b, h])
            ref[b, h] = (torch.softmax(s, dim=0) @ v).numpy()
    q_lat = oracle.absorb_q(q, w_uk)
    o_lat = oracle.decode_mla(q_lat, qr, torch.cat([c, kr], dim=-1), lens, scale, d_c)
    got = oracle.up_v(o_lat, w_uv)
    assert np.abs(got - ref).max() <= 1e-10


def test_identity_projection():
    q = _rand((2, 3, 8), 16)
    eye = torch.eye(8, dtype=torch.float64).expand(3, 8, 8)
    assert np.array_equal(oracle.absorb_q(q, eye), q.numpy())
    assert np.array_equal(oracle.up_v(q, eye), q.numpy())
