"""Pins for the oracle's sliding-window decode.

* PyTorch's CPU scaled-dot-product attention in float64 with native GQA head
  sharing and an explicit boolean mask that admits exactly the positions
  [n - window, n) (a library routine, the mask built independently of the
  oracle's slicing);
* brute force with pure-Python loops on tiny shapes;
* special cases: window >= n is the full decode; window = 1 returns the
  newest value exactly; a window over a padded cache never reads the padding;
* the bound the page states for Mistral 7B: with the window, the cache a
  decode step reads stops growing at w positions (bytes computed by the
  cache-size helper at seq_len = w, whatever the sequence length).
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _rand(shape, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64)


@pytest.mark.parametrize("h_q,h_kv,window", [(8, 2, 5), (4, 4, 1), (6, 1, 17), (8, 8, 40)])
def test_window_matches_sdpa_with_explicit_mask(h_q, h_kv, window):
    B, T, d = 3, 33, 8
    q = _rand((B, h_q, d), 1)
    k = _rand((B, h_kv, T, d), 2)
    v = _rand((B, h_kv, T, d), 3)
    lens = [33, 12, 3]
    got = oracle.decode_gqa_window(q, k, v, lens, 0.4, window)
    for b, n in enumerate(lens):
        mask = torch.zeros((1, 1, 1, T), dtype=torch.bool)
        for t in range(T):
            mask[..., t] = (t < n) and (t >= n - window)
        ref = F.scaled_dot_product_attention(q[b:b + 1, :, None], k[b:b + 1], v[b:b + 1],
                                             attn_mask=mask, enable_gqa=True, scale=0.4)[0, :, 0]
        assert np.abs(got[b] - ref.numpy()).max() <= 1e-12


def test_window_matches_brute_force():
    B, h_q, h_kv, T, d, window = 2, 4, 2, 9, 3, 4
    q = _rand((B, h_q, d), 4)
    k = _rand((B, h_kv, T, d), 5)
    v = _rand((B, h_kv, T, d), 6)
    lens = [9, 6]
    got = oracle.decode_gqa_window(q, k, v, lens, 0.7, window)
    g = h_q // h_kv
    for b, n in enumerate(lens):
        for i in range(h_q):
            j = i // g
            ts = [t for t in range(T) if n - window <= t < n]
            s = [0.7 * math.fsum(float(q[b, i, c]) * float(k[b, j, t, c]) for c in range(d)) for t in ts]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = math.fsum(e)
            for c in range(d):
                o = math.fsum(e[u] / z * float(v[b, j, t, c]) for u, t in enumerate(ts))
                assert abs(got[b, i, c] - o) <= 1e-12


def test_window_special_cases():
    B, h_q, h_kv, T, d = 2, 4, 2, 16, 8
    q = _rand((B, h_q, d), 7)
    k = _rand((B, h_kv, T, d), 8)
    v = _rand((B, h_kv, T, d), 9)
    lens = [16, 7]
    full = oracle.decode_gqa(q, k, v, lens, 0.5)
    assert np.array_equal(oracle.decode_gqa_window(q, k, v, lens, 0.5, 16), full)
    assert np.array_equal(oracle.decode_gqa_window(q, k, v, lens, 0.5, 1000), full)
    one = oracle.decode_gqa_window(q, k, v, lens, 0.5, 1)
    for b, n in enumerate(lens):
        for i in range(h_q):
            assert np.array_equal(one[b, i], v[b, i // 2, n - 1].numpy())
    kp, vp = k.clone(), v.clone()
    kp[1, :, 7:] = float("nan")
    vp[1, :, 7:] = float("nan")
    kp[0, :, :10] = float("nan")                 # before the window of row 0 (n=16, window=6)
    vp[0, :, :10] = float("nan")
    a = oracle.decode_gqa_window(q, kp, vp, lens, 0.5, 6)
    b = oracle.decode_gqa_window(q, k, v, lens, 0.5, 6)
    assert np.isfinite(a).all() and np.array_equal(a, b)
    assert oracle.window_start(100, 4096) == 0 and oracle.window_start(5000, 4096) == 904


def test_window_bounds_the_cache_read_per_step():
    """Mistral 7B: 32 query heads over 8 KV groups, d_k = d_v = 128, 32 layers, w = 4096, fp16:
    the cache a step reads is the helper's bytes at seq_len = w for any longer sequence."""
    per_pos = oracle.kv_cache_bytes(32, 8, 128, 1, 1, 2)
    bound = oracle.kv_cache_bytes(32, 8, 128, 4096, 1, 2)
    for n in [100, 4096, 10_000, 128_000]:
        assert min(n, 4096) * per_pos <= bound
    assert bound == 8 * (128 + 128) * 2 * 32 * 4096
