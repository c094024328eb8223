"""Pins for the fp64 oracle: each test checks it against something other than itself.

What pins what:
* the pages' printed cache sizes (golden/cache_bytes.json) -> cache arithmetic;
* PyTorch's CPU scaled-dot-product attention, float64, with native GQA head
  sharing and with the causal mask -> group map, scale, softmax, lengths;
* pure-Python brute force (a different statement of the definition) -> all
  of decode_gqa and decode_mla on tiny shapes;
* closed forms: one position returns its value, equal keys average the
  values, the pages' 0.8/0.2 worked example, a dominant score;
* invariants: weights sum to 1, permutations, NaN in padding is never read;
* the MLA absorption identity with explicit up-projections, and MLA written
  as MQA with one wide head.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed, dtype=torch.float64):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64).to(dtype)


# --------------------------------------------------------------------------- cache arithmetic

def test_cache_bytes_match_pages():
    data = _load("cache_bytes.json")
    for case in data["kv"]:
        got = oracle.kv_cache_bytes(*case["args"])
        assert got == case["bytes"], case["cite"]
        if "printed_gib_3dp" in case:
            assert f"{got / 2**30:.3f}" == case["printed_gib_3dp"], case["cite"]


def test_mla_cache_elements_match_pages():
    data = _load("cache_bytes.json")
    for case in data["mla"]:
        assert oracle.mla_cache_bytes(*case["args"]) == case["elements"], case["cite"]
        if "mha_elements" in case:
            mha = oracle.kv_cache_bytes(1, 128, 128, 1, 1, 1)
            assert mha == case["mha_elements"]
            assert mha // case["elements"] == case["ratio"]
        if "gqa_equiv_kv_heads" in case:
            assert 2 * case["gqa_equiv_kv_heads"] * case["head_dim"] == case["elements"]


def test_mla_cache_bytes_match_pages():
    """The MLA row per token scaled by bytes per value, layers, tokens and
    sequences: each factor differs from 1 in some case, so dropping any fails."""
    data = _load("cache_bytes.json")
    for i in (0, 3, 4, 5):                                  # layers, tokens, sequences, bytes
        assert any(c["args"][i] != 1 for c in data["mla_bytes"])
    for case in data["mla_bytes"]:
        assert oracle.mla_cache_bytes(*case["args"]) == case["bytes"], case["cite"]
        if "mha_args" in case:
            mha = oracle.kv_cache_bytes(*case["mha_args"])
            assert mha == case["mha_bytes"]
            assert case["bytes"] < mha / 3                  # that notebook's own check


def test_cache_ratios_match_pages():
    data = _load("cache_bytes.json")
    nb = data["ratios"][0]
    for name, kvh in nb["kv_heads"].items():
        per_tok = oracle.kv_cache_bytes(1, kvh, nb["head_dim"], 1, 1, 2)
        assert per_tok == nb["per_token_bytes_fp16"][name]
    mha = oracle.kv_cache_bytes(1, nb["kv_heads"]["MHA"], nb["head_dim"], 1, 1, 2)
    for name, r in nb["expected_ratio"].items():
        assert mha / oracle.kv_cache_bytes(1, nb["kv_heads"][name], nb["head_dim"], 1, 1, 2) == r
    gen = data["ratios"][1]
    for gq, r in zip(gen["groups"], gen["expected_ratio"]):
        for (L, d, t) in [(12, 64, 4096), (80, 128, 1), (1, 32, 777)]:
            assert oracle.kv_cache_bytes(L, gen["h"], d, t) == r * oracle.kv_cache_bytes(L, gq, d, t)


# --------------------------------------------------------------------------- library routine (SDPA)

def _sdpa_decode_rows(q, k, v, scale=None):
    """q [B,Hq,T,d], k/v [B,Hkv,T,d] float64 -> causal SDPA with native GQA, [B,Hq,T,d]."""
    return F.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=True, scale=scale)


def test_gqa_matches_sdpa_causal_rows():
    """Causal prefill attention through PyTorch's CPU SDPA with native GQA head
    sharing, in float64 ("Attention variants: MQA, GQA, and MLA", section
    "Against the real libraries" checks its own implementation this way).

    Row t of causal attention over T positions is a decode step that attends
    over positions 0..t; every row pins the oracle with n = t + 1. Shapes and
    seed are this test's own: 3 KV heads shared by 12 query heads.
    """
    B, Hq, Hkv, T, d = 3, 12, 3, 50, 24
    q = _rand((B, Hq, T, d), 123)
    k = _rand((B, Hkv, T, d), 124)
    v = _rand((B, Hkv, T, d), 125)
    ref = _sdpa_decode_rows(q, k, v)
    for t in [0, 1, 2, 13, 31, T - 1]:
        got = oracle.decode_gqa(q[:, :, t], k, v, [t + 1] * B, 1.0 / math.sqrt(d))
        assert np.abs(got - ref[:, :, t].numpy()).max() <= 1e-12


@pytest.mark.parametrize("h_q,h_kv", [(8, 8), (8, 4), (8, 2), (8, 1), (6, 3), (12, 4)])
def test_gqa_matches_sdpa_group_map_and_scale(h_q, h_kv):
    B, T, d = 2, 37, 16
    q = _rand((B, h_q, 1, d), 1)
    k = _rand((B, h_kv, T, d), 2)
    v = _rand((B, h_kv, T, d + 3), 3)   # value width differs from key width on purpose
    scale = 0.37
    ref = F.scaled_dot_product_attention(q, k, v, enable_gqa=True, scale=scale)[:, :, 0]
    got = oracle.decode_gqa(q[:, :, 0], k, v, [T, T], scale)
    assert np.abs(got - ref.numpy()).max() <= 1e-12


def test_gqa_equals_mha_on_explicitly_repeated_kv():
    """Repeating each KV head over its consecutive group (torch.repeat_interleave) gives MHA."""
    B, h_q, h_kv, T, d = 3, 12, 3, 20, 8
    q = _rand((B, h_q, d), 4)
    k = _rand((B, h_kv, T, d), 5)
    v = _rand((B, h_kv, T, d), 6)
    lens = [20, 7, 1]
    kk = k.repeat_interleave(h_q // h_kv, dim=1)
    vv = v.repeat_interleave(h_q // h_kv, dim=1)
    got = oracle.decode_gqa(q, k, v, lens, 0.5)
    mha = oracle.decode_gqa(q, kk, vv, lens, 0.5)
    assert np.abs(got - mha).max() <= 1e-12
    for b, n in enumerate(lens):   # and MHA itself against the library routine, per length
        ref = F.scaled_dot_product_attention(q[b:b + 1, :, None], kk[b:b + 1, :, :n], vv[b:b + 1, :, :n],
                                             scale=0.5)[:, :, 0]
        assert np.abs(mha[b] - ref[0].numpy()).max() <= 1e-12


def test_mqa_every_head_reads_the_one_shared_head():
    B, h_q, T, d = 2, 5, 11, 6
    q = _rand((B, h_q, d), 7)
    k = _rand((B, 1, T, d), 8)
    v = _rand((B, 1, T, d), 9)
    got = oracle.decode_gqa(q, k, v, [T, 4], 0.3)
    for i in range(h_q):
        single = oracle.decode_gqa(q[:, i:i + 1], k, v, [T, 4], 0.3)
        assert np.abs(got[:, i:i + 1] - single).max() <= 1e-14


# --------------------------------------------------------------------------- brute force

@pytest.mark.parametrize("h_q,h_kv,D,T,lens", [
    (4, 4, 3, 5, [5, 2]), (4, 2, 4, 6, [6, 1]), (6, 2, 2, 7, [3, 7]), (6, 3, 5, 4, [4, 4]),
    (8, 1, 3, 9, [9, 5]), (8, 8, 2, 3, [0, 3]), (6, 6, 4, 8, [8, 8]), (8, 4, 8, 16, [16, 9]),
])
def test_gqa_matches_brute_force(h_q, h_kv, D, T, lens):
    B = len(lens)
    q = _rand((B, h_q, D), 10 + h_q)
    k = _rand((B, h_kv, T, D), 20 + T)
    v = _rand((B, h_kv, T, D), 30 + D)
    got = oracle.decode_gqa(q, k, v, lens, 0.7)
    ref = np.array(brute.brute_gqa(q, k, v, lens, 0.7))
    assert got.shape == ref.shape
    assert np.abs(got - ref).max() <= 1e-12


def test_brute_group_map_is_the_pages_ceiling_formula():
    # h=8 query heads, 2 groups: heads 1..4 -> group 1, 5..8 -> group 2 (the fifth page's example)
    assert [brute.kv_head_of(i, 8, 2) for i in range(1, 9)] == [1, 1, 1, 1, 2, 2, 2, 2]
    # 32 query heads, 8 KV heads: Q1..Q4 share K1/V1, Q29..Q32 share K8/V8 (the third page)
    assert [brute.kv_head_of(i, 32, 8) for i in (1, 4, 5, 8, 29, 32)] == [1, 1, 2, 2, 8, 8]


@pytest.mark.parametrize("H,T,d_c,d_r,lens", [(3, 5, 4, 2, [5, 3]), (2, 7, 6, 3, [1, 7]), (4, 4, 8, 4, [0, 4])])
def test_mla_matches_brute_force(H, T, d_c, d_r, lens):
    B = len(lens)
    qn = _rand((B, H, d_c), 40)
    qr = _rand((B, H, d_r), 41)
    lat = _rand((B, T, d_c + d_r), 42)
    got = oracle.decode_mla(qn, qr, lat, lens, 0.41, d_c)
    ref = np.array(brute.brute_mla(qn, qr, lat, lens, 0.41, d_c))
    assert np.abs(got - ref).max() <= 1e-12


# --------------------------------------------------------------------------- closed forms

def test_single_position_returns_its_value_exactly():
    q = _rand((2, 4, 8), 50)
    k = _rand((2, 2, 6, 8), 51)
    v = _rand((2, 2, 6, 8), 52)
    got = oracle.decode_gqa(q, k, v, [1, 1], 0.9)
    for i in range(4):
        assert np.array_equal(got[:, i], v[:, i // 2, 0].numpy())


def test_equal_keys_average_the_values():
    B, h_q, h_kv, T, d = 1, 4, 2, 9, 5
    q = _rand((B, h_q, d), 53)
    k = _rand((B, h_kv, 1, d), 54).expand(B, h_kv, T, d).contiguous()
    v = _rand((B, h_kv, T, d), 55)
    got = oracle.decode_gqa(q, k, v, [6], 1.3)
    for i in range(h_q):
        assert np.abs(got[0, i] - v[0, i // 2, :6].numpy().mean(axis=0)).max() <= 1e-14


def test_worked_example_weights():
    ex = _load("worked_example.json")
    vals = _rand((2, 7), 56)                               # value vectors of tokens 5 and 12
    w1, w3 = ex["heads"]["1"], ex["heads"]["3"]
    # One key dimension; scores equal to ln(weight) give exactly those weights.
    k = torch.tensor([[math.log(w1[0])], [math.log(w1[1])]], dtype=torch.float64)
    q = torch.tensor([[1.0], [0.3], [0.0]], dtype=torch.float64)   # heads 1, 2, 3; head 3 scores equally
    out = oracle.decode_gqa(q[None], k[None, None], vals[None, None], [2], 1.0)
    assert np.abs(out[0, 0] - (w1[0] * vals[0] + w1[1] * vals[1]).numpy()).max() <= 1e-15
    assert np.abs(out[0, 2] - (w3[0] * vals[0] + w3[1] * vals[1]).numpy()).max() <= 1e-15


def test_dominant_score_and_no_overflow():
    """Scores of order 1e4 must not overflow: the row maximum is subtracted before exp."""
    d, T = 4, 6
    k = torch.zeros(1, 1, T, d, dtype=torch.float64)
    k[0, 0, :, 0] = torch.tensor([1.0, 3.0, 2.0, -1.0, 2.9, 0.0])
    q = torch.tensor([[[5000.0, 0, 0, 0]]], dtype=torch.float64)
    v = _rand((1, 1, T, d), 57)
    out = oracle.decode_gqa(q, k, v, [T], 1.0)
    assert np.isfinite(out).all()
    assert np.array_equal(out[0, 0], v[0, 0, 1].numpy())   # every other weight underflows to 0


# --------------------------------------------------------------------------- invariants

def test_weights_are_a_distribution():
    q = _rand((3, 6, 10), 60)
    k = _rand((3, 3, 40, 10), 61)
    for W in oracle.decode_gqa_weights(q, k, [40, 13, 1], 0.31):
        assert (W >= 0).all()
        assert np.abs(W.sum(axis=1) - 1.0).max() <= 1e-14


@pytest.mark.parametrize("h_q,h_kv", [(6, 3), (8, 1), (4, 4), (12, 2)])
def test_weights_equal_sdpa_with_one_hot_values(h_q, h_kv):
    """The weights against a library routine: with the identity matrix as the
    values (value of position t = unit vector e_t), SDPA's output row is the
    softmax weight vector itself. Group map, scale and lengths all enter."""
    B, T, d = 3, 23, 7
    q = _rand((B, h_q, d), 160 + h_q)
    k = _rand((B, h_kv, T, d), 170 + h_kv)
    lens = [23, 9, 1]
    got = oracle.decode_gqa_weights(q, k, lens, 0.43)
    for b, n in enumerate(lens):
        eye = torch.eye(n, dtype=torch.float64).expand(1, h_kv, n, n)
        ref = F.scaled_dot_product_attention(q[b:b + 1, :, None], k[b:b + 1, :, :n], eye,
                                             scale=0.43, enable_gqa=True)[0, :, 0]
        assert got[b].shape == (h_q, n)
        assert np.abs(got[b] - ref.numpy()).max() <= 1e-14
    # and weights @ V is the decode output
    v = _rand((B, h_kv, T, 5), 180)
    out = oracle.decode_gqa(q, k, v, lens, 0.43)
    g = h_q // h_kv
    for b, n in enumerate(lens):
        for i in range(h_q):
            assert np.abs(got[b][i] @ v[b, i // g, :n].numpy() - out[b, i]).max() <= 1e-14


def test_position_and_batch_permutations():
    B, h_q, h_kv, T, d = 3, 4, 2, 12, 6
    q = _rand((B, h_q, d), 62)
    k = _rand((B, h_kv, T, d), 63)
    v = _rand((B, h_kv, T, d), 64)
    lens = [12, 8, 5]
    base = oracle.decode_gqa(q, k, v, lens, 0.4)
    perm = torch.randperm(8, generator=torch.Generator().manual_seed(1))
    k2, v2 = k.clone(), v.clone()
    k2[1, :, :8] = k[1, :, perm]
    v2[1, :, :8] = v[1, :, perm]
    assert np.abs(oracle.decode_gqa(q, k2, v2, lens, 0.4) - base).max() <= 1e-14
    bp = [2, 0, 1]
    got = oracle.decode_gqa(q[bp], k[bp], v[bp], [lens[i] for i in bp], 0.4)
    assert np.array_equal(got, base[bp])


def test_padding_is_never_read():
    B, h_q, h_kv, T, d = 2, 4, 1, 10, 4
    q = _rand((B, h_q, d), 65)
    k = _rand((B, h_kv, T, d), 66)
    v = _rand((B, h_kv, T, d), 67)
    lens = [6, 3]
    base = oracle.decode_gqa(q, k, v, lens, 0.5)
    k2, v2 = k.clone(), v.clone()
    k2[0, :, 6:] = float("nan")
    v2[0, :, 6:] = float("inf")
    k2[1, :, 3:] = float("nan")
    v2[1, :, 3:] = float("nan")
    got = oracle.decode_gqa(q, k2, v2, lens, 0.5)
    assert np.array_equal(got, base) and np.isfinite(got).all()
    lat = _rand((B, T, 6), 68)
    lat2 = lat.clone()
    lat2[0, 6:] = float("nan")
    lat2[1, 3:] = float("nan")
    qn, qr = _rand((B, 3, 4), 69), _rand((B, 3, 2), 70)
    assert np.array_equal(oracle.decode_mla(qn, qr, lat2, lens, 0.5, 4),
                          oracle.decode_mla(qn, qr, lat, lens, 0.5, 4))


def test_zero_length_and_clamping():
    q = _rand((3, 2, 4), 71)
    k = _rand((3, 1, 5, 4), 72)
    v = _rand((3, 1, 5, 4), 73)
    got = oracle.decode_gqa(q, k, v, [0, 9, -3], 0.5)
    assert np.array_equal(got[0], np.zeros((2, 4)))
    assert np.array_equal(got[2], np.zeros((2, 4)))
    assert np.array_equal(got[1], oracle.decode_gqa(q, k, v, [0, 5, 0], 0.5)[1])


def test_bf16_inputs_are_widened_exactly():
    q = _rand((1, 2, 8), 74, torch.bfloat16)
    k = _rand((1, 1, 5, 8), 75, torch.bfloat16)
    v = _rand((1, 1, 5, 8), 76, torch.bfloat16)
    a = oracle.decode_gqa(q, k, v, [5], 0.25)
    b = oracle.decode_gqa(q.double(), k.double(), v.double(), [5], 0.25)
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------- MLA

def test_mla_absorption_identity():
    """Scoring against up-projected keys equals scoring the absorbed query against the latent,
    and averaging up-projected values equals up-projecting the averaged latent."""
    B, H, T, d_c, d_r, d_h = 2, 4, 9, 16, 4, 6
    c = _rand((B, T, d_c), 80)
    kr = _rand((B, T, d_r), 81)
    W_uk = _rand((H, d_c, d_h), 82)
    W_uv = _rand((H, d_c, d_h), 83)
    q = _rand((B, H, d_h), 84)          # per-head query before absorption
    qr = _rand((B, H, d_r), 85)
    lens = [9, 4]
    scale = 1.0 / math.sqrt(d_h + d_r)
    # un-absorbed: materialise per-head keys and values from the latent
    ref = np.zeros((B, H, d_h))
    for b in range(B):
        n = lens[b]
        for h in range(H):
            kh = (c[b, :n] @ W_uk[h]).numpy()
            vh = (c[b, :n] @ W_uv[h]).numpy()
            s = scale * (kh @ q[b, h].numpy() + kr[b, :n].numpy() @ qr[b, h].numpy())
            w = np.exp(s - s.max())
            ref[b, h] = (w / w.sum()) @ vh
    q_abs = torch.einsum("bhd,hcd->bhc", q, W_uk)
    lat = torch.cat([c, kr], dim=-1)
    o_lat = oracle.decode_mla(q_abs, qr, lat, lens, scale, d_c)
    got = np.einsum("bhc,hcd->bhd", o_lat, W_uv.numpy())
    assert np.abs(got - ref).max() <= 1e-10


def test_mla_is_mqa_with_one_wide_head():
    B, H, T, d_c, d_r = 2, 6, 11, 12, 4
    qn, qr = _rand((B, H, d_c), 86), _rand((B, H, d_r), 87)
    lat = _rand((B, T, d_c + d_r), 88)
    lens = [11, 3]
    got = oracle.decode_mla(qn, qr, lat, lens, 0.2, d_c)
    q = torch.cat([qn, qr], dim=-1)
    via_gqa = oracle.decode_gqa(q, lat[:, None], lat[:, None, :, :d_c], lens, 0.2)
    assert np.abs(got - via_gqa).max() <= 1e-13


def test_mla_rotary_part_enters_the_score_only():
    B, H, T, d_c, d_r = 1, 3, 8, 6, 2
    qn, qr = _rand((B, H, d_c), 89), _rand((B, H, d_r), 90)
    lat = _rand((B, T, d_c + d_r), 91)
    a = oracle.decode_mla(qn, qr, lat, [T], 0.5, d_c)
    b = oracle.decode_mla(qn, torch.zeros_like(qr), lat, [T], 0.5, d_c)
    assert np.abs(a - b).max() > 1e-3                      # the rotary score term matters
    lat2 = lat.clone()
    lat2[..., d_c:] = 0.0
    c = oracle.decode_mla(qn, qr, lat2, [T], 0.5, d_c)
    d = oracle.decode_mla(qn, torch.zeros_like(qr), lat, [T], 0.5, d_c)
    assert np.array_equal(c, d)                             # with no rotary score, keys are the latent alone


# --------------------------------------------------------------------------- log-sum-exp

def test_lse_closed_form_and_brute():
    # scores ln 2 and ln 3 (one key dimension, q = 1, scale 1): log(2 + 3)
    k = torch.tensor([[[[math.log(2.0)], [math.log(3.0)], [99.0]]]], dtype=torch.float64)
    q = torch.ones(1, 1, 1, dtype=torch.float64)
    assert abs(oracle.decode_gqa_lse(q, k, [2], 1.0)[0, 0] - math.log(5.0)) <= 1e-15
    assert oracle.decode_gqa_lse(q, k, [0], 1.0)[0, 0] == -np.inf
    # against scalar loops with math.fsum, and the weights recovered from it sum to one
    qq, kk = _rand((2, 6, 5), 92), _rand((2, 3, 9, 5), 93)
    lse = oracle.decode_gqa_lse(qq, kk, [9, 4], 0.6)
    for b, n in enumerate([9, 4]):
        for i in range(6):
            s = [0.6 * math.fsum(x * y for x, y in zip(qq[b, i].tolist(), kk[b, i // 2, t].tolist()))
                 for t in range(n)]
            assert abs(lse[b, i] - math.log(math.fsum(math.exp(x) for x in s))) <= 1e-12
            assert abs(math.fsum(math.exp(x - lse[b, i]) for x in s) - 1.0) <= 1e-14
