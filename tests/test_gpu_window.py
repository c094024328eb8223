"""GPU parity of sliding-window decode against the oracle.

Tolerances as for the full decode (bf16 storage: 2e-3 plus half a bf16 ulp of
the reference for a bf16 output; fp32: 1e-5). Positions before the window
and past the end hold NaN: they must never be read. A window at least as
long as the sequence must reproduce the full decode bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu


def _m():
    import mla_kv_cache_amd as m
    return m


def _f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _half_ulp_bf16(x):
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


CASES = [
    # (B, h_q, h_kv, D, T_max, dtype, lens, window)
    (3, 8, 2, 128, 1000, torch.bfloat16, [1000, 517, 3], 100),
    (2, 28, 4, 128, 1500, torch.bfloat16, [1500, 300], 512),   # groups of 7
    (2, 32, 32, 128, 2100, torch.bfloat16, [2100, 1500], 700),
    (2, 16, 2, 128, 3000, torch.bfloat16, [3000, 64], 1),
    (2, 64, 8, 128, 5000, torch.bfloat16, [5000, 4097], 4096),
    (2, 32, 2, 128, 900, torch.bfloat16, [900, 300], 65),
    (2, 16, 4, 64, 1200, torch.bfloat16, [1200, 10], 513),
    (3, 32, 1, 128, 2000, torch.bfloat16, [2000, 1000, 40], 300),   # MQA, matrix cores
    (2, 128, 1, 64, 900, torch.bfloat16, [900, 129], 128),
    (2, 64, 1, 128, 700, torch.float32, [700, 90], 100),
    (2, 8, 8, 64, 300, torch.float32, [300, 257], 33),
    (2, 16, 4, 128, 513, torch.float32, [513, 200], 256),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}_hq{c[1]}_hkv{c[2]}_D{c[3]}_w{c[7]}_{str(c[5])[6:]}")
def test_window_matches_oracle(gpu, case):
    m = _m()
    B, h_q, h_kv, D, T, dt, lens, window = case
    w = W.small_gqa(B, h_q, h_kv, D, T, dtype=dt, seed=13)
    q, k, v, l = W.gqa_inputs(w, device="cpu", seq_lens=lens)
    for b, n in enumerate(lens):          # outside [n - window, n): never read
        lo = oracle.window_start(n, window)
        k[b, :, :lo] = float("nan")
        v[b, :, :lo] = float("nan")
        k[b, :, n:] = float("nan")
        v[b, :, n:] = float("nan")
    ref = oracle.decode_gqa_window(q, k, v, l, w.scale, window)
    out = m.attn_decode_gqa_window(q.to(gpu), k.to(gpu), v.to(gpu), l.to(gpu), window, scale=w.scale)
    got = _f64(out)
    assert np.isfinite(got).all()
    tol = 1e-5 if dt == torch.float32 else 2e-3
    bound = tol + (_half_ulp_bf16(ref) if dt == torch.bfloat16 else 0.0)
    assert np.all(np.abs(got - ref) <= bound), float(np.abs(got - ref).max())


def test_window_covering_the_sequence_is_the_full_decode(gpu):
    m = _m()
    w = W.small_gqa(2, 16, 2, 128, 1500, dtype=torch.bfloat16, seed=14)
    q, k, v, l = W.gqa_inputs(w, device="cpu", seq_lens=[1500, 900])
    args = (q.to(gpu), k.to(gpu), v.to(gpu), l.to(gpu))
    full = m.attn_decode_gqa(*args, scale=w.scale)
    for window in (1500, 1 << 20):
        out = m.attn_decode_gqa_window(*args, window, scale=w.scale)
        assert torch.equal(out.view(torch.int16), full.view(torch.int16))


def test_full_size_window_every_row(gpu):
    """The 8B-shaped layer (B=32, h_q=32, h_kv=8, D=128, T=4096) with Mistral's 4096 window
    cut to 1024, and the 70B-shaped ragged layer with the full 4096 window: every row
    against the oracle."""
    m = _m()
    wl = W.GQA4_8B
    q, k, v, l = W.gqa_inputs(wl, device="cpu")
    window = 1024
    out = _f64(m.attn_decode_gqa_window(q.to(gpu), k.to(gpu), v.to(gpu), l.to(gpu), window, scale=wl.scale))
    for b in range(wl.B):
        ref = oracle.decode_gqa_window(q[b:b + 1], k[b:b + 1], v[b:b + 1], l[b:b + 1], wl.scale, window)[0]
        assert np.all(np.abs(out[b] - ref) <= 2e-3 + _half_ulp_bf16(ref)), b
        assert np.all(np.abs(out[b] - ref) <= _half_ulp_bf16(ref) + 1e-5), b  # rounded once to bf16
    w8 = W.GQA8_70B
    q, k, v, l = W.gqa_inputs(w8, device="cpu")
    out = _f64(m.attn_decode_gqa_window(q.to(gpu), k.to(gpu), v.to(gpu), l.to(gpu), 4096, scale=w8.scale))
    for b in range(w8.B):
        ref = oracle.decode_gqa_window(q[b:b + 1], k[b:b + 1], v[b:b + 1], l[b:b + 1], w8.scale, 4096)[0]
        assert np.all(np.abs(out[b] - ref) <= 2e-3 + _half_ulp_bf16(ref)), b
        assert np.all(np.abs(out[b] - ref) <= _half_ulp_bf16(ref) + 1e-5), b  # rounded once to bf16
