"""GPU parity of the decode step (append the new row, then attend) against the oracle.

* The cache writes (attn_kv_append, attn_latent_append and the writes inside
  the fused steps) are byte work: compared bit for bit with the oracle's
  caches, over the whole cache, so a stray write anywhere fails.
* The fused step's output equals, bit for bit, the library's own append
  followed by the plain decode over seq_lens + 1 (the same kernels on the
  same data, in a fixed order), and the oracle's step within the decode
  tolerances (bf16 storage: 2e-3 plus half a bf16 ulp of the reference for a
  bf16 output; fp32 storage: 1e-5).
* A token-by-token walk from an empty cache, and lengths at the edges: empty
  (0), negative (read as 0), the last row (T_max - 1) and a full cache.
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


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


def _rand(shape, seed, dtype):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(dtype)


GQA_CASES = [
    # (B, h_q, h_kv, D, T_max, dtype, lens before the step)
    (4, 8, 2, 128, 1000, torch.bfloat16, [0, 517, 999, 1000]),
    (3, 32, 32, 128, 700, torch.bfloat16, [699, 300, -5]),
    (2, 16, 2, 128, 1500, torch.bfloat16, [1499, 1023]),
    (2, 16, 4, 64, 640, torch.bfloat16, [639, 64]),
    (2, 16, 1, 128, 900, torch.bfloat16, [63, 511]),
    (2, 32, 2, 128, 777, torch.bfloat16, [776, 100]),
    (3, 32, 1, 128, 900, torch.bfloat16, [899, 128, 0]),     # MQA, matrix cores
    (2, 28, 4, 128, 700, torch.bfloat16, [699, 0]),          # groups of 7
    (2, 128, 2, 64, 500, torch.bfloat16, [255, 499]),
    (2, 32, 1, 64, 300, torch.float32, [299, 31]),
    (2, 8, 8, 64, 300, torch.float32, [299, 0]),
    (2, 16, 4, 128, 513, torch.float32, [512, 200]),
]


def _gqa_inputs(case, seed=5):
    B, h_q, h_kv, D, T, dt, lens = case
    w = W.small_gqa(B, h_q, h_kv, D, T, dtype=dt, seed=seed)
    q, k, v, _ = W.gqa_inputs(w, device="cpu", seq_lens=[min(max(x, 0), T) for x in lens])
    kn = _rand((B, h_kv, D), seed + 100, dt)
    vn = _rand((B, h_kv, D), seed + 101, dt)
    return w, q, k, v, kn, vn, torch.tensor(lens, dtype=torch.int32)


@pytest.mark.parametrize("case", GQA_CASES, ids=lambda c: f"B{c[0]}_hq{c[1]}_hkv{c[2]}_D{c[3]}_{str(c[5])[6:]}")
def test_kv_append_is_bit_exact(gpu, case):
    m = _m()
    w, q, k, v, kn, vn, lens = _gqa_inputs(case)
    gk, gv = k.to(gpu), v.to(gpu)
    m.attn_kv_append(kn.to(gpu), vn.to(gpu), gk, gv, lens.to(gpu))
    ek, ev = oracle.append_kv(k, v, kn, vn, lens)
    assert torch.equal(_bits(gk), _bits(ek)) and torch.equal(_bits(gv), _bits(ev))


@pytest.mark.parametrize("case", GQA_CASES, ids=lambda c: f"B{c[0]}_hq{c[1]}_hkv{c[2]}_D{c[3]}_{str(c[5])[6:]}")
def test_gqa_step_matches_oracle_and_append_then_decode(gpu, case):
    m = _m()
    w, q, k, v, kn, vn, lens = _gqa_inputs(case)
    ref, ek, ev = oracle.decode_gqa_step(q, kn, vn, k, v, lens, w.scale)
    gq, gkn, gvn, gl = q.to(gpu), kn.to(gpu), vn.to(gpu), lens.to(gpu)
    gk, gv = k.to(gpu), v.to(gpu)
    out = m.attn_decode_gqa_step(gq, gkn, gvn, gk, gv, gl, scale=w.scale)
    assert torch.equal(_bits(gk), _bits(ek)) and torch.equal(_bits(gv), _bits(ev))
    got = _f64(out)
    tol = 1e-5 if w.dtype == torch.float32 else 2e-3
    bound = tol + (_half_ulp_bf16(ref) if w.dtype == torch.bfloat16 else 0.0)
    assert np.all(np.abs(got - ref) <= bound), float(np.abs(got - ref).max())
    # the same as the library's own append followed by the plain decode over lens + 1
    gk2, gv2 = k.to(gpu), v.to(gpu)
    m.attn_kv_append(gkn, gvn, gk2, gv2, gl)
    n1 = torch.clamp(lens.to(torch.int64).clamp(min=0) + 1, max=w.T_max).to(torch.int32).to(gpu)
    out2 = m.attn_decode_gqa(gq, gk2, gv2, n1, scale=w.scale)
    assert torch.equal(_bits(out), _bits(out2))


def test_gqa_step_never_reads_past_the_new_row(gpu):
    m = _m()
    case = (2, 16, 2, 128, 1024, torch.bfloat16, [300, 700])
    w, q, k, v, kn, vn, lens = _gqa_inputs(case)
    for b, n in enumerate([300, 700]):
        k[b, :, n:] = float("nan")
        v[b, :, n:] = float("nan")
    ref, ek, ev = oracle.decode_gqa_step(q, kn, vn, k, v, lens, w.scale)
    gk, gv = k.to(gpu), v.to(gpu)
    out = m.attn_decode_gqa_step(q.to(gpu), kn.to(gpu), vn.to(gpu), gk, gv, lens.to(gpu), scale=w.scale)
    assert np.isfinite(_f64(out)).all()
    assert np.all(np.abs(_f64(out) - ref) <= 2e-3 + _half_ulp_bf16(ref))
    assert torch.equal(_bits(gk), _bits(ek)) and torch.equal(_bits(gv), _bits(ev))


def test_gqa_token_by_token_walk(gpu):
    """Steps from an empty cache: every step matches the oracle's step on the same state."""
    m = _m()
    B, h_q, h_kv, D, T_max, steps = 2, 16, 2, 128, 96, 70
    w = W.small_gqa(B, h_q, h_kv, D, T_max, dtype=torch.bfloat16, seed=9)
    kc = torch.zeros((B, h_kv, T_max, D), dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    gk, gv = kc.to(gpu), vc.to(gpu)
    for t in range(steps):
        q = _rand((B, h_q, D), 1000 + t, torch.bfloat16)
        kn = _rand((B, h_kv, D), 2000 + t, torch.bfloat16)
        vn = _rand((B, h_kv, D), 3000 + t, torch.bfloat16)
        lens = torch.full((B,), t, dtype=torch.int32)
        ref, kc, vc = oracle.decode_gqa_step(q, kn, vn, kc, vc, lens, w.scale)
        out = m.attn_decode_gqa_step(q.to(gpu), kn.to(gpu), vn.to(gpu), gk, gv, lens.to(gpu), scale=w.scale)
        assert np.all(np.abs(_f64(out) - ref) <= 2e-3 + _half_ulp_bf16(ref)), t
    assert torch.equal(_bits(gk), _bits(kc)) and torch.equal(_bits(gv), _bits(vc))


MLA_CASES = [
    # (B, H, T_max, lens before the step)
    (3, 128, 1200, [0, 700, 1199]),
    (2, 64, 700, [699, 31]),
    (2, 32, 300, [300, -1]),
    (2, 256, 400, [399, 128]),
]


@pytest.mark.parametrize("case", MLA_CASES, ids=lambda c: f"B{c[0]}_H{c[1]}_T{c[2]}")
def test_mla_step_matches_oracle_and_append_then_decode(gpu, case):
    m = _m()
    B, H, T, lens = case
    w = W.small_mla(B, H, T, seed=21)
    qn, qr, lat, _ = W.mla_inputs(w, device="cpu", seq_lens=[min(max(x, 0), T) for x in lens])
    new = _rand((B, w.d_c + w.d_r), 77, torch.bfloat16)
    ln = torch.tensor(lens, dtype=torch.int32)
    ref, elat = oracle.decode_mla_step(qn, qr, new, lat, ln, w.scale, w.d_c)
    glat = lat.to(gpu)
    out = m.attn_decode_mla_step(qn.to(gpu), qr.to(gpu), new.to(gpu), glat, ln.to(gpu), w.scale)
    assert torch.equal(_bits(glat), _bits(elat))
    assert np.all(np.abs(_f64(out) - ref) <= 2e-3 + _half_ulp_bf16(ref)), float(np.abs(_f64(out) - ref).max())
    glat2 = lat.to(gpu)
    m.attn_latent_append(new.to(gpu), glat2, ln.to(gpu))
    assert torch.equal(_bits(glat2), _bits(elat))
    n1 = torch.clamp(ln.to(torch.int64).clamp(min=0) + 1, max=T).to(torch.int32).to(gpu)
    out2 = m.attn_decode_mla(qn.to(gpu), qr.to(gpu), glat2, n1, w.scale)
    assert torch.equal(_bits(out), _bits(out2))


def test_full_size_gqa8_step_every_row(gpu):
    """The 70B-shaped layer (B=16, h_q=64, h_kv=8, D=128, T_max=32768, ragged lengths) at full
    size, through the step: every written row bit-exact, every output row against the oracle."""
    m = _m()
    w = W.GQA8_70B
    q, k, v, lens = W.gqa_inputs(w, device="cpu")
    before = (lens - 1).to(torch.int32)                     # the step appends the last row itself
    kn = k[torch.arange(w.B), :, (lens - 1).long()].clone()
    vn = v[torch.arange(w.B), :, (lens - 1).long()].clone()
    gk, gv = k.to(gpu), v.to(gpu)
    gk[torch.arange(w.B), :, (lens - 1).long()] = 0           # the step must write these rows back
    gv[torch.arange(w.B), :, (lens - 1).long()] = 0
    out = m.attn_decode_gqa_step(q.to(gpu), kn.to(gpu), vn.to(gpu), gk, gv, before.to(gpu), scale=w.scale)
    assert torch.equal(_bits(gk), _bits(k)) and torch.equal(_bits(gv), _bits(v))
    got = _f64(out)
    for b in range(w.B):
        ref = oracle.decode_gqa(q[b:b + 1], k[b:b + 1], v[b:b + 1], lens[b:b + 1], w.scale)[0]
        assert np.all(np.abs(got[b] - ref) <= 2e-3 + _half_ulp_bf16(ref))
        assert np.all(np.abs(got[b] - ref) <= _half_ulp_bf16(ref) + 1e-5)  # rounded once to bf16
