"""GPU parity of the MLA absorption products against the oracle.

bf16 inputs, fp32 accumulation, bf16 output: the bound is half a bf16 ulp of
the fp64 reference (the output rounding) plus 1e-5 relative for the fp32
accumulation. Ragged batches (B not a multiple of the 32-row tile) check the
masked rows; several column groups check the work-group split. The whole
absorbed layer (absorb, decode over the latent, up-project) is checked stage
by stage against the oracle on the GPU's own intermediates, and end to end.
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


def _bound(ref):
    return _half_ulp_bf16(ref) + 1e-5 * np.abs(ref) + 1e-6


def _rand(shape, seed, scale=1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float32) * scale).to(torch.bfloat16)


@pytest.mark.parametrize("B,H,d_h,d_c", [(64, 128, 128, 512), (5, 3, 64, 96), (33, 2, 16, 32), (70, 4, 128, 160)])
def test_absorb_q_matches_oracle(gpu, B, H, d_h, d_c):
    m = _m()
    q = _rand((B, H, d_h), 1)
    w = _rand((H, d_c, d_h), 2, 1.0 / np.sqrt(d_c))        # the page's init scale
    got = _f64(m.attn_mla_absorb_q(q.to(gpu), w.to(gpu)))
    ref = oracle.absorb_q(q, w)
    assert np.all(np.abs(got - ref) <= _bound(ref)), float(np.abs(got - ref).max())


@pytest.mark.parametrize("B,H,d_c,d_v", [(64, 128, 512, 128), (5, 3, 160, 96), (33, 2, 16, 32), (70, 2, 512, 256),
                                         (3, 1, 272, 160)])
def test_up_v_matches_oracle(gpu, B, H, d_c, d_v):
    m = _m()
    o = _rand((B, H, d_c), 3, 0.3)
    w = _rand((H, d_c, d_v), 4, 1.0 / np.sqrt(d_c))
    got = _f64(m.attn_mla_up_v(o.to(gpu), w.to(gpu)))
    ref = oracle.up_v(o, w)
    assert np.all(np.abs(got - ref) <= _bound(ref)), float(np.abs(got - ref).max())


def test_absorbed_layer_stage_by_stage(gpu):
    """DeepSeek-V2 shapes (H=128, d_h=128, d_c=512, d_r=64, d_v=128), B=8, T=1024."""
    m = _m()
    B, H, d_h, d_c, d_r, d_v, T = 8, 128, 128, 512, 64, 128, 1024
    wl = W.small_mla(B, H, T, seed=51)
    _, qr, lat, lens = W.mla_inputs(wl, device="cpu", seq_lens=[1024, 700, 513, 64, 1, 900, 333, 1000])
    q = _rand((B, H, d_h), 52)
    w_uk = _rand((H, d_c, d_h), 53, 1.0 / np.sqrt(d_c))
    w_uv = _rand((H, d_c, d_v), 54, 1.0 / np.sqrt(d_c))
    scale = 1.0 / np.sqrt(d_h + d_r)
    q_lat = m.attn_mla_absorb_q(q.to(gpu), w_uk.to(gpu))
    ref_lat = oracle.absorb_q(q, w_uk)
    assert np.all(np.abs(_f64(q_lat) - ref_lat) <= _bound(ref_lat))
    o_lat = m.attn_decode_mla(q_lat, qr.to(gpu), lat.to(gpu), lens.to(gpu), scale)
    ref_o = oracle.decode_mla(q_lat.cpu(), qr, lat, lens, scale, d_c)
    assert np.all(np.abs(_f64(o_lat) - ref_o) <= 2e-3 + _half_ulp_bf16(ref_o))
    out = m.attn_mla_up_v(o_lat, w_uv.to(gpu))
    ref = oracle.up_v(o_lat.cpu(), w_uv)
    assert np.all(np.abs(_f64(out) - ref) <= _bound(ref))
    # end to end against the fp64 chain on the exact inputs: three bf16 roundings in between
    e2e = oracle.up_v(oracle.decode_mla(ref_lat, qr, lat, lens, scale, d_c), w_uv)
    assert np.abs(_f64(out) - e2e).max() <= 2e-2
