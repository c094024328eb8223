"""GPU parity at the largest shapes the library accepts.

* Longest rows: a (sequence, KV head) slab of the contiguous caches is
  addressed with 32-bit byte offsets, so the host accepts T_max * row bytes
  below 2^31 and refuses 2^31. The tests run one row below that limit, with
  two slabs per cache (the second starts past 4 GiB of the tensor) or two
  sequences (MLA), against the fp64 oracle on the full rows.
* Most sequences: B = 65535, the host's limit, with short ragged rows.
* Page pools past 4 GiB: every used page lies beyond the first 4 GiB of its
  pool (page offsets are 64-bit), the rest of the pool is zeros; the paged
  decode must give the contiguous decode's bits and match the oracle.

The scores of long rows are made peaked (the query scaled by 4, exact in
bf16) so that each output is carried by a few rows and a misread row changes
it by O(1); the last row of each sequence holds a copy of one head's query,
so that head's output is that last row, the highest byte offset of the slab.
Tolerances are those of the other parity tests (2e-3 on fp32-written results,
plus half a bf16 ulp of the oracle value on bf16 results).
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


def _half_ulp_bf16(x):
    a = np.abs(x)
    return 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - 8)


def _f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _assert_bf16_close(out, ref, what):
    err = np.abs(_f64(out) - ref)
    bad = err > 2e-3 + _half_ulp_bf16(ref)
    assert not bad.any(), (what, float(err.max()), np.argwhere(bad)[:4].tolist())


# Largest row count below a slab of 2^31 bytes, in whole 64-row tiles.
def _longest_rows(row_bytes):
    return (2 ** 31 - 1) // row_bytes // 64 * 64


def test_longest_gqa_rows(gpu):
    m = _m()
    D, h_kv = 128, 2
    T = _longest_rows(D * 2)
    with pytest.raises(m.AttnError):   # a slab of exactly 2^31 bytes is refused
        m.attn_decode_gqa_plan(1, 16, h_kv, D, 2 ** 31 // (D * 2))
    n = T - 3                          # ragged tail inside the last tile
    w = W.small_gqa(1, 16, h_kv, D, T, seed=71)
    q, k, v, lens = W.gqa_inputs(w, seq_lens=[n])
    for j in range(h_kv):              # head 8 j scores its KV head's last row far above the rest
        k[0, j, n - 1] = q[0, 8 * j] * 2
    q = q * 4
    gk, gv, gl = k.to(gpu), v.to(gpu), lens.to(gpu)
    # groups of 8 (16x16 matrix-core kernel) and of 4 (position-per-lane kernel)
    for heads in (list(range(16)), [0, 1, 2, 3, 8, 9, 10, 11]):
        qs = q[:, heads].contiguous()
        ref = oracle.decode_gqa(qs, k, v, lens, w.scale)
        for j in range(h_kv):          # the planted head returns the last row
            h = heads.index(8 * j)
            assert np.abs(ref[0, h] - _f64(v[0, j, n - 1])).max() < 1e-6
        gq = qs.to(gpu)
        _assert_bf16_close(m.attn_decode_gqa(gq, gk, gv, gl, scale=w.scale), ref, len(heads))
        po, pl = m.attn_decode_gqa_partial(gq, gk, gv, gl, 4096, scale=w.scale)
        got = m.attn_decode_merge(po, pl, gl, T, 4096, out_dtype=torch.float32)
        err = float(np.abs(_f64(got) - ref).max())
        assert err <= 2e-3, (len(heads), err)
        del po, pl, got
    torch.cuda.synchronize()


def test_longest_mla_rows(gpu):
    m = _m()
    row = (512 + 64) * 2
    T = _longest_rows(row)
    with pytest.raises(m.AttnError):
        m.attn_decode_mla_plan(1, 128, 512, 64, (2 ** 31 + row - 1) // row)
    lens = [T, T - 7]
    w = W.small_mla(2, 128, T, seed=72)
    qn, qr, lat, l = W.mla_inputs(w, seq_lens=lens)
    for b, n in enumerate(lens):       # head 0 scores the sequence's last row far above the rest
        lat[b, n - 1, :512] = qn[b, 0]
        lat[b, n - 1, 512:] = qr[b, 0]
    qn, qr = qn * 4, qr * 4
    ref = oracle.decode_mla(qn, qr, lat, l, w.scale, w.d_c)
    for b, n in enumerate(lens):
        assert np.abs(ref[b, 0] - _f64(lat[b, n - 1, :512])).max() < 1e-6
    gqn, gqr, glat, gl = qn.to(gpu), qr.to(gpu), lat.to(gpu), l.to(gpu)
    del lat
    _assert_bf16_close(m.attn_decode_mla(gqn, gqr, glat, gl, w.scale), ref, "mla")
    P = 32768
    po, pl = m.attn_decode_mla_partial(gqn, gqr, glat, gl, w.scale, P)
    got = m.attn_decode_merge(po, pl, gl, T, P, out_dtype=torch.float32)
    err = float(np.abs(_f64(got) - ref).max())
    assert err <= 2e-3, err
    torch.cuda.synchronize()


def _many_lens(B, T, seed):
    g = torch.Generator().manual_seed(seed)
    lens = torch.randint(0, T + 1, (B,), generator=g, dtype=torch.int32)
    lens[::5] = 0
    lens[1::7] = T
    return lens


@pytest.mark.parametrize("h_q", [8, 16])
def test_most_gqa_sequences(gpu, h_q):
    m = _m()
    B, h_kv, D, T = 65535, 2, 64, 24
    with pytest.raises(m.AttnError):
        m.attn_decode_gqa_plan(B + 1, h_q, h_kv, D, T)
    lens = _many_lens(B, T, 73 + h_q)
    w = W.small_gqa(B, h_q, h_kv, D, T, seed=74 + h_q)
    q, k, v, l = W.gqa_inputs(w, seq_lens=lens)
    ref = oracle.decode_gqa(q, k, v, l, w.scale)
    gq, gk, gv, gl = q.to(gpu), k.to(gpu), v.to(gpu), l.to(gpu)
    out = m.attn_decode_gqa(gq, gk, gv, gl, scale=w.scale)
    _assert_bf16_close(out, ref, h_q)
    empty = (lens == 0).nonzero().flatten().to(gpu)
    assert torch.equal(out[empty], torch.zeros_like(out[empty]))


def test_most_mla_sequences(gpu):
    m = _m()
    B, H, T = 65535, 32, 12
    with pytest.raises(m.AttnError):
        m.attn_decode_mla_plan(B + 1, H, 512, 64, T)
    lens = _many_lens(B, T, 75)
    w = W.small_mla(B, H, T, seed=76)
    qn, qr, lat, l = W.mla_inputs(w, seq_lens=lens)
    ref = oracle.decode_mla(qn, qr, lat, l, w.scale, w.d_c)
    out = m.attn_decode_mla(qn.to(gpu), qr.to(gpu), lat.to(gpu), l.to(gpu), w.scale)
    _assert_bf16_close(out, ref, "mla")
    empty = (lens == 0).nonzero().flatten().to(gpu)
    assert torch.equal(out[empty], torch.zeros_like(out[empty]))


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16)


def _high_pages(cache, lens, page_size, num_pages, gpu):
    """Scatter the used pages of cache [B, heads, T, row] to the top of a zero pool of num_pages
    pages (every 37th slot from the last down); returns (CPU pool, GPU pool, table)."""
    B, H, T, R = cache.shape
    npg = T // page_size
    used = [(b, i) for b in range(B) for i in range(npg) if i * page_size < lens[b]]
    pool = torch.zeros((num_pages, H, page_size, R), dtype=cache.dtype)
    gpool = torch.zeros((num_pages, H, page_size, R), dtype=cache.dtype, device=gpu)
    table = torch.full((B, npg), 1 << 30, dtype=torch.int32)   # past the last page: never read
    for k, (b, i) in enumerate(used):
        slot = num_pages - 1 - 37 * k
        pool[slot] = cache[b, :, i * page_size:(i + 1) * page_size]
        gpool[slot] = pool[slot].to(gpu)
        table[b, i] = slot
    return pool, gpool, table


def test_paged_pools_past_4gib(gpu):
    m = _m()
    ps, lens = 64, [1024, 517, 1000]
    w = W.small_gqa(3, 64, 8, 128, 1024, seed=77)
    q, k, v, l = W.gqa_inputs(w, seq_lens=lens)
    num_pages = 36000                                  # 128 KiB pages: 4.4 GiB per pool
    kp, gkp, table = _high_pages(k, lens, ps, num_pages, gpu)
    vp, gvp, _ = _high_pages(v, lens, ps, num_pages, gpu)
    assert int(table[table < (1 << 30)].min()) * kp[0].numel() * 2 > 2 ** 32
    gt, gl, gk, gv = table.to(gpu), l.to(gpu), k.to(gpu), v.to(gpu)
    for g in (8, 4):                                   # 16x16 matrix-core and position-per-lane kernels
        qs = q.view(3, 8, 8, 128)[:, :, :g].reshape(3, 8 * g, 128).contiguous()
        gq = qs.to(gpu)
        out = m.attn_decode_gqa_paged(gq, gkp, gvp, gt, gl, scale=w.scale)
        lin = m.attn_decode_gqa(gq, gk, gv, gl, scale=w.scale)
        assert torch.equal(_bits(out), _bits(lin)), g
        ref = oracle.decode_gqa_paged(qs, kp, vp, table, l, w.scale, ps)
        _assert_bf16_close(out, ref, g)
    del kp, gkp, vp, gvp
    torch.cuda.synchronize()

    lens = [1024, 700]
    wm = W.small_mla(2, 128, 1024, seed=78)
    qn, qr, lat, l = W.mla_inputs(wm, seq_lens=lens)
    num_pages = 62000                                  # 72 KiB pages: 4.3 GiB
    lp, glp, table = _high_pages(lat[:, None], lens, ps, num_pages, gpu)
    lp, glp = lp[:, 0], glp[:, 0]
    assert int(table[table < (1 << 30)].min()) * lp[0].numel() * 2 > 2 ** 32
    gqn, gqr, gl = qn.to(gpu), qr.to(gpu), l.to(gpu)
    out = m.attn_decode_mla_paged(gqn, gqr, glp, table.to(gpu), gl, wm.scale)
    lin = m.attn_decode_mla(gqn, gqr, lat.to(gpu), gl, wm.scale)
    assert torch.equal(_bits(out), _bits(lin))
    ref = oracle.decode_mla_paged(qn, qr, lp, table, l, wm.scale, wm.d_c, ps)
    _assert_bf16_close(out, ref, "mla")
