"""GPU parity of decode over a paged KV cache.

Pages are cut from a linear cache with torch's reshape and scattered over a
random permutation of physical slots; unused pages hold NaN and table
entries past a sequence's last page hold garbage indices, so any read of
them shows. The paged kernels run the same arithmetic as the contiguous ones
on the same positions in the same order, so their output must equal the
library's contiguous decode bit for bit (except bf16 pages of 16 rows, which
take the per-row kernel); it must also match the oracle within the decode
tolerances. Appends into pages are byte work and compared exactly.
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


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


def _half_ulp_bf16(x):
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def _paginate_kv(cache, lens, page_size, seed, spare=3):
    """[B, h_kv, T, D] -> (pages [num_pages, h_kv, ps, D], table int32 [B, T/ps]). Pages holding no
    valid position are not stored; their table entries and `spare` extra pages are garbage / NaN."""
    B, H, T, D = cache.shape
    npg = T // page_size
    used = [(b, i) for b in range(B) for i in range(npg) if i * page_size < lens[b]]
    g = torch.Generator().manual_seed(seed)
    slots = torch.randperm(len(used) + spare, generator=g)
    pages = torch.full((len(used) + spare, H, page_size, D), float("nan"), dtype=cache.dtype)
    table = torch.full((B, npg), -1, dtype=torch.int32)
    for k, (b, i) in enumerate(used):
        pages[slots[k]] = cache[b, :, i * page_size:(i + 1) * page_size]
        table[b, i] = int(slots[k])
    table[table < 0] = 1 << 30            # garbage past the last page: never read
    return pages, table


def _kernel(dt, D, g, ps):
    """Which kernel serves a shape (page size 0: contiguous), as the library's header states it:
    bf16 groups of 8 to 64, and of 3, 5, 6, 7, on 16 x 16 matrix-core tiles of 64 or 16 positions
    (groups up to 32, groups of 64), power-of-two groups up to 8 position-per-lane and groups of 16
    to 128 on 32 x 32 tiles (pages of 32 rows), anything else per row."""
    if dt == torch.float32:
        return "generic"
    tile16 = 64 if g <= 32 else 16
    if g & (g - 1):  # not a power of two
        return "mma16" if ps == 0 or ps % tile16 == 0 else "generic"
    if 8 <= g <= 64 and (ps == 0 or ps % tile16 == 0):
        return "mma16"
    if g <= 8 and ps % 32 == 0:
        return "po"
    if 16 <= g <= 128 and ps % 32 == 0:
        return "matrix"
    return "generic"


CASES = [
    # (B, h_q, h_kv, D, max_pages, page_size, dtype, lens)
    (3, 8, 2, 128, 16, 64, torch.bfloat16, [1024, 517, 1]),
    (2, 32, 32, 128, 6, 128, torch.bfloat16, [768, 300]),
    (2, 16, 1, 128, 4, 256, torch.bfloat16, [1000, 64]),
    (2, 64, 8, 128, 8, 256, torch.bfloat16, [2048, 1200]),
    (2, 32, 2, 128, 10, 64, torch.bfloat16, [640, 0]),
    (2, 16, 4, 64, 12, 64, torch.bfloat16, [700, 65]),
    (2, 8, 2, 128, 32, 16, torch.bfloat16, [500, 17]),          # small pages: per-row gather
    (2, 8, 2, 128, 16, 32, torch.bfloat16, [512, 33]),          # one tile per page
    (3, 32, 4, 64, 24, 32, torch.bfloat16, [700, 33, 768]),
    (3, 32, 1, 128, 16, 64, torch.bfloat16, [1024, 100, 1]),     # MQA, matrix cores
    (2, 64, 2, 128, 20, 32, torch.bfloat16, [640, 45]),          # groups of 32 in 32-row pages: 32 x 32 tiles
    (2, 12, 4, 128, 16, 64, torch.bfloat16, [1000, 100]),        # groups of 3: 16 x 16 tiles
    (2, 28, 4, 128, 32, 32, torch.bfloat16, [900, 31]),          # groups of 7 in 32-row pages: per-row gather
    (2, 128, 2, 64, 8, 32, torch.bfloat16, [256, 77]),
    (2, 64, 1, 128, 32, 16, torch.bfloat16, [500, 17]),          # 16-row pages: chunks of 16 heads
    (2, 32, 1, 64, 10, 32, torch.float32, [300, 12]),
    (2, 32, 2, 128, 20, 32, torch.bfloat16, [640, 100]),        # groups of 16 in 32-row pages
    (2, 16, 1, 64, 40, 16, torch.bfloat16, [640, 5]),           # groups of 16 in 16-row pages
    (2, 16, 2, 128, 8, 64, torch.bfloat16, [500, 64]),          # groups of 8 in 64-row pages
    (2, 16, 4, 128, 8, 64, torch.float32, [512, 200]),
    (2, 16, 8, 64, 20, 16, torch.float32, [320, 100]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}_hq{c[1]}_hkv{c[2]}_D{c[3]}_ps{c[5]}_{str(c[6])[6:]}")
def test_paged_matches_contiguous_and_oracle(gpu, case):
    m = _m()
    B, h_q, h_kv, D, max_pages, ps, dt, lens = case
    T = max_pages * ps
    w = W.small_gqa(B, h_q, h_kv, D, T, dtype=dt, seed=31)
    q, k, v, l = W.gqa_inputs(w, device="cpu", seq_lens=lens)
    kp, table = _paginate_kv(k, lens, ps, 1)
    vp, _ = _paginate_kv(v, lens, ps, 1)
    out = m.attn_decode_gqa_paged(q.to(gpu), kp.to(gpu), vp.to(gpu), table.to(gpu), l.to(gpu), scale=w.scale)
    lin = m.attn_decode_gqa(q.to(gpu), k.to(gpu), v.to(gpu), l.to(gpu), scale=w.scale)
    # The paged decode runs the contiguous decode's arithmetic in its order
    # when both take the same kernel (bit-identical); pages that do not hold
    # whole tiles of that kernel take another one: tolerance only.
    same_kernel = _kernel(dt, D, h_q // h_kv, ps) == _kernel(dt, D, h_q // h_kv, 0)
    if same_kernel:
        assert torch.equal(_bits(out), _bits(lin))
    ref = oracle.decode_gqa_paged(q, kp, vp, table, l, w.scale, ps)
    tol = 1e-5 if dt == torch.float32 else 2e-3
    bound = tol + (_half_ulp_bf16(ref) if dt == torch.bfloat16 else 0.0)
    assert np.all(np.abs(_f64(out) - ref) <= bound), float(np.abs(_f64(out) - ref).max())


def test_shared_prefix_pages(gpu):
    m = _m()
    ps, h_q, h_kv, D = 64, 16, 2, 128
    g = torch.Generator().manual_seed(5)
    pages = torch.randn((6, h_kv, ps, D), generator=g).to(torch.bfloat16)
    vpages = torch.randn((6, h_kv, ps, D), generator=g).to(torch.bfloat16)
    table = torch.tensor([[0, 1, 2, 3], [0, 1, 4, 5]], dtype=torch.int32)   # pages 0-1 shared
    lens = torch.tensor([256, 200], dtype=torch.int32)
    q = torch.randn((2, h_q, D), generator=g).to(torch.bfloat16)
    out = m.attn_decode_gqa_paged(q.to(gpu), pages.to(gpu), vpages.to(gpu), table.to(gpu), lens.to(gpu),
                                  scale=0.088)
    ref = oracle.decode_gqa_paged(q, pages, vpages, table, lens, 0.088, ps)
    assert np.all(np.abs(_f64(out) - ref) <= 2e-3 + _half_ulp_bf16(ref))


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_paged_append_is_bit_exact(gpu, dt):
    m = _m()
    ps, h_kv, D = 16, 4, 128
    g = torch.Generator().manual_seed(6)
    kp = torch.randn((10, h_kv, ps, D), generator=g).to(dt)
    vp = torch.randn((10, h_kv, ps, D), generator=g).to(dt)
    table = torch.tensor([[3, 0, 5], [1, 2, 4], [7, 8, 12345]], dtype=torch.int32)
    lens = torch.tensor([17, 48, 33], dtype=torch.int32)     # row 1 of page 0; sequence 1 full; bad entry
    kn = torch.randn((3, h_kv, D), generator=g).to(dt)
    vn = torch.randn((3, h_kv, D), generator=g).to(dt)
    gk, gv = kp.to(gpu), vp.to(gpu)
    m.attn_kv_append_paged(kn.to(gpu), vn.to(gpu), gk, gv, table.to(gpu), lens.to(gpu))
    ek, ev = oracle.append_kv_paged(kp, vp, table, kn, vn, lens, ps)
    # by hand: only sequence 0 writes (page 0, row 1); 1 is full, 2 names no page
    hk, hv = kp.clone(), vp.clone()
    hk[0, :, 1], hv[0, :, 1] = kn[0], vn[0]
    assert torch.equal(_bits(ek), _bits(hk)) and torch.equal(_bits(ev), _bits(hv))
    assert torch.equal(_bits(gk), _bits(ek)) and torch.equal(_bits(gv), _bits(ev))


MLA_CASES = [
    # (B, H, max_pages, page_size, lens)
    (3, 128, 16, 64, [1024, 500, 1]),
    (2, 64, 8, 32, [256, 31]),
    (2, 128, 4, 256, [1024, 700]),
    (2, 256, 10, 64, [640, 0]),
]


@pytest.mark.parametrize("case", MLA_CASES, ids=lambda c: f"B{c[0]}_H{c[1]}_ps{c[3]}")
def test_mla_paged_matches_contiguous_and_oracle(gpu, case):
    m = _m()
    B, H, max_pages, ps, lens = case
    T = max_pages * ps
    w = W.small_mla(B, H, T, seed=41)
    qn, qr, lat, l = W.mla_inputs(w, device="cpu", seq_lens=lens)
    lp, table = _paginate_kv(lat[:, None], lens, ps, 2)
    lp = lp[:, 0].contiguous()                                    # [num_pages, ps, 576]
    out = m.attn_decode_mla_paged(qn.to(gpu), qr.to(gpu), lp.to(gpu), table.to(gpu), l.to(gpu), w.scale)
    lin = m.attn_decode_mla(qn.to(gpu), qr.to(gpu), lat.to(gpu), l.to(gpu), w.scale)
    assert torch.equal(_bits(out), _bits(lin))
    ref = oracle.decode_mla_paged(qn, qr, lp, table, l, w.scale, w.d_c, ps)
    assert np.all(np.abs(_f64(out) - ref) <= 2e-3 + _half_ulp_bf16(ref))


def test_mla_paged_append_is_bit_exact(gpu):
    m = _m()
    ps, W_ = 32, 576
    g = torch.Generator().manual_seed(7)
    lp = torch.randn((6, ps, W_), generator=g).to(torch.bfloat16)
    table = torch.tensor([[5, 2], [0, 1]], dtype=torch.int32)
    lens = torch.tensor([40, 3], dtype=torch.int32)
    new = torch.randn((2, W_), generator=g).to(torch.bfloat16)
    gl = lp.to(gpu)
    m.attn_latent_append_paged(new.to(gpu), gl, table.to(gpu), lens.to(gpu))
    e = lp.clone()
    e[2, 8] = new[0]
    e[0, 3] = new[1]
    assert torch.equal(_bits(gl), _bits(e))


def test_full_size_gqa8_paged(gpu):
    """The 70B-shaped layer in 64-position pages (4096 pages of 8 KV heads): the paged decode
    equals the contiguous decode bit for bit; every row against the oracle."""
    m = _m()
    w = W.GQA8_70B
    q, k, v, lens = W.gqa_inputs(w, device="cpu")
    ps = 64
    kp, table = _paginate_kv(k, lens.tolist(), ps, 3, spare=0)
    vp, _ = _paginate_kv(v, lens.tolist(), ps, 3, spare=0)
    del k, v
    gq, gl = q.to(gpu), lens.to(gpu)
    out = m.attn_decode_gqa_paged(gq, kp.to(gpu), vp.to(gpu), table.to(gpu), gl, scale=w.scale)
    ref_rows = {b: oracle.decode_gqa_paged(q[b:b + 1], kp, vp, table[b:b + 1], lens[b:b + 1], w.scale, ps)[0]
                for b in range(w.B)}
    got = _f64(out)
    for b, ref in ref_rows.items():
        assert np.all(np.abs(got[b] - ref) <= 2e-3 + _half_ulp_bf16(ref))
        assert np.all(np.abs(got[b] - ref) <= _half_ulp_bf16(ref) + 1e-5)  # rounded once to bf16
