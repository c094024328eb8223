"""Host-side checks of the C ABI (no GPU needed).

* the shared library exports every function include/attn_decode.h declares,
  and the Python binding attaches a signature to each;
* the cache-size helpers reproduce the pages' printed numbers exactly and
  agree with the oracle's arithmetic on random arguments;
* every argument check returns its status before anything is enqueued
  (these calls never reach the HIP runtime, so they run without a GPU);
* the split-KV plan and workspace sizes are consistent.
"""

import ctypes
import json
import os
import random
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_decode.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def lib():
    from mla_kv_cache_amd import _lib
    san = os.environ.get("ATTN_ABI_TEST_LIB")
    if san:
        # A host-only sanitizer build of the same entry points (test_sanitized_host.py):
        # the kernel launchers are stand-ins that count every launch reached.
        lib = ctypes.CDLL(san)
        for name, (res, args) in _lib.SIGNATURES.items():
            if name == "attn_decode_gqa_noalloc":   # HIP source, not in the host-only build
                continue
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        yield lib
        n = ctypes.c_int.in_dll(lib, "attn_sanitize_launches").value
        print(f"\nsanitized library: {n} launches reached")
        assert n == 0
        return
    if not os.path.exists(_lib.LIB_PATH):
        from mla_kv_cache_amd import build
        build.build()
    yield _lib.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    from mla_kv_cache_amd import _lib
    names = _declared()
    assert len(names) >= 12
    for name in names:
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, name
    assert set(_lib.SIGNATURES) == set(names)


def test_status_strings(lib):
    for st in (OK, INVALID, UNSUPPORTED, WORKSPACE, -4, 7):
        assert lib.attn_status_str(st)


# --------------------------------------------------------------------------- helpers

def test_kv_helper_reproduces_page_numbers(lib):
    data = json.load(open(os.path.join(ROOT, "tests", "golden", "cache_bytes.json")))
    for case in data["kv"]:
        assert lib.attn_kv_cache_bytes(*case["args"]) == case["bytes"], case["cite"]
    for case in data["mla"]:
        assert lib.attn_mla_cache_bytes(*case["args"]) == case["elements"], case["cite"]


def test_mla_helper_reproduces_scaled_page_numbers(lib):
    data = json.load(open(os.path.join(ROOT, "tests", "golden", "cache_bytes.json")))
    for case in data["mla_bytes"]:
        assert lib.attn_mla_cache_bytes(*case["args"]) == case["bytes"], case["cite"]


def test_helpers_agree_with_oracle_and_saturate(lib):
    rng = random.Random(0)
    for _ in range(500):
        a = [rng.randint(0, 200), rng.randint(0, 128), rng.randint(0, 256), rng.randint(0, 1 << 20),
             rng.randint(0, 64), rng.choice([1, 2, 4])]
        assert lib.attn_kv_cache_bytes(*a) == oracle.kv_cache_bytes(*a)
        m = [a[0], rng.randint(0, 1024), rng.randint(0, 128), a[3], a[4], a[5]]
        assert lib.attn_mla_cache_bytes(*m) == oracle.mla_cache_bytes(*m)
    assert lib.attn_kv_cache_bytes(1 << 40, 1 << 20, 128, 1, 1, 2) == 2**64 - 1
    assert lib.attn_mla_cache_bytes(2**64 - 1, 1, 1, 1, 1, 1) == 2**64 - 1


def test_python_helper_defaults():
    import mla_kv_cache_amd as m
    assert m.attn_kv_cache_bytes(32, 32, 128, 1) == 524288
    assert m.attn_mla_cache_bytes(1, 512, 64, 1, 1, 1) == 576


# --------------------------------------------------------------------------- argument checks

P16 = ctypes.c_void_p(1 << 20)        # a fake, aligned, never-dereferenced device address
P16b = ctypes.c_void_p(1 << 30)
P16c = ctypes.c_void_p(1 << 34)
OUT = ctypes.c_void_p(1 << 38)
WS = ctypes.c_void_p(1 << 42)
LENS = ctypes.c_void_p(1 << 44)
NULL = ctypes.c_void_p(0)


def _gqa(lib, **kw):
    a = dict(q=P16, k=P16b, v=P16c, lens=LENS, B=2, h_q=8, h_kv=2, D=128, T=1024, scale=0.1,
             dt=BF16, out=OUT, ws=WS, wsb=1 << 30)
    a.update(kw)
    return lib.attn_decode_gqa(a["q"], a["k"], a["v"], a["lens"], a["B"], a["h_q"], a["h_kv"],
                               a["D"], a["T"], a["scale"], a["dt"], a["out"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(h_q=6, h_kv=4), INVALID),
    (dict(B=0), INVALID), (dict(h_kv=0), INVALID), (dict(T=0), INVALID), (dict(D=-1), INVALID),
    (dict(q=NULL), INVALID), (dict(k=NULL), INVALID), (dict(v=NULL), INVALID),
    (dict(lens=NULL), INVALID), (dict(out=NULL), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(T=(1 << 30) + 1), INVALID),
    (dict(T=1 << 23, B=1, h_q=2, h_kv=1), UNSUPPORTED),   # one 2 GiB K slab: past 32-bit offsets
    (dict(T=(1 << 23) - 1, B=1, h_q=2, h_kv=1, wsb=0), WORKSPACE),
    (dict(D=96), UNSUPPORTED), (dict(D=256), UNSUPPORTED),
    (dict(h_q=24, h_kv=1), UNSUPPORTED), (dict(h_q=36, h_kv=4), UNSUPPORTED),   # groups of 24, 9
    (dict(h_q=48, h_kv=4), UNSUPPORTED),              # groups of 12: not a power of two above 8
    (dict(h_q=512, h_kv=2), UNSUPPORTED),             # groups of 256: above the 128 built
    (dict(dt=7), UNSUPPORTED),
    (dict(q=ctypes.c_void_p((1 << 20) + 8)), UNSUPPORTED),
    (dict(out=ctypes.c_void_p((1 << 38) + 2)), UNSUPPORTED),
    (dict(out=P16b), INVALID),                       # output overlaps the K cache
    (dict(ws=NULL), WORKSPACE), (dict(wsb=16), WORKSPACE),
])
def test_gqa_argument_checks(lib, kw, expect):
    assert _gqa(lib, **kw) == expect


@pytest.mark.parametrize("h_q,h_kv", [(12, 4), (10, 2), (12, 2), (28, 4), (40, 8)])
def test_gqa_groups_of_three_to_seven_are_planned(lib, h_q, h_kv):
    """Every group size from 1 to 8 is built (here 3, 5, 6, 7, 5): the plan succeeds."""
    ws = ctypes.c_size_t(0)
    for dt in (0, BF16):
        assert lib.attn_decode_gqa_plan(2, h_q, h_kv, 128, 1024, dt, None, None, ctypes.byref(ws)) == OK
        assert ws.value > 0


def test_gqa_partial_and_merge_checks(lib):
    f = lib.attn_decode_gqa_partial
    args = [P16, P16b, P16c, LENS, 2, 8, 2, 128, 1024, 0.1, BF16]
    assert f(*args, 0, OUT, WS, None) == INVALID          # partition size must be >= 1
    assert f(*args, 256, OUT, NULL, None) == INVALID       # missing lse buffer
    assert f(*args, 256, OUT, OUT, None) == INVALID        # lse overlaps out
    m = lib.attn_decode_merge
    assert m(OUT, WS, LENS, 2, 8, 128, 1024, 0, BF16, P16, None) == INVALID
    assert m(OUT, WS, LENS, 2, 8, 130, 1024, 256, BF16, P16, None) == UNSUPPORTED
    assert m(OUT, WS, LENS, 2, 8, 128, 1024, 256, 5, P16, None) == UNSUPPORTED
    assert m(OUT, WS, NULL, 2, 8, 128, 1024, 256, BF16, P16, None) == INVALID
    assert m(OUT, WS, LENS, 2, 8, 128, 1024, 256, BF16, OUT, None) == INVALID


def test_mla_argument_checks(lib):
    f = lib.attn_decode_mla
    good = dict(qn=P16, qr=P16b, lat=P16c, lens=LENS, B=4, H=128, dc=512, dr=64, T=4096,
                scale=0.07, out=OUT, ws=WS, wsb=1 << 30)

    def call(**kw):
        a = dict(good)
        a.update(kw)
        return f(a["qn"], a["qr"], a["lat"], a["lens"], a["B"], a["H"], a["dc"], a["dr"], a["T"],
                 a["scale"], a["out"], a["ws"], a["wsb"], None)

    assert call(B=0) == INVALID
    assert call(qn=NULL) == INVALID
    assert call(dc=256) == UNSUPPORTED
    assert call(H=48) == UNSUPPORTED
    assert call(scale=float("nan")) == INVALID
    assert call(B=65535, H=32896, T=1) == INVALID     # 2^31 rows (b, h) or more
    assert lib.attn_decode_mla_plan(65535, 32896, 512, 64, 1, None, None, None) == INVALID
    assert lib.attn_decode_mla_plan(65535, 32768, 512, 64, 1, None, None, None) == OK
    assert call(wsb=64) == WORKSPACE
    assert call(out=P16c) == INVALID                  # output overlaps the latent cache
    assert call(lat=ctypes.c_void_p((1 << 34) + 4)) == UNSUPPORTED
    # one sequence's rows must stay below 2 GiB (32-bit offsets in the kernels)
    big = (1 << 31) // 1152 + 1
    assert call(B=1, T=big) == UNSUPPORTED
    assert call(B=1, T=big - 1, wsb=0) == WORKSPACE    # the shape passes; stops at the workspace
    assert lib.attn_decode_mla_plan(1, 128, 512, 64, big, None, None, None) == UNSUPPORTED
    assert lib.attn_decode_mla_plan(1, 128, 512, 64, big - 1, None, None, None) == OK
    P, NP, ws = ctypes.c_int(), ctypes.c_int(), ctypes.c_size_t()
    assert lib.attn_decode_mla_plan(64, 128, 512, 64, 4096, ctypes.byref(P), ctypes.byref(NP),
                                    ctypes.byref(ws)) == OK
    assert NP.value * P.value >= 4096 and 64 * NP.value >= 256
    assert ws.value >= 64 * 128 * NP.value * (512 + 1) * 4


# --------------------------------------------------------------------------- plans

@pytest.mark.parametrize("B,h_q,h_kv,D,T,dt", [
    (1, 8, 2, 64, 256, F32), (8, 32, 32, 128, 4096, BF16), (32, 32, 8, 128, 4096, BF16),
    (16, 64, 8, 128, 32768, BF16), (3, 16, 16, 64, 777, F32),
])
def test_gqa_plan_consistency(lib, B, h_q, h_kv, D, T, dt):
    P, NP, ws = ctypes.c_int(), ctypes.c_int(), ctypes.c_size_t()
    assert lib.attn_decode_gqa_plan(B, h_q, h_kv, D, T, dt, ctypes.byref(P), ctypes.byref(NP),
                                    ctypes.byref(ws)) == OK
    assert P.value >= 1 and NP.value == -(-T // P.value)
    assert (NP.value - 1) * P.value < T <= NP.value * P.value
    rows = B * h_q * NP.value
    assert ws.value >= rows * D * 4 + rows * 4
    assert lib.attn_decode_gqa_workspace_bytes(B, h_q, h_kv, D, T, dt) == ws.value
    assert lib.attn_decode_gqa_workspace_bytes(B, h_q + 1, h_kv, D, T, dt) == 0


def test_full_size_plans_fill_the_chip(lib):
    for (B, hq, hkv, T) in [(8, 32, 32, 4096), (32, 32, 8, 4096), (16, 64, 8, 32768)]:
        P, NP = ctypes.c_int(), ctypes.c_int()
        assert lib.attn_decode_gqa_plan(B, hq, hkv, 128, T, BF16, ctypes.byref(P), ctypes.byref(NP),
                                        None) == OK
        assert B * hkv * NP.value >= 1024        # at least 2 partitions per resident work-group (512)


def test_step_and_append_argument_checks(lib):
    f = lib.attn_decode_gqa_step
    KN, VN = ctypes.c_void_p(1 << 46), ctypes.c_void_p(1 << 47)

    def step(**kw):
        a = dict(q=P16, kn=KN, vn=VN, k=P16b, v=P16c, lens=LENS, B=2, h_q=8, h_kv=2, D=128, T=1024,
                 scale=0.1, dt=BF16, out=OUT, ws=WS, wsb=1 << 30)
        a.update(kw)
        return f(a["q"], a["kn"], a["vn"], a["k"], a["v"], a["lens"], a["B"], a["h_q"], a["h_kv"],
                 a["D"], a["T"], a["scale"], a["dt"], a["out"], a["ws"], a["wsb"], None)

    assert step(kn=NULL) == INVALID
    assert step(vn=NULL) == INVALID
    assert step(kn=P16b) == INVALID                       # new rows inside the K cache
    assert step(vn=KN) == INVALID                         # k_new and v_new overlap
    assert step(kn=ctypes.c_void_p((1 << 46) + 8)) == UNSUPPORTED
    assert step(ws=P16b) == INVALID                       # workspace inside the K cache
    assert step(wsb=16) == WORKSPACE
    assert step(D=96) == UNSUPPORTED
    a = lib.attn_kv_append
    assert a(NULL, VN, P16b, P16c, LENS, 2, 2, 128, 1024, BF16, None) == INVALID
    assert a(KN, VN, P16b, P16b, LENS, 2, 2, 128, 1024, BF16, None) == INVALID   # K and V caches overlap
    assert a(KN, VN, P16b, P16c, LENS, 2, 2, 100, 1024, BF16, None) == UNSUPPORTED
    m = lib.attn_decode_mla_step
    LN = ctypes.c_void_p(1 << 46)
    assert m(P16, P16b, NULL, P16c, LENS, 4, 128, 512, 64, 4096, 0.07, OUT, WS, 1 << 30, None) == INVALID
    assert m(P16, P16b, P16c, P16c, LENS, 4, 128, 512, 64, 4096, 0.07, OUT, WS, 1 << 30, None) == INVALID
    la = lib.attn_latent_append
    assert la(NULL, P16c, LENS, 4, 512, 64, 4096, None) == INVALID
    assert la(LN, P16c, LENS, 4, 512, 60, 4096, None) == UNSUPPORTED          # row not whole 16-byte pieces
    assert la(P16c, P16c, LENS, 4, 512, 64, 4096, None) == INVALID            # new row inside the cache


def test_window_argument_checks(lib):
    f = lib.attn_decode_gqa_window
    base = [P16, P16b, P16c, LENS, 2, 8, 2, 128, 1024]
    assert f(*base, 0, 0.1, BF16, OUT, WS, 1 << 30, None) == INVALID        # window must be >= 1
    assert f(*base, -4, 0.1, BF16, OUT, WS, 1 << 30, None) == INVALID
    assert f(*base, 64, 0.1, BF16, OUT, WS, 16, None) == WORKSPACE
    need = lib.attn_decode_gqa_workspace_bytes(2, 8, 2, 128, 64, BF16)
    assert 0 < need < lib.attn_decode_gqa_workspace_bytes(2, 8, 2, 128, 1024, BF16)
    assert f(*base, 64, 0.1, BF16, OUT, WS, need - 1, None) == WORKSPACE


def test_paged_argument_checks(lib):
    f = lib.attn_decode_gqa_paged
    BT = ctypes.c_void_p(1 << 45)

    def call(**kw):
        a = dict(q=P16, k=P16b, v=P16c, bt=BT, lens=LENS, B=2, h_q=8, h_kv=2, D=128, num_pages=64,
                 ps=64, maxp=16, scale=0.1, dt=BF16, out=OUT, ws=WS, wsb=1 << 30)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["bt"], a["lens"], a["B"], a["h_q"], a["h_kv"], a["D"],
                 a["num_pages"], a["ps"], a["maxp"], a["scale"], a["dt"], a["out"], a["ws"], a["wsb"], None)

    assert call(bt=NULL) == INVALID
    assert call(ps=48) == UNSUPPORTED            # not a power of two
    assert call(ps=8) == UNSUPPORTED             # below the smallest page
    assert call(maxp=0) == INVALID
    assert call(num_pages=0) == INVALID
    assert call(bt=ctypes.c_void_p((1 << 45) + 2)) == UNSUPPORTED
    assert call(out=P16b) == INVALID             # output inside the K pages
    assert call(wsb=16) == WORKSPACE
    m = lib.attn_decode_mla_paged
    assert m(P16, P16b, P16c, BT, LENS, 4, 128, 512, 64, 64, 16, 16, 0.07, OUT, WS, 1 << 30, None) == UNSUPPORTED
    assert m(P16, P16b, P16c, NULL, LENS, 4, 128, 512, 64, 64, 64, 16, 0.07, OUT, WS, 1 << 30, None) == INVALID
    ap = lib.attn_kv_append_paged
    KN, VN = ctypes.c_void_p(1 << 46), ctypes.c_void_p(1 << 47)
    assert ap(KN, VN, P16b, P16c, NULL, LENS, 2, 2, 128, 64, 64, 16, BF16, None) == INVALID
    assert ap(KN, VN, P16b, P16b, BT, LENS, 2, 2, 128, 64, 64, 16, BF16, None) == INVALID
    la = lib.attn_latent_append_paged
    assert la(KN, P16c, BT, LENS, 4, 512, 60, 64, 64, 16, None) == UNSUPPORTED



def test_absorb_argument_checks(lib):
    a, u = lib.attn_mla_absorb_q, lib.attn_mla_up_v
    assert a(P16, P16b, OUT, 0, 128, 128, 512, None) == INVALID
    assert a(NULL, P16b, OUT, 64, 128, 128, 512, None) == INVALID
    assert a(P16, P16b, OUT, 64, 128, 120, 512, None) == UNSUPPORTED      # d_h not a multiple of 16
    assert a(P16, P16b, OUT, 64, 128, 128, 500, None) == UNSUPPORTED      # d_c not a multiple of 32
    assert a(P16, P16b, P16b, 64, 128, 128, 512, None) == INVALID         # output over the weights
    assert a(ctypes.c_void_p((1 << 20) + 2), P16b, OUT, 64, 128, 128, 512, None) == UNSUPPORTED
    assert u(P16, P16b, OUT, 64, 128, 512, 100, None) == UNSUPPORTED      # d_v not a multiple of 32
    assert u(P16, P16b, P16, 64, 128, 512, 128, None) == INVALID          # output over o_lat
