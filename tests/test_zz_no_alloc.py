"""The allocation-free GQA entry point (attn_decode_gqa_noalloc), through the C ABI.

It runs attn_decode_gqa's plan and kernels with the library's static scratch
array as the workspace, so its output must equal attn_decode_gqa's bit for
bit. Two calls in a row, the second on a smaller input (the scratch keeps the
first call's contents, which must not leak into the second), and shapes of
both kernels (the work-balanced split and fixed partitions); a shape whose
workspace exceeds the scratch is rejected before any launch.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu


def _lib():
    from mla_kv_cache_amd import _lib
    return _lib.load()


def _call_noalloc(lib, q, k, v, lens, scale, out):
    B, h_q, D = q.shape
    _, h_kv, T, _ = k.shape
    dt = 1 if q.dtype == torch.bfloat16 else 0
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    return lib.attn_decode_gqa_noalloc(p(q), p(k), p(v), p(lens), B, h_q, h_kv, D, T, scale, dt, p(out),
                                       stream)


@pytest.mark.parametrize("first,second", [
    # (B, h_q, h_kv, D, T_max, dtype, seed)
    ((16, 64, 8, 128, 4096, torch.bfloat16, 41), (3, 64, 8, 128, 1000, torch.bfloat16, 42)),   # split, g = 8
    ((8, 32, 1, 128, 8192, torch.bfloat16, 43), (2, 32, 1, 128, 300, torch.bfloat16, 44)),     # MQA, matrix cores
    ((4, 16, 4, 64, 2048, torch.float32, 45), (1, 8, 2, 64, 256, torch.float32, 46)),         # fixed partitions
])
def test_noalloc_matches_attn_decode_gqa(gpu, first, second):
    import mla_kv_cache_amd as m
    lib = _lib()
    for (B, h_q, h_kv, D, T, dt, seed) in (first, second):
        w = W.small_gqa(B, h_q, h_kv, D, T, dtype=dt, seed=seed, lens=(0, T))
        q, k, v, lens = W.gqa_inputs(w)
        gq, gk, gv, gl = q.to(gpu), k.to(gpu), v.to(gpu), lens.to(gpu)
        ref = m.attn_decode_gqa(gq, gk, gv, gl, scale=w.scale)
        out = torch.full_like(gq, float("nan"))
        assert _call_noalloc(lib, gq, gk, gv, gl, w.scale, out) == 0
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (B, h_q, h_kv)
        expect = oracle.decode_gqa(q, k, v, lens, w.scale)
        tol = 1e-5 if dt == torch.float32 else 2e-3 + 2.0 ** (np.floor(np.log2(np.maximum(np.abs(expect), 2.0 ** -126))) - 8)
        assert np.all(np.abs(out.double().cpu().numpy() - expect) <= tol)


def test_noalloc_rejects_shapes_beyond_the_scratch(gpu):
    lib = _lib()
    # fp32 fixed partitions: B * h_q * NP * D * 4 bytes of partials, far above 32 MiB
    B, h_q, h_kv, D, T = 256, 128, 8, 128, 65536
    need = lib.attn_decode_gqa_workspace_bytes(B, h_q, h_kv, D, T, 0)
    assert need > 32 << 20
    fake = ctypes.c_void_p(1 << 40)     # never dereferenced: the check returns first
    st = lib.attn_decode_gqa_noalloc(fake, ctypes.c_void_p(1 << 41), ctypes.c_void_p(1 << 42),
                                     ctypes.c_void_p(1 << 43), B, h_q, h_kv, D, T, 0.1, 0,
                                     ctypes.c_void_p(1 << 44), None)
    assert st == -3
