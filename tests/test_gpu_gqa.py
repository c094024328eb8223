"""GPU parity of the GQA/MHA/MQA decode path against the fp64 oracle.

Every case goes through the C ABI (via the ctypes binding) on seeded inputs
from ``workloads``; the oracle sees the very same values, widened to fp64.

Tolerances (max-abs, from the stated target of the method: fp32 accumulation
over bf16 storage within 2e-3, fp32 storage within 1e-5):
* fp32-output comparisons (merge written in fp32): 2e-3 for bf16 inputs,
  1e-5 for fp32 inputs -- the kernel's own arithmetic only;
* bf16-output comparisons: 2e-3 plus half a bf16 ulp of the oracle value,
  the unavoidable rounding of the result to bf16 (for the full-size
  workloads |out| < 0.25, so the bound stays below 2.5e-3);
* bit-exact: one cached position returns its value, NaN in padding changes
  nothing, repeated runs are identical.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu


def _m():
    import mla_kv_cache_amd as m
    return m


def _half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    a = np.abs(x)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 8)


def _f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _inputs(w, dev, seq_lens=None):
    q, k, v, lens = W.gqa_inputs(w, device="cpu", seq_lens=seq_lens)
    return (q, k, v, lens), (q.to(dev), k.to(dev), v.to(dev), lens.to(dev))


def _run_fp32_out(m, gq, gk, gv, gl, P, scale):
    po, pl = m.attn_decode_gqa_partial(gq, gk, gv, gl, P, scale=scale)
    return m.attn_decode_merge(po, pl, gl, gk.shape[2], P, out_dtype=torch.float32)


CASES = [
    # (B, h_q, h_kv, D, T_max, dtype, lens)
    (3, 8, 2, 128, 1000, torch.bfloat16, [1000, 517, 1]),
    (2, 32, 32, 128, 700, torch.bfloat16, [700, 333]),
    (2, 16, 1, 128, 900, torch.bfloat16, [899, 64]),
    (2, 16, 2, 128, 1500, torch.bfloat16, [1500, 1033]),
    (1, 32, 2, 128, 640, torch.bfloat16, [640]),
    (2, 8, 4, 64, 1200, torch.bfloat16, [1200, 10]),
    (2, 8, 8, 64, 300, torch.float32, [300, 257]),
    (1, 8, 2, 64, 256, torch.float32, [256]),
    (2, 16, 4, 128, 513, torch.float32, [513, 200]),
    (2, 16, 2, 64, 777, torch.float32, [777, 31]),
    # MQA and groups of 16 to 128 query heads per KV head (matrix-core kernel for bf16,
    # chunks of 16 heads for fp32)
    (2, 32, 1, 128, 1000, torch.bfloat16, [1000, 517]),
    (3, 64, 1, 128, 700, torch.bfloat16, [700, 1, 333]),
    (2, 128, 1, 128, 600, torch.bfloat16, [600, 45]),
    (2, 64, 2, 64, 900, torch.bfloat16, [900, 130]),
    (2, 128, 2, 64, 400, torch.bfloat16, [257, 400]),
    (2, 32, 2, 128, 800, torch.bfloat16, [800, 799]),
    (2, 32, 1, 64, 500, torch.float32, [500, 77]),
    (1, 128, 1, 128, 300, torch.float32, [300]),
    # groups that are not powers of two (3, 5, 6, 7: the 16 x 16 kernel's masked head
    # columns for bf16, the generic kernel for fp32)
    (2, 12, 4, 128, 900, torch.bfloat16, [900, 333]),
    (2, 10, 2, 64, 500, torch.bfloat16, [500, 129]),
    (3, 28, 4, 128, 700, torch.bfloat16, [700, 1, 64]),
    (2, 12, 2, 128, 600, torch.float32, [600, 77]),
    (2, 21, 3, 64, 300, torch.float32, [300, 10]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}_hq{c[1]}_hkv{c[2]}_D{c[3]}_T{c[4]}_{str(c[5])[6:]}")
@pytest.mark.parametrize("P", [0, 64, 100, 4096])
def test_gqa_matches_oracle(gpu, case, P):
    m = _m()
    B, h_q, h_kv, D, T, dt, lens = case
    w = W.small_gqa(B, h_q, h_kv, D, T, dtype=dt, seed=11)
    (q, k, v, l), (gq, gk, gv, gl) = _inputs(w, gpu, lens)
    ref = oracle.decode_gqa(q, k, v, l, w.scale)
    tol = 1e-5 if dt == torch.float32 else 2e-3
    if P == 0:
        out = m.attn_decode_gqa(gq, gk, gv, gl, scale=w.scale)
        got = _f64(out)
        bound = tol + (_half_ulp_bf16(ref) if dt == torch.bfloat16 else 0.0)
        assert np.all(np.abs(got - ref) <= bound), float(np.abs(got - ref).max())
        if dt == torch.bfloat16:  # the fp32 result rounded once to bf16
            assert np.all(np.abs(got - ref) <= _half_ulp_bf16(ref) + 1e-5), float(np.abs(got - ref).max())
    else:
        got = _f64(_run_fp32_out(m, gq, gk, gv, gl, P, w.scale))
        err = float(np.abs(got - ref).max())
        assert err <= tol, err


def test_tiny_fp32_workload(gpu):
    """The tiny fp32 workload (B=1, h_q=8, h_kv=2, D=64, T=256), end to end."""
    m = _m()
    w = W.TINY_GQA
    (q, k, v, l), (gq, gk, gv, gl) = _inputs(w, gpu)
    out = m.attn_decode_gqa(gq, gk, gv, gl, scale=w.scale)
    ref = oracle.decode_gqa(q, k, v, l, w.scale)
    assert out.dtype == torch.float32 and out.shape == (1, 8, 64)
    assert float(np.abs(_f64(out) - ref).max()) <= 1e-5


@pytest.mark.parametrize("h_q,h_kv,D", [(16, 4, 128), (32, 1, 128), (128, 1, 128), (64, 2, 64), (32, 2, 128),
                                         (12, 4, 128), (28, 4, 64)])
def test_single_position_is_bit_exact(gpu, h_q, h_kv, D):
    m = _m()
    g = h_q // h_kv
    for dt in (torch.bfloat16, torch.float32):
        w = W.small_gqa(3, h_q, h_kv, D, 300, dtype=dt, seed=5)
        (q, k, v, l), (gq, gk, gv, gl) = _inputs(w, gpu, [1, 1, 1])
        out = m.attn_decode_gqa(gq, gk, gv, gl)
        expect = gv[:, :, 0].repeat_interleave(g, dim=1)
        assert torch.equal(out, expect)


def test_zero_and_clamped_lengths(gpu):
    m = _m()
    w = W.small_gqa(4, 8, 2, 128, 200, seed=6)
    (q, k, v, l), (gq, gk, gv, gl) = _inputs(w, gpu, [0, 500, -7, 200])
    out = m.attn_decode_gqa(gq, gk, gv, gl)
    assert torch.equal(out[0], torch.zeros_like(out[0]))
    assert torch.equal(out[2], torch.zeros_like(out[2]))
    same = m.attn_decode_gqa(gq, gk, gv, torch.tensor([0, 200, 0, 200], dtype=torch.int32, device=gpu))
    assert torch.equal(out[1], same[1])                      # 500 is clamped to T_max = 200
    ref = oracle.decode_gqa(q, k, v, l, w.scale)
    bound = 2e-3 + _half_ulp_bf16(ref)
    assert np.all(np.abs(_f64(out) - ref) <= bound)


@pytest.mark.parametrize("h_q,h_kv", [(16, 2), (64, 1)])
def test_nan_padding_is_never_read(gpu, h_q, h_kv):
    m = _m()
    w = W.small_gqa(2, h_q, h_kv, 128, 1024, seed=7)
    (q, k, v, l), (gq, gk, gv, gl) = _inputs(w, gpu, [700, 129])
    base = m.attn_decode_gqa(gq, gk, gv, gl)
    gk2, gv2 = gk.clone(), gv.clone()
    gk2[0, :, 700:] = float("nan")
    gv2[0, :, 700:] = float("nan")
    gk2[1, :, 129:] = float("inf")
    gv2[1, :, 129:] = float("nan")
    out = m.attn_decode_gqa(gq, gk2, gv2, gl)
    assert torch.equal(out, base)
    assert torch.isfinite(out).all()


def test_deterministic(gpu):
    m = _m()
    w = W.small_gqa(4, 32, 8, 128, 4096, seed=8, lens=(1, 4096))
    _, (gq, gk, gv, gl) = _inputs(w, gpu)
    a = m.attn_decode_gqa(gq, gk, gv, gl)
    b = m.attn_decode_gqa(gq, gk, gv, gl)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_partition_size_does_not_change_the_result(gpu):
    """Split-KV regrouping: one partition vs many agree within fp32 rounding."""
    m = _m()
    w = W.small_gqa(2, 32, 8, 128, 3000, seed=9)
    (q, k, v, l), (gq, gk, gv, gl) = _inputs(w, gpu, [3000, 1777])
    one = _f64(_run_fp32_out(m, gq, gk, gv, gl, 3000, w.scale))
    many = _f64(_run_fp32_out(m, gq, gk, gv, gl, 128, w.scale))
    assert float(np.abs(one - many).max()) <= 1e-5


def test_runs_on_a_side_stream(gpu):
    m = _m()
    w = W.small_gqa(2, 8, 2, 128, 512, seed=10)
    (q, k, v, l), (gq, gk, gv, gl) = _inputs(w, gpu)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = m.attn_decode_gqa(gq, gk, gv, gl)
    s.synchronize()
    ref = oracle.decode_gqa(q, k, v, l, w.scale)
    assert np.all(np.abs(_f64(out) - ref) <= 2e-3 + _half_ulp_bf16(ref))


def test_partials_match_oracle_per_partition(gpu):
    """Stage 1 alone: each partition's output is the softmax average over its own positions."""
    m = _m()
    w = W.small_gqa(1, 8, 2, 128, 600, seed=12)
    (q, k, v, l), (gq, gk, gv, gl) = _inputs(w, gpu, [600])
    P = 256
    po, pl = m.attn_decode_gqa_partial(gq, gk, gv, gl, P, scale=w.scale)
    po, pl = _f64(po), _f64(pl)
    for p in range(3):
        lo, hi = p * P, min(p * P + P, 600)
        ref = oracle.decode_gqa(q, k[:, :, lo:hi], v[:, :, lo:hi], [hi - lo], w.scale)
        assert float(np.abs(po[:, :, p] - ref).max()) <= 2e-3
        lse2 = oracle.decode_gqa_lse(q, k[:, :, lo:hi], [hi - lo], w.scale) / math.log(2)
        assert float(np.abs(pl[:, :, p] - lse2).max()) <= 1e-4


# --------------------------------------------------------------------------- full-size workloads

def _full_parity(w):
    """Every output row of a full-size workload against the oracle, in the
    benchmark's launch configuration (one sequence of the oracle at a time)."""
    m = _m()
    dev = torch.device("cuda:0")
    (q, k, v, l), (gq, gk, gv, gl) = _inputs(w, dev)
    out = m.attn_decode_gqa(gq, gk, gv, gl, scale=w.scale)
    got = _f64(out)
    del gq, gk, gv
    assert np.isfinite(got).all()
    worst = excess = 0.0
    for b in range(w.B):
        ref = oracle.decode_gqa(q[b:b + 1], k[b:b + 1], v[b:b + 1], l[b:b + 1], w.scale)[0]
        err = np.abs(got[b] - ref)
        worst = max(worst, float(err.max()))
        excess = max(excess, float((err - _half_ulp_bf16(ref)).max()))
        assert np.all(err <= 2e-3 + _half_ulp_bf16(ref)), (b, float(err.max()))
        # the fp32-accumulated result rounded once to bf16: half a bf16 ulp plus 1e-5
        assert np.all(err <= _half_ulp_bf16(ref) + 1e-5), (b, float((err - _half_ulp_bf16(ref)).max()))
    return worst, excess


@pytest.mark.parametrize("name", ["mha7b", "gqa4", "gqa8", "mqa"])
def test_full_size_workload_every_row(gpu, name):
    worst, excess = _full_parity(W.NAMED[name])
    print(f"{name}: worst max-abs error over all rows {worst:.3e}; beyond the bf16 rounding {excess:.3e}")


@pytest.mark.parametrize("B,h_q,h_kv,D", [(150, 8, 2, 64), (100, 64, 8, 128), (70, 16, 16, 128)])
def test_persistent_split_many_sequences(gpu, B, h_q, h_kv, D):
    """The bf16 kernel splits the non-empty (sequence, KV head, partition) items
    evenly over its resident work-groups, scanning the lengths 64 sequences at
    a time. More than 64 sequences, empty, one-position and full rows mixed
    in: every row gets exactly its own partitions, for planned and explicit
    partition sizes (including ones that do not divide the tile)."""
    m = _m()
    g = torch.Generator().manual_seed(21 + B)
    T = 300
    lens = torch.randint(0, T + 1, (B,), generator=g, dtype=torch.int32)
    lens[::7] = 0
    lens[3::11] = 1
    lens[5::13] = T
    w = W.small_gqa(B, h_q, h_kv, D, T, seed=22 + B)
    (q, k, v, l), (gq, gk, gv, gl) = _inputs(w, gpu, lens)
    ref = oracle.decode_gqa(q, k, v, l, w.scale)
    out = m.attn_decode_gqa(gq, gk, gv, gl, scale=w.scale)
    assert np.all(np.abs(_f64(out) - ref) <= 2e-3 + _half_ulp_bf16(ref))
    for P in (32, 100, 512):
        got = _f64(_run_fp32_out(m, gq, gk, gv, gl, P, w.scale))
        assert float(np.abs(got - ref).max()) <= 2e-3, P
    empty = (lens == 0).nonzero().flatten().tolist()
    assert torch.equal(out[empty], torch.zeros_like(out[empty]))


@pytest.mark.parametrize("B,h_q,h_kv,D,T,seed", [
    (3, 32, 8, 128, 1000, 31),     # a few pairs over many work-groups
    (1, 8, 8, 64, 40, 32),         # fewer units than work-groups: runs left empty
    (40, 64, 8, 128, 2000, 33),    # ragged, pairs cut between work-groups
    (2, 8, 1, 128, 700, 34),       # MQA
    (5, 16, 8, 64, 130, 35),       # units of one and two tiles' worth
    (9, 32, 1, 128, 1500, 37),     # MQA on the matrix cores
    (6, 128, 2, 64, 600, 38),      # groups of 64
])
def test_split_stages_match_one_call(gpu, B, h_q, h_kv, D, T, seed):
    """The work-balanced split: its two stages called one after the other give
    the bits of the one-call entry point, which matches the oracle, for shapes
    where the units are fewer than the work-groups (empty runs are skipped by
    the merge) and where rows are cut between work-groups."""
    m = _m()
    g = torch.Generator().manual_seed(seed)
    lens = torch.randint(0, T + 1, (B,), generator=g, dtype=torch.int32)
    lens[0] = T
    if B > 2:
        lens[1] = 0
    w = W.small_gqa(B, h_q, h_kv, D, T, seed=seed)
    (q, k, v, l), (gq, gk, gv, gl) = _inputs(w, gpu, lens)
    ws = torch.empty(m.attn_decode_gqa_workspace_bytes(B, h_q, h_kv, D, T), dtype=torch.uint8, device=gpu)
    full = m.attn_decode_gqa(gq, gk, gv, gl, scale=w.scale)
    m.attn_decode_gqa_split(gq, gk, gv, gl, ws, scale=w.scale)
    got = m.attn_decode_gqa_split_merge(gq, gk, gv, gl, ws, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(got, full)
    ref = oracle.decode_gqa(q, k, v, l, w.scale)
    assert np.all(np.abs(_f64(full) - ref) <= 2e-3 + _half_ulp_bf16(ref))
    zero = (lens == 0).nonzero().flatten().tolist()
    assert torch.equal(full[zero], torch.zeros_like(full[zero]))


def test_split_stages_reject_unsplit_shapes(gpu):
    """fp32 caches run on fixed partitions: the stage entry points say so."""
    m = _m()
    for dt, h_q, h_kv in ((torch.float32, 8, 2), (torch.float32, 32, 1)):
        w = W.small_gqa(2, h_q, h_kv, 128, 64, dtype=dt, seed=36)
        _, (gq, gk, gv, gl) = _inputs(w, gpu)
        ws = torch.empty(1 << 20, dtype=torch.uint8, device=gpu)
        with pytest.raises(m.AttnError):
            m.attn_decode_gqa_split(gq, gk, gv, gl, ws)
        with pytest.raises(m.AttnError):
            m.attn_decode_gqa_split_merge(gq, gk, gv, gl, ws)
