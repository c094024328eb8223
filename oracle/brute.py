"""Pure-Python scalar statement of decode attention, for tiny shapes only.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

A second, structurally different statement of the same definition as
``attention.decode_gqa``: no numpy, no matrix products, Python floats
(IEEE double) with ``math.fsum`` for every sum and the 1-indexed group map
of "Attention variants: MQA, GQA, and MLA" -- "GQA: interpolating with
groups" (query head i uses KV head ceil(i * h_kv / h_q)). The softmax is
written from its textbook form: exp of each score minus the maximum,
divided by the sum of those exps.
"""

import math


def _as_lists(x):
    """Nested lists of Python floats from a numpy array or CPU torch tensor."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).tolist()
    except Exception:  # pragma: no cover
        pass
    return x.tolist() if hasattr(x, "tolist") else x


def kv_head_of(i_one_based: int, h_q: int, h_kv: int) -> int:
    """1-indexed KV head of 1-indexed query head i: ceil(i * h_kv / h_q), in integers."""
    return -((-i_one_based * h_kv) // h_q)


def brute_gqa(q, k_cache, v_cache, seq_lens, scale):
    """Returns nested lists out[b][i][d] (floats)."""
    q, k, v = _as_lists(q), _as_lists(k_cache), _as_lists(v_cache)
    lens = [int(x) for x in _as_lists(seq_lens)]
    B, h_q, h_kv = len(q), len(q[0]), len(k[0])
    T_max, Dv = len(k[0][0]), len(v[0][0][0])
    out = []
    for b in range(B):
        n = min(max(lens[b], 0), T_max)
        rows = []
        for i1 in range(1, h_q + 1):
            j = kv_head_of(i1, h_q, h_kv) - 1
            qi = q[b][i1 - 1]
            if n == 0:
                rows.append([0.0] * Dv)
                continue
            scores = [scale * math.fsum(a * c for a, c in zip(qi, k[b][j][t])) for t in range(n)]
            top = max(scores)
            e = [math.exp(s - top) for s in scores]
            z = math.fsum(e)
            w = [x / z for x in e]
            rows.append([math.fsum(w[t] * v[b][j][t][d] for t in range(n)) for d in range(Dv)])
        out.append(rows)
    return out


def brute_mla(q_nope, q_rope, latent, seq_lens, scale, d_c):
    """Returns nested lists out[b][h][c] (floats) for absorbed MLA."""
    qn, qr, lat = _as_lists(q_nope), _as_lists(q_rope), _as_lists(latent)
    lens = [int(x) for x in _as_lists(seq_lens)]
    B, H, T_max = len(qn), len(qn[0]), len(lat[0])
    out = []
    for b in range(B):
        n = min(max(lens[b], 0), T_max)
        rows = []
        for h in range(H):
            if n == 0:
                rows.append([0.0] * d_c)
                continue
            scores = []
            for t in range(n):
                r = lat[b][t]
                dot_c = math.fsum(x * y for x, y in zip(qn[b][h], r[:d_c]))
                dot_r = math.fsum(x * y for x, y in zip(qr[b][h], r[d_c:]))
                scores.append(scale * (dot_c + dot_r))
            top = max(scores)
            e = [math.exp(s - top) for s in scores]
            z = math.fsum(e)
            rows.append([math.fsum(e[t] / z * lat[b][t][c] for t in range(n)) for c in range(d_c)])
        out.append(rows)
    return out
