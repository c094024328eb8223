"""Seeded synthetic workloads: shapes and input generators, nothing else.

This module is shared by the tests, ``bench.py`` and the smoke check. It holds
no part of the attention arithmetic: it only names the workload shapes and
draws their inputs from a seeded CPU ``torch.Generator``, so that the HIP
library and the fp64 oracle see the very same values.

Recipe (also stated in the design doc):

* ``torch.Generator('cpu').manual_seed(seed)``, seed 0 for the named workloads
  (the pages seed their own examples with 0).
* Draw order: ``seq_lens`` (only when ragged), then the query (MLA: the
  absorbed part, then the rotary part), then K, then V (MLA: the latent rows).
* Every floating tensor is drawn N(0, 1) in float32, one batch element at a
  time (b = 0 .. B-1), then rounded to the storage dtype (bf16 by
  round-to-nearest-even, or kept fp32). Padding positions t >= seq_len are
  drawn like the rest.
* Ragged lengths are ``torch.randint(lo, hi + 1, (B,))`` in int32, both ends
  inclusive.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Tuple

import torch


@dataclass(frozen=True)
class GQAWorkload:
    name: str
    B: int
    h_q: int
    h_kv: int
    D: int
    T_max: int
    dtype: torch.dtype
    lens: Optional[Tuple[int, int]] = None   # (lo, hi) inclusive for ragged batches; None = all T_max
    seed: int = 0

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


@dataclass(frozen=True)
class MLAWorkload:
    name: str
    B: int
    H: int
    d_c: int
    d_r: int
    T_max: int
    head_dim_for_scale: int = 192          # 128 un-absorbed head dims + 64 rotary dims
    lens: Optional[Tuple[int, int]] = None
    dtype: torch.dtype = torch.bfloat16
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim_for_scale)


# The five named workloads.
TINY_GQA = GQAWorkload("tiny GQA g=4 fp32 (B=1, h_q=8, h_kv=2, D=64, T=256)",
                       B=1, h_q=8, h_kv=2, D=64, T_max=256, dtype=torch.float32)
MHA_7B = GQAWorkload("MHA Llama-2-7B layer (B=8, h=32, D=128, T=4096, bf16)",
                     B=8, h_q=32, h_kv=32, D=128, T_max=4096, dtype=torch.bfloat16)
GQA4_8B = GQAWorkload("GQA g=4 8B layer (B=32, h_q=32, h_kv=8, D=128, T=4096, bf16)",
                      B=32, h_q=32, h_kv=8, D=128, T_max=4096, dtype=torch.bfloat16)
GQA8_70B = GQAWorkload("GQA g=8 70B layer ragged (B=16, h_q=64, h_kv=8, D=128, "
                       "seq_lens~U[1024,32768], T_max=32768, bf16)",
                       B=16, h_q=64, h_kv=8, D=128, T_max=32768, dtype=torch.bfloat16,
                       lens=(1024, 32768))
MQA_7B = GQAWorkload("MQA 7B-shaped layer (B=32, h_q=32, h_kv=1, D=128, T=32768, bf16)",
                     B=32, h_q=32, h_kv=1, D=128, T_max=32768, dtype=torch.bfloat16)
MLA_V2 = MLAWorkload("MLA absorbed DeepSeek-V2 layer (B=64, H=128, d_c=512, d_r=64, T=4096, bf16)",
                     B=64, H=128, d_c=512, d_r=64, T_max=4096)

NAMED = {"tiny": TINY_GQA, "mha7b": MHA_7B, "gqa4": GQA4_8B, "gqa8": GQA8_70B, "mla": MLA_V2,
         "mqa": MQA_7B}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator("cpu")
    g.manual_seed(int(seed))
    return g


def _draw_lens(g, B, T_max, lens):
    if lens is None:
        return torch.full((B,), T_max, dtype=torch.int32)
    lo, hi = lens
    return torch.randint(int(lo), int(hi) + 1, (B,), generator=g, dtype=torch.int32)


def _fill(dst: torch.Tensor, g: torch.Generator) -> None:
    """Fill dst one batch element at a time with N(0,1) fp32 draws rounded to dst.dtype."""
    for b in range(dst.shape[0]):
        chunk = torch.randn(tuple(dst.shape[1:]), generator=g, dtype=torch.float32)
        dst[b].copy_(chunk.to(dst.dtype))


def gqa_inputs(w: GQAWorkload, device="cpu", seq_lens=None):
    """Draw (q, k_cache, v_cache, seq_lens) for a GQA workload.

    ``seq_lens`` may be given explicitly (a list or int32 tensor); it is then
    not drawn, and the draw order starts with q.
    """
    g = _gen(w.seed)
    if seq_lens is None:
        lens = _draw_lens(g, w.B, w.T_max, w.lens)
    else:
        lens = torch.as_tensor(seq_lens, dtype=torch.int32).reshape(w.B).clone()
    q = torch.empty((w.B, w.h_q, w.D), dtype=w.dtype, device=device)
    k = torch.empty((w.B, w.h_kv, w.T_max, w.D), dtype=w.dtype, device=device)
    v = torch.empty((w.B, w.h_kv, w.T_max, w.D), dtype=w.dtype, device=device)
    _fill(q, g)
    _fill(k, g)
    _fill(v, g)
    return q, k, v, lens.to(device)


def mla_inputs(w: MLAWorkload, device="cpu", seq_lens=None):
    """Draw (q_nope, q_rope, latent, seq_lens) for an MLA workload."""
    g = _gen(w.seed)
    if seq_lens is None:
        lens = _draw_lens(g, w.B, w.T_max, w.lens)
    else:
        lens = torch.as_tensor(seq_lens, dtype=torch.int32).reshape(w.B).clone()
    qn = torch.empty((w.B, w.H, w.d_c), dtype=w.dtype, device=device)
    qr = torch.empty((w.B, w.H, w.d_r), dtype=w.dtype, device=device)
    lat = torch.empty((w.B, w.T_max, w.d_c + w.d_r), dtype=w.dtype, device=device)
    _fill(qn, g)
    _fill(qr, g)
    _fill(lat, g)
    return qn, qr, lat, lens.to(device)


def small_gqa(B, h_q, h_kv, D, T_max, dtype=torch.bfloat16, lens=None, seed=0, name="case"):
    """A GQA workload descriptor for parity cases of arbitrary shape."""
    return GQAWorkload(name, B=B, h_q=h_q, h_kv=h_kv, D=D, T_max=T_max, dtype=dtype,
                       lens=lens, seed=seed)


def small_mla(B, H, T_max, d_c=512, d_r=64, lens=None, seed=0, name="case"):
    return MLAWorkload(name, B=B, H=H, d_c=d_c, d_r=d_r, T_max=T_max, lens=lens, seed=seed)
