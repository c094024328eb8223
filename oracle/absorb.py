"""fp64 definition of the MLA absorption products on either side of the decode.

TEST INFRASTRUCTURE ONLY -- see the package docstring. The product path never
imports this module.

Source (page title -- section): "Attention variants: MQA, GQA, and MLA" --
"MLA: cache a latent, not the keys and values" (decode sketch). The key
up-projection W_UK [H, d_c, d_h] is absorbed into the query: per head h,
q_lat[b, h, c] = sum_d q[b, h, d] * W_UK[h, c, d]; the scores then run against
the latent. The value up-projection W_UV [H, d_c, d_v] is applied after the
average: o[b, h, d] = sum_c o_lat[b, h, c] * W_UV[h, c, d]. Both are plain
per-head matrix products, written out here one head at a time.
"""

from __future__ import annotations

import numpy as np

from .attention import _f64


def absorb_q(q, w_uk) -> np.ndarray:
    """q [B, H, d_h], W_UK [H, d_c, d_h] -> q_lat float64 [B, H, d_c]."""
    B, H, d_h = q.shape
    Hw, d_c, d_hw = w_uk.shape
    if Hw != H or d_hw != d_h:
        raise ValueError("q and W_UK disagree on H or d_h")
    out = np.zeros((B, H, d_c), dtype=np.float64)
    for h in range(H):
        out[:, h] = _f64(q[:, h]) @ _f64(w_uk[h]).T          # [B, d_h] @ [d_h, d_c]
    return out


def up_v(o_lat, w_uv) -> np.ndarray:
    """o_lat [B, H, d_c], W_UV [H, d_c, d_v] -> o float64 [B, H, d_v]."""
    B, H, d_c = o_lat.shape
    Hw, d_cw, d_v = w_uv.shape
    if Hw != H or d_cw != d_c:
        raise ValueError("o_lat and W_UV disagree on H or d_c")
    out = np.zeros((B, H, d_v), dtype=np.float64)
    for h in range(H):
        out[:, h] = _f64(o_lat[:, h]) @ _f64(w_uv[h])         # [B, d_c] @ [d_c, d_v]
    return out
