"""Plain fp64 CPU oracle for single-token decode attention over a KV cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code, constant or helper with the HIP library under
``mla_kv_cache_amd/``; the two meet only through the seeded input
generators in ``workloads/``, which hold none of the method's arithmetic.

What it computes is the plain definition of the method, written out in
float64 on the exact input values (bf16 inputs are widened exactly):

* ``attention.decode_gqa`` -- one query token per head against a cache of
  ``h_kv`` shared K/V heads; MHA when ``h_kv == h_q``, MQA when ``h_kv == 1``.
* ``attention.decode_mla`` -- absorbed multi-head latent attention: every
  head scores against one cached latent plus a decoupled rotary key, and
  averages the latent itself.
* ``step.decode_gqa_step`` / ``step.decode_mla_step`` -- one decode step:
  the new token's K/V (or latent) row is written at ``seq_lens[b]``, then the
  token attends over the extended cache (``step.append_kv`` /
  ``step.append_latent`` are the writes alone).
* ``window.decode_gqa_window`` -- sliding-window decode: each row attends over
  its last ``window`` cached positions.
* ``paged.decode_gqa_paged`` / ``paged.decode_mla_paged`` -- decode over a
  paged cache whose block table maps logical pages to physical ones
  (``paged.append_kv_paged`` writes one new row into its page).
* ``absorb.absorb_q`` / ``absorb.up_v`` -- the MLA key up-projection absorbed
  into the query before the decode, and the value up-projection after it.
* ``cache.kv_cache_bytes`` / ``cache.mla_cache_bytes`` -- the cache-size
  arithmetic.
* ``brute`` -- pure-Python scalar loops for tiny shapes (a second,
  structurally different statement of the same definition).

Every function is pinned by tests that do not re-type its formula: the
pages' printed numbers, closed forms, invariants, a library routine
(PyTorch's scaled-dot-product attention on CPU in float64) and brute force.
No function here is "parity unpinned".
"""

from .attention import (  # noqa: F401
    decode_gqa,
    decode_mla,
    decode_gqa_weights,
    decode_gqa_lse,
    clamp_len,
)
from .step import append_kv, append_latent, decode_gqa_step, decode_mla_step  # noqa: F401
from .window import decode_gqa_window, window_start  # noqa: F401
from .paged import decode_gqa_paged, decode_mla_paged, append_kv_paged  # noqa: F401
from .absorb import absorb_q, up_v  # noqa: F401
from .cache import kv_cache_bytes, mla_cache_bytes  # noqa: F401
from . import brute  # noqa: F401
