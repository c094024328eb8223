"""KV-cache size arithmetic, exact integers.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Sources (page title -- section):

* "Attention variants: MQA, GQA, and MLA" -- "The KV cache bill, worked
  numerically": per layer the cache holds K and V, each of shape
  (batch, kv_heads, seq, head_dim); bytes = 2 * layers * kv_heads * head_dim
  * seq * bytes_per_element * batch. The page's Python helper takes
  (n_layers, n_kv_heads, head_dim, seq_len, batch=1, bytes_per_elem=2).
* Same page -- "MLA: cache a latent, not the keys and values": per token per
  layer MLA caches d_c latent values plus a d_r rotary key, nothing else.
* "Grouped-Query Attention: Fewer KV Heads, Same Quality" -- "Counting every
  parameter and byte": the same count written as L * h * (d_k + d_v) * 2.
"""


def kv_cache_bytes(n_layers: int, n_kv_heads: int, head_dim: int, seq_len: int,
                   batch: int = 1, bytes_per_elem: int = 2) -> int:
    """Bytes of K plus V for a whole model: K and V are each [batch, kv_heads, seq, head_dim] per layer."""
    per_tensor = int(batch) * int(n_kv_heads) * int(seq_len) * int(head_dim)
    return int(n_layers) * 2 * per_tensor * int(bytes_per_elem)


def mla_cache_bytes(n_layers: int, d_c: int, d_r: int, seq_len: int,
                    batch: int = 1, bytes_per_elem: int = 2) -> int:
    """Bytes of an MLA cache: one (d_c + d_r)-wide row per token per layer per sequence."""
    return int(n_layers) * int(batch) * int(seq_len) * (int(d_c) + int(d_r)) * int(bytes_per_elem)
