"""KV-cache size arithmetic, exact integers.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Sources (page title -- section):

* "Attention variants: MQA, GQA, and MLA" -- "The KV cache bill, worked
  numerically": a layer stores a key tensor and a value tensor, each with one
  head_dim-wide vector per (sequence, KV head, cached token); the byte count is
  the product of the factor 2 (keys and values), layers, KV heads, head_dim,
  tokens, sequences and bytes per value. The page's helper takes its
  arguments in the order (n_layers, n_kv_heads, head_dim, seq_len, batch,
  bytes_per_elem) with batch and bytes_per_elem defaulting to 1 and 2.
* Same page -- "MLA: cache a latent, not the keys and values": per token per
  layer MLA caches d_c latent values plus a d_r rotary key, nothing else;
  "KV cache variants: MHA, GQA, MLA" -- "MLA (DeepSeek-V2 style)" counts the
  same row (there without a rotary part) at 2 bytes per value.
* "Grouped-Query Attention: Fewer KV Heads, Same Quality" -- "Counting every
  parameter and byte": the same count written as L * h * (d_k + d_v) * 2.
"""


def kv_cache_bytes(n_layers: int, n_kv_heads: int, head_dim: int, seq_len: int,
                   batch: int = 1, bytes_per_elem: int = 2) -> int:
    """Bytes of the key and value caches of a whole model (every layer, every sequence)."""
    per_tensor = int(batch) * int(n_kv_heads) * int(seq_len) * int(head_dim)
    return int(n_layers) * 2 * per_tensor * int(bytes_per_elem)


def mla_cache_bytes(n_layers: int, d_c: int, d_r: int, seq_len: int,
                    batch: int = 1, bytes_per_elem: int = 2) -> int:
    """Bytes of an MLA cache: one (d_c + d_r)-wide row per token per layer per sequence."""
    return int(n_layers) * int(batch) * int(seq_len) * (int(d_c) + int(d_r)) * int(bytes_per_elem)
