"""Closed-form KV-cache sizes the pages reason with.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* A decoder-only Transformer keeps keys and values for every layer and every
  token: N x L entries ([S §2]; [P seg. 4]).
* YOCO keeps one global cache of N entries plus a constant-size cache per
  self-decoder layer (a sliding window of C tokens), i.e. O(N + C L)
  ([S §2]; [P seg. 8], [P seg. 12]).
* The per-token saving therefore tends to the layer count ([P seg. 22]).

Sizes are in bytes; kv_width = n_kv_heads * head_dim; both K and V counted.
"""

__all__ = ["transformer_kv_cache_bytes", "yoco_kv_cache_bytes"]


def transformer_kv_cache_bytes(n_tokens, n_layers, kv_width, bytes_per_elem):
    """Every layer caches K and V for every token."""
    return 2 * n_tokens * n_layers * kv_width * bytes_per_elem


def yoco_kv_cache_bytes(n_tokens, n_layers, kv_width, bytes_per_elem, window):
    """One global K/V for all tokens + a window-sized cache per self-decoder layer."""
    n_self = n_layers // 2
    global_cache = 2 * n_tokens * kv_width * bytes_per_elem
    self_caches = n_self * 2 * min(window, n_tokens) * kv_width * bytes_per_elem
    return global_cache + self_caches
