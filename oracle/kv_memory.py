"""KV-cache size arithmetic — test infrastructure (oracle side).

The "Inference optimization" lesson (KV cache section, memory formula; Build it,
Step 6: KV cache memory profiler) sizes the cache as two tensors (K and V) per
layer, per KV head, per head-dimension element, per token.  The "Serving engine
internals" lesson (PagedAttention section) prices a fixed per-request
reservation against the tokens a request actually uses.
"""

from __future__ import annotations


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, dtype_bytes: int = 2) -> int:
    """Bytes of K plus V for one token across all layers."""
    return 2 * num_layers * num_kv_heads * head_dim * dtype_bytes


def kv_bytes(num_layers: int, num_kv_heads: int, head_dim: int, seq_len: int, dtype_bytes: int = 2) -> int:
    """Bytes of K plus V for a sequence of `seq_len` tokens."""
    return kv_bytes_per_token(num_layers, num_kv_heads, head_dim, dtype_bytes) * seq_len


def reservation_waste(reserved_tokens: int, used_tokens: float) -> float:
    """Share of a contiguous per-request reservation that goes unused."""
    return 1.0 - float(used_tokens) / float(reserved_tokens)


def paged_waste(used_tokens: int, block_size: int) -> float:
    """Share of a request's paged allocation that goes unused: only the last
    block is partly empty, because blocks are taken as tokens arrive."""
    blocks = -(-int(used_tokens) // block_size)
    return 1.0 - used_tokens / float(blocks * block_size)
