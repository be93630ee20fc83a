"""Closed forms for paged KV memory (oracle; test infrastructure only).

Sources:
* "Tech Radar: vLLM v1 Production Engine Architecture & Distributed KV Cache
  Optimization", section "Mathematical Modeling of PagedAttention v3 Memory
  Bounds": blocks per sequence are the ceiling of length over block size; the
  bytes of one block are 2 * layers * KV heads * head dim * block size *
  element bytes; internal fragmentation is the unused slots of the last block
  over the allocated slots, bounded by block size over length.
* "High-Throughput Local LLM Infrastructure ...", section "7.2 GPU VRAM
  Sizing Formulas": KV bytes per sequence (2 * layers * KV heads * head dim
  * context * element bytes) and the concurrency bound floor((VRAM - weights)
  / per-sequence KV).
"""

from fractions import Fraction


def num_blocks(seq_len: int, block_size: int) -> int:
    """Blocks a sequence of ``seq_len`` tokens occupies: ceil(S / B)."""
    if seq_len < 0 or block_size <= 0:
        raise ValueError("seq_len >= 0 and block_size > 0 required")
    return -(-seq_len // block_size)


def block_bytes(layers: int, kv_heads: int, head_dim: int, block_size: int,
                elem_bytes: int) -> int:
    """Bytes of one physical block holding K and V for every layer."""
    return 2 * layers * kv_heads * head_dim * block_size * elem_bytes


def paged_bytes(seq_len: int, layers: int, kv_heads: int, head_dim: int,
                block_size: int, elem_bytes: int) -> int:
    """Bytes a sequence holds under paging: its blocks times block bytes."""
    return num_blocks(seq_len, block_size) * block_bytes(
        layers, kv_heads, head_dim, block_size, elem_bytes)


def kv_bytes(seq_len: int, layers: int, kv_heads: int, head_dim: int,
             elem_bytes: int) -> int:
    """Token-exact KV bytes of one sequence: 2 * L * H_kv * D * S * bytes."""
    return 2 * layers * kv_heads * head_dim * seq_len * elem_bytes


def internal_fragmentation(seq_len: int, block_size: int) -> Fraction:
    """Unused slots of the terminal block over all allocated slots (exact)."""
    nb = num_blocks(seq_len, block_size)
    if nb == 0:
        return Fraction(0)
    unused = (block_size - seq_len % block_size) % block_size
    return Fraction(unused, nb * block_size)


def max_concurrency(total_vram: float, weights: float, kv_per_seq: float) -> int:
    """floor((total VRAM - weight memory) / per-sequence KV memory)."""
    return int((total_vram - weights) // kv_per_seq)
