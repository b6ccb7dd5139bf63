"""Pool sizing arithmetic (host).

  * one layer's page holds K and V for block_size tokens:
    ``2 * block_size * num_kv_heads * head_dim * elem_bytes`` bytes
    ("Paging saves no KV bytes", section 2, page_size formula);
  * blocks that fit = available bytes // page bytes // layers, an integer
    division ("Paging saves no KV bytes", section 2, get_num_blocks);
  * max concurrency = num_blocks / cdiv(max_len, block_size)
    ("Paging saves no KV bytes", section 4).
"""
from __future__ import annotations


def cdiv(a: int, b: int) -> int:
    return -(-int(a) // int(b))


def pool_block_bytes(block_size: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes of one block in ONE pool (K or V) of one layer."""
    return int(block_size) * int(num_kv_heads) * int(head_dim) * int(elem_bytes)


def page_bytes(block_size: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes of one block of one layer counting both K and V."""
    return 2 * pool_block_bytes(block_size, num_kv_heads, head_dim, elem_bytes)


def bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return 2 * int(num_layers) * int(num_kv_heads) * int(head_dim) * int(elem_bytes)


def num_blocks_for(available_bytes: int, page: int, num_layers: int) -> int:
    return max(int(available_bytes) // int(page) // int(num_layers), 0)


def max_concurrency(num_blocks: int, max_len: int, block_size: int) -> float:
    return int(num_blocks) / cdiv(max_len, block_size)


def slots_allocated(num_tokens: int, block_size: int) -> int:
    return cdiv(num_tokens, block_size) * int(block_size)
