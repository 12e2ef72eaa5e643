"""KV-cache sizing: bytes per token and pool sizes.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Formula from "苦猿的大模型日记 · Day45 · 大模型推理加速", PART 02 (the one-line
per-token formula): KV bytes per token = 2 (K and V) x num_layers x
num_kv_heads x head_dim x dtype_bytes.  fp8 and int8 store one byte per
element; their per-(block, KV head) fp32 scales are extra and counted
separately.
"""
from __future__ import annotations

DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1, "int8": 1}


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, dtype: str) -> int:
    return 2 * num_layers * num_kv_heads * head_dim * DTYPE_BYTES[dtype]


def blocks_for_tokens(num_tokens: int, block_size: int) -> int:
    """Blocks a sequence of ``num_tokens`` occupies: ceil(n / block_size)
    ("大模型推理加速核心KV Cache 复用机制与内存布局优化" §三, ``allocate``)."""
    return (num_tokens + block_size - 1) // block_size


def pool_bytes(num_layers: int, num_blocks: int, num_kv_heads: int, head_dim: int,
               block_size: int, dtype: str) -> int:
    """Bytes of ONE pool (K or V): every block holds block_size tokens of every
    layer and KV head."""
    return num_layers * num_blocks * num_kv_heads * block_size * head_dim * DTYPE_BYTES[dtype]


def scale_bytes(num_layers: int, num_blocks: int, num_kv_heads: int) -> int:
    """Bytes of ONE fp8 / int8 scale array (K or V): one fp32 per (layer, block, KV head)."""
    return num_layers * num_blocks * num_kv_heads * 4
