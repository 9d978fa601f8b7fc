"""Byte and utilisation bookkeeping (oracle, test infrastructure only).

Everything here is the KV-size formula of [MiniPaged-Qwen] §2,
M_KV = 2 * N_layer * L * H_kv * D * bytes (K and V, every layer and KV
head, L tokens), applied to a pool of blocks and to one block table.  The
result keys are the names [leetcode-22]'s asserted tests check.
"""
from __future__ import annotations

from typing import Dict


def kv_cache_bytes(tokens: int, num_layers: int, num_kv_heads: int, head_dim: int,
                   dtype_bytes: int) -> int:
    """M_KV of [MiniPaged-Qwen] §2 for ``tokens`` tokens."""
    return 2 * num_layers * tokens * num_kv_heads * head_dim * dtype_bytes


def estimate_kv_cache_bytes(num_blocks: int, block_size: int, num_layers: int,
                            num_kv_heads: int, head_dim: int, dtype_bytes: int = 2) -> Dict[str, int]:
    """Capacity of a pool of ``num_blocks`` blocks of ``block_size`` tokens
    ([leetcode-22] Step 4 TODO 1): M_KV of one token and of every token the
    pool can hold."""
    shape = dict(num_blocks=num_blocks, block_size=block_size, num_layers=num_layers,
                 num_kv_heads=num_kv_heads, head_dim=head_dim, dtype_bytes=dtype_bytes)
    bad = [k for k, x in shape.items() if x <= 0]
    if bad:
        raise ValueError(f"ledger dimensions must be positive: {', '.join(bad)}")
    per_token = kv_cache_bytes(1, num_layers, num_kv_heads, head_dim, dtype_bytes)
    return {"kv_bytes_per_token": per_token,
            "kv_bytes_per_block": per_token * block_size,
            "total_cache_bytes": kv_cache_bytes(num_blocks * block_size, num_layers, num_kv_heads, head_dim,
                                                dtype_bytes)}


def tail_waste(seq_len: int, block_size: int) -> int:
    """Unused slots of the last block ([MiniPaged-Qwen] §6.2): 0 when
    L mod bs == 0, else bs - (L mod bs)."""
    r = seq_len % block_size
    return 0 if r == 0 else block_size - r


def allocation_report(num_table_blocks: int, seq_len: int, block_size: int) -> Dict[str, float]:
    """How much of a table's blocks a sequence of ``seq_len`` tokens fills
    ([leetcode-22] Step 4 ``allocation_report``): the slots the table
    covers, the ones past the last token, and the filled fraction."""
    slots = num_table_blocks * block_size
    empty = slots - seq_len
    return {"allocated_tokens": slots, "unused_tail_tokens": empty,
            "utilization": 1.0 - empty / slots if slots else 0.0}
