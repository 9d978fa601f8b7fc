"""Byte and utilisation bookkeeping (oracle, test infrastructure only)."""
from __future__ import annotations

from typing import Dict


def estimate_kv_cache_bytes(num_blocks: int, block_size: int, num_layers: int,
                            num_kv_heads: int, head_dim: int, dtype_bytes: int = 2) -> Dict[str, int]:
    """Capacity ledger ([leetcode-22] Step 4 TODO 1; [MiniPaged-Qwen] §2's
    M_KV = 2 * N_layer * L * H_kv * D * bytes): one token holds K and V for
    every layer and KV head; a block holds block_size tokens; the pool holds
    num_blocks blocks."""
    dims = (num_blocks, block_size, num_layers, num_kv_heads, head_dim, dtype_bytes)
    if any(x <= 0 for x in dims):
        raise ValueError("all ledger dimensions must be positive")
    per_token = 2 * num_layers * num_kv_heads * head_dim * dtype_bytes
    per_block = block_size * per_token
    return {"kv_bytes_per_token": per_token, "kv_bytes_per_block": per_block,
            "total_cache_bytes": num_blocks * per_block}


def tail_waste(seq_len: int, block_size: int) -> int:
    """Unused slots of the last block ([MiniPaged-Qwen] §6.2): 0 when
    L mod bs == 0, else bs - (L mod bs)."""
    r = seq_len % block_size
    return 0 if r == 0 else block_size - r


def allocation_report(num_table_blocks: int, seq_len: int, block_size: int) -> Dict[str, float]:
    """Logical tokens, allocated tokens, unused tail and utilisation
    ([leetcode-22] Step 4 ``allocation_report``)."""
    allocated = num_table_blocks * block_size
    return {"logical_tokens": seq_len, "allocated_tokens": allocated,
            "unused_tail_tokens": allocated - seq_len,
            "utilization": (seq_len / allocated) if allocated else 0.0}
