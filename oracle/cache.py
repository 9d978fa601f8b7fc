"""Paged KV pool, cache write and logical gather (oracle, test infrastructure only).

Pool layout follows [MiniPaged-Qwen] §11: separate ``key_cache`` and
``value_cache`` arrays of shape [num_blocks, H_kv, block_size, D], indexed
[physical_block, kvh, block_offset, :].  Storage keeps the dtype's raw values
(numpy uint16 bit patterns for bf16), so a write is an exact copy.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

from .slots import split_slot


def new_pool(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
             fill: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Two pool arrays filled with the scalar array ``fill`` (a poison value,
    so that any read of a slot no write touched is visible)."""
    shape = (num_blocks, num_kv_heads, block_size, head_dim)
    k = np.empty(shape, dtype=fill.dtype)
    k[...] = fill
    v = np.empty(shape, dtype=fill.dtype)
    v[...] = fill
    return k, v


def write_kv(key: np.ndarray, value: np.ndarray, slot_mapping: Sequence[int],
             key_cache: np.ndarray, value_cache: np.ndarray, block_size: int) -> None:
    """Cache write ([MiniPaged-Qwen] §12): for each new token i,
    (pb, off) = split(slot_mapping[i]) and
    key_cache[pb, :, off, :] = key[i]; value_cache[pb, :, off, :] = value[i].

    Reading for slots outside [0, num_blocks * block_size) (the pages never
    produce one): the token is skipped and nothing is written.
    """
    capacity = key_cache.shape[0] * block_size
    for i, slot in enumerate(slot_mapping):
        slot = int(slot)
        if slot < 0 or slot >= capacity:
            continue
        pb, off = split_slot(slot, block_size)
        key_cache[pb, :, off, :] = key[i]
        value_cache[pb, :, off, :] = value[i]


def copy_blocks(pairs: Sequence[Tuple[int, int]], key_cache: np.ndarray,
                value_cache: np.ndarray) -> None:
    """Copy-on-write copies ([impl-detail] "Copy-on-Write机制": the new block
    takes the shared block's k and v): for each (src, dst) in order,
    key_cache[dst] = key_cache[src] and value_cache[dst] = value_cache[src],
    every head and token row.  Pairs with an id outside [0, num_blocks) are
    skipped."""
    n = key_cache.shape[0]
    for src, dst in pairs:
        src, dst = int(src), int(dst)
        if not (0 <= src < n and 0 <= dst < n):
            continue
        key_cache[dst] = key_cache[src]
        value_cache[dst] = value_cache[src]


def gather_blocks(ids: Sequence[int], key_cache: np.ndarray, value_cache: np.ndarray) -> np.ndarray:
    """Swap-out staging ([impl-detail] "异构内存支持": a block's k and v go to
    host memory): blocks ``ids`` in order as one array [n, 2, H, bs, D]
    (K half, then V half)."""
    return np.stack([np.stack([key_cache[int(i)], value_cache[int(i)]]) for i in ids]) \
        if len(ids) else np.empty((0, 2) + key_cache.shape[1:], key_cache.dtype)


def scatter_blocks(staged: np.ndarray, ids: Sequence[int], key_cache: np.ndarray,
                   value_cache: np.ndarray) -> None:
    """Swap-in: staged block j back into block ids[j] of both pools."""
    for j, i in enumerate(ids):
        key_cache[int(i)] = staged[j, 0]
        value_cache[int(i)] = staged[j, 1]


def gather_logical(cache: np.ndarray, block_table: Sequence[int], seq_len: int) -> np.ndarray:
    """Logically contiguous [H_kv, seq_len, D] view of one sequence: blocks in
    TABLE order (never sorted by physical id), concatenated along the token
    axis and truncated to seq_len ([leetcode-22] Step 4 TODO 4
    ``get_physical_cache``; [MiniPaged-Qwen] §13 and §16.6)."""
    if seq_len == 0:
        return cache[:0].reshape(cache.shape[1], 0, cache.shape[3])
    block_size = cache.shape[2]
    nb = -(-seq_len // block_size)
    blocks = [cache[int(pb)] for pb in block_table[:nb]]
    return np.concatenate(blocks, axis=1)[:, :seq_len, :]
