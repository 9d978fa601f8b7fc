"""Address translation (oracle, test infrastructure only).

[MiniPaged-Qwen] §3 and §4.1 define the four-step translation from a token
position to a flat slot; §11 defines the inverse split of a slot back into
(physical block, offset); §14 defines the GQA head map.
"""


def slot_of(block_table, token_pos: int, block_size: int) -> int:
    """Flat slot of logical position ``token_pos`` ([MiniPaged-Qwen] §3, §4.1).

    logical_block = floor(token_pos / block_size)
    block_offset  = token_pos mod block_size
    physical_block = block_table[logical_block]
    slot = physical_block * block_size + block_offset
    """
    logical_block = token_pos // block_size
    block_offset = token_pos % block_size
    physical_block = block_table[logical_block]
    return physical_block * block_size + block_offset


def split_slot(slot: int, block_size: int):
    """(physical_block, block_offset) of a flat slot ([MiniPaged-Qwen] §11)."""
    return slot // block_size, slot % block_size


def kv_head_of(q_head: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head ``q_head`` under GQA ([MiniPaged-Qwen] §14):
    group_size = H_q / H_kv and kvh = floor(qh / group_size)."""
    group_size = num_q_heads // num_kv_heads
    return q_head // group_size
