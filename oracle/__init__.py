"""CPU oracle for the paged KV cache hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the
``paged_kv_cache_128_amd`` package and its HIP library) never imports it, and
this package never imports the product path: the two share no code.  The only
shared module is ``synth`` (seeded input generation, no method arithmetic).

Everything here is plain, slow and written to be checked by eye against the
pages it follows.  Floating point is evaluated in float64.  Page shorthands
used in the docstrings:

* [MiniPaged-Qwen]  -- "MiniPaged-Qwen：Paged KV Cache 与 KV Block Manager"
  (blog.zsmgc.love), cited by its numbered sections.
* [mini-vLLM BM]    -- "从零实现一个 mini vLLM — Block Manager" (yjxyzxyz.cn),
  cited by its section headings.
* [leetcode-22]     -- "22. vLLM PagedAttention | vLLM 分页注意力"
  (datawhalechina llm-algo-leetcode), cited by its Step / test headings.
* [impl-detail]     -- "paged-attention-impl-detail" (guijiagi.com), cited by
  its section headings.

Pins (checks against values the pages print, closed forms, library routines
and brute force) live in ``tests/test_oracle_*.py``.  Functions with no such
pin say "parity unpinned" in their docstring.
"""
from .manager import (BlockManager, ManagerError, InvalidArgument, OutOfBlocks,
                      NotLive, AlreadyPrefilled, blocks_needed)
from .slots import slot_of, split_slot, kv_head_of
from .cache import new_pool, write_kv, gather_logical, copy_blocks, gather_blocks, scatter_blocks
from .attention import (widen, decode_attention, decode_attention_online,
                        contiguous_attention, prefill_attention)
from .ledger import estimate_kv_cache_bytes, allocation_report, tail_waste

__all__ = [
    "BlockManager", "ManagerError", "InvalidArgument", "OutOfBlocks", "NotLive",
    "AlreadyPrefilled", "blocks_needed", "slot_of", "split_slot", "kv_head_of",
    "new_pool", "write_kv", "gather_logical", "copy_blocks", "gather_blocks", "scatter_blocks", "widen", "decode_attention",
    "decode_attention_online", "contiguous_attention", "prefill_attention", "estimate_kv_cache_bytes",
    "allocation_report", "tail_waste",
]
