"""Replays of the seeded ``synth`` workloads on the oracle (test infrastructure).

Each replay drives the oracle manager and the oracle pool through the same
event order the GPU side uses: churn events, history prefill + write, then the
measured append + write.  Nothing here is shared with the GPU side.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

import synth

from .cache import new_pool, write_kv
from .manager import BlockManager


@dataclasses.dataclass
class OracleDecodeState:
    manager: BlockManager
    key_cache: np.ndarray
    value_cache: np.ndarray
    step_slots: List[int]
    block_tables: np.ndarray
    context_lens: np.ndarray
    prefill_slots: List[List[int]]


def replay_churn(mgr: BlockManager, events) -> None:
    for ev in events:
        if ev[0] == "prefill":
            mgr.allocate_for_prefill(ev[1], ev[2])
        elif ev[0] == "grow":
            for _ in range(ev[2]):
                mgr.append_slots_for_decode(list(ev[1]))
        elif ev[0] == "free":
            mgr.free_sequence(ev[1])
        else:
            raise ValueError(ev)


def decode_state(wl: "synth.DecodeWorkload", width: Optional[int] = None,
                 pad: int = -1) -> OracleDecodeState:
    cfg = wl.cfg
    mgr = BlockManager(cfg.num_blocks, cfg.block_size, wl.initial_free_order)
    replay_churn(mgr, wl.churn)
    fill = synth.poison_array((), cfg.dtype)
    kc, vc = new_pool(cfg.num_blocks, cfg.num_kv_heads, cfg.block_size, cfg.head_dim, fill)
    ids = wl.seq_ids
    prefill_slots = []
    for b in ids:
        slots = mgr.allocate_for_prefill(b, int(wl.context_lens[b]) - 1)
        write_kv(wl.hist_k[b], wl.hist_v[b], slots, kc, vc, cfg.block_size)
        prefill_slots.append(slots)
    step = mgr.append_slots_for_decode(ids)
    write_kv(wl.new_k, wl.new_v, step, kc, vc, cfg.block_size)
    if width is None:
        width = max(len(mgr.block_table(b)) for b in ids)
    return OracleDecodeState(mgr, kc, vc, step, mgr.block_tables(ids, width, pad),
                             mgr.context_lens(ids), prefill_slots)


def serving_replay(trace: "synth.ServingTrace"):
    """Oracle replay of the serving trace: initial prefill of every row, then
    per step the batched append, the write of the step's K/V rows, a yield
    (the caller may run the oracle attention on the state), and the finishes
    with their refills.  Yields (step, manager, key_cache, value_cache,
    row_ids, step_slots)."""
    cfg = trace.cfg
    mgr = BlockManager(cfg.num_blocks, cfg.block_size)
    fill = synth.poison_array((), cfg.dtype)
    kc, vc = new_pool(cfg.num_blocks, cfg.num_kv_heads, cfg.block_size, cfg.head_dim, fill)
    B = len(trace.prompt_lens)
    row_ids = list(range(B))
    for b in range(B):
        slots = mgr.allocate_for_prefill(b, int(trace.prompt_lens[b]))
        write_kv(trace.hist_k[b], trace.hist_v[b], slots, kc, vc, cfg.block_size)
    for st in trace.steps:
        slots = mgr.append_slots_for_decode(row_ids)
        write_kv(st.new_k, st.new_v, slots, kc, vc, cfg.block_size)
        yield st, mgr, kc, vc, row_ids, slots
        for r in st.refills:
            mgr.free_sequence(r.old_id)
            s = mgr.allocate_for_prefill(r.new_id, r.prompt_len)
            write_kv(r.k, r.v, s, kc, vc, cfg.block_size)
            row_ids[r.row] = r.new_id
