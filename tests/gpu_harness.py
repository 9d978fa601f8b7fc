"""Shared set-up for the GPU tests: replays a ``synth`` workload through the
product path (C++ block manager, HIP write and attention via the binding)
and, separately, through the oracle.  Nothing here is imported by the
product or by the oracle."""
from __future__ import annotations

import numpy as np
import torch

import synth

TORCH_DTYPE = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def to_device(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Storage-dtype numpy array -> device tensor with identical bits."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def bits_u(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy unsigned integers of the same bits."""
    t = t.contiguous().cpu()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.int32).numpy().view(np.uint32)


def replay_churn_device(mgr, events):
    for ev in events:
        if ev[0] == "prefill":
            mgr.allocate_for_prefill(ev[1], ev[2], want_slots=False)
        elif ev[0] == "grow":
            for _ in range(ev[2]):
                mgr.append_slots_for_decode(list(ev[1]))
        else:
            mgr.free_sequence(ev[1])


def engine_for(wl: synth.DecodeWorkload, width=None, partition_tokens=None, poison=True):
    """Product-path state of a single-step decode workload after the history
    prefill (not yet the measured step)."""
    from paged_kv_cache_128_amd.engine import PagedKVEngine
    cfg = wl.cfg
    B = len(wl.context_lens)
    if width is None:
        width = int(-(-int(wl.context_lens.max()) // cfg.block_size))
    part = cfg.partition_tokens if partition_tokens is None else partition_tokens
    eng = PagedKVEngine(cfg.num_blocks, cfg.num_kv_heads, cfg.block_size, cfg.head_dim,
                        TORCH_DTYPE[cfg.dtype], B, width, wl.initial_free_order,
                        fill_bits=synth.POISON_BITS[cfg.dtype] if poison else None,
                        partition_tokens=part, num_q_heads=cfg.num_q_heads)
    replay_churn_device(eng.manager, wl.churn)
    lens = [int(L) - 1 for L in wl.context_lens]
    k = to_device(np.concatenate(wl.hist_k, axis=0), cfg.dtype)
    v = to_device(np.concatenate(wl.hist_v, axis=0), cfg.dtype)
    eng.prefill_many(list(range(B)), list(range(B)), lens, k, v)
    return eng


def run_step(eng, wl: synth.DecodeWorkload, out_dtype=None):
    cfg = wl.cfg
    B = len(wl.context_lens)
    ids = np.arange(B, dtype=np.int64)
    nk = to_device(wl.new_k, cfg.dtype)
    nv = to_device(wl.new_v, cfg.dtype)
    q = to_device(wl.q, cfg.dtype)
    out = None
    if out_dtype is not None:
        out = torch.empty((B, cfg.num_q_heads, cfg.head_dim), dtype=out_dtype, device="cuda")
    o = eng.decode_step(ids, nk, nv, q, cfg.scale, out=out)
    torch.cuda.synchronize()
    return o
