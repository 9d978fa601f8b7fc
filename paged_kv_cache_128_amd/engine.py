"""One layer's paged KV cache on one GPU: the pool, the host block manager,
device-resident block tables and the decode step that ties them together.

A decode step is the hot path of [MiniPaged-Qwen] §10 and §13 in order:

  1. block manager append for every row (one batched C call; all or nothing,
     [mini-vLLM BM] "Block Manager 和 Scheduler 如何协作"), then, when
     sequences share blocks, the copies of the blocks the append copied on
     write ([impl-detail] "Copy-on-Write机制"),
  2. the write of the new K/V rows ([MiniPaged-Qwen] §12), with the blocks
     the append opened published into the device block table and the
     lengths stored on the device, the step's slots and lengths travelling
     in kernel arguments,
  3. paged_decode_attention over the updated cache ([MiniPaged-Qwen] §13),
     so the new token attends to itself ([MiniPaged-Qwen] §1.1: append, then
     attend over positions 0..L).

With the stream attention path (partition_tokens 0), steps 2 and 3 are one
launch (pkv_decode_step) plus the merge; otherwise they are a write launch
and the attention.  With dtype torch.float8_e4m3fn the pool holds 8-bit
rows with one scale byte each ([impl-detail] "实践建议"): writes quantise
(paged_kv_write_fp8 / pkv_decode_write_fp8) and attention reads them back
(paged_decode_attention_fp8); the query keeps its 16-bit type.

Rows are batch positions; each live sequence occupies one row.  All device
memory comes from torch; all work runs in libpkv on torch's current stream.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np
import torch

from . import (KVBlockManager, copy_blocks, copy_table_rows, decode_step, decode_step_fp8, decode_step_noalloc,
               decode_write,
               decode_write_fp8,
               gather_blocks, scatter_blocks, copy_blocks_fp8, gather_blocks_fp8, scatter_blocks_fp8,
               new_fp8_pool, new_pool, paged_decode_attention, paged_decode_attention_fp8,
               paged_kv_write, paged_kv_write_fp8, paged_prefill_attention, paged_prefill_attention_fp8,
               prefill_fp8_workspace_size, workspace_size)


def _check_distinct(rows: Sequence[int]) -> None:
    if len(set(int(r) for r in rows)) != len(rows):
        raise ValueError("rows must be distinct")


class _HostStage:
    """Pinned host staging for the small host-to-device copies of admissions
    (slots, table rows, chunk offsets): a bump arena whose copies are queued
    without synchronising the stream.  When the arena wraps, the device is
    synchronised once, so every copy out of the previous lap has run before
    its bytes are reused, whichever stream it was queued on."""

    def __init__(self, nbytes: int, device):
        self.device = device
        self.buf = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        self.off = 0

    def _stage(self, arr: np.ndarray):
        """The bytes of arr in the arena (None when larger than the arena)."""
        n = arr.nbytes
        if n > self.buf.numel():
            return None
        at = (self.off + 255) & ~255
        if at + n > self.buf.numel():
            torch.cuda.synchronize(self.device)
            at = 0
        self.off = at + n
        host = self.buf[at:at + n]
        host.numpy()[:] = arr.view(np.uint8).reshape(-1)
        return host.view(_TORCH_OF[arr.dtype])

    def to_device(self, arr: np.ndarray) -> torch.Tensor:
        arr = np.ascontiguousarray(arr)
        host = self._stage(arr)
        if host is None:                             # larger than the arena: a plain copy
            return torch.from_numpy(arr).to(self.device)
        return host.to(self.device, non_blocking=True)

    def copy_into(self, dst: torch.Tensor, arr: np.ndarray) -> None:
        """arr into the contiguous device tensor dst by one host-to-device
        copy from the arena (no device-side copy kernel)."""
        arr = np.ascontiguousarray(arr)
        host = self._stage(arr)
        if host is None:
            host = torch.from_numpy(arr)
        dst.copy_(host.view(dst.shape), non_blocking=True)


_TORCH_OF = {np.dtype(np.int64): torch.int64, np.dtype(np.int32): torch.int32}


class PagedKVEngine:
    def __init__(self, num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
                 dtype: torch.dtype, max_rows: int, max_blocks_per_seq: int,
                 initial_free_order: Optional[Sequence[int]] = None, device="cuda",
                 fill_bits: Optional[int] = None, partition_tokens: int = 0,
                 num_q_heads: Optional[int] = None):
        self.device = torch.device(device)
        self.num_blocks = num_blocks
        self.num_kv_heads = num_kv_heads
        self.block_size = block_size
        self.head_dim = head_dim
        self.dtype = dtype
        self.max_rows = max_rows
        self.width = max_blocks_per_seq
        self.partition_tokens = partition_tokens
        self.manager = KVBlockManager(num_blocks, block_size, initial_free_order)
        self.fp8 = dtype == torch.float8_e4m3fn
        if self.fp8:
            (self.pool, self.key_cache, self.value_cache, self.scales, self.key_scales,
             self.value_scales) = new_fp8_pool(num_blocks, num_kv_heads, block_size, head_dim,
                                               self.device, poison=fill_bits is not None)
        else:
            self.pool, self.key_cache, self.value_cache = new_pool(
                num_blocks, num_kv_heads, block_size, head_dim, dtype, self.device, fill_bits)
        self.tables = torch.full((max_rows, self.width), -1, dtype=torch.int32, device=self.device)
        self.row_seq: Dict[int, int] = {}
        self.d_lens = torch.zeros(max_rows, dtype=torch.int32, device=self.device)
        self.slots = np.empty(max_rows, dtype=np.int64)      # last step's slots (host)
        self.lens = np.empty(max_rows, dtype=np.int32)       # last step's lengths (host)
        self._newb = np.empty(max_rows, dtype=np.int32)
        self._ids = np.empty(max_rows, dtype=np.int64)       # the step's sequence ids
        # the persistent host arrays' addresses, for the per-step append
        self._addr = tuple(x.__array_interface__["data"][0] for x in (self._ids, self.slots, self.lens, self._newb))
        self._ws = None
        self._pf_ws = None         # 16-bit staging of 8-bit prefill
        self._nq = num_q_heads
        self._sharing = False      # set once any table shares a block
        self._stage = _HostStage(4 << 20, self.device)
        self._copy_stream = None   # swap-out device-to-host copies (default priority)
        self._swap_done: Dict[int, torch.cuda.Event] = {}

    # -- admission / release ------------------------------------------------
    def prefill(self, seq_id: int, row: int, key: torch.Tensor, value: torch.Tensor,
                num_tokens: Optional[int] = None) -> np.ndarray:
        """Admit ``seq_id`` into ``row`` with its prompt K/V ([n, H_kv, D]
        device tensors, n may be 0): allocate, write, publish the table row."""
        n = key.shape[0] if num_tokens is None else num_tokens
        slots = self.manager.allocate_for_prefill(seq_id, n)
        if n > 0:
            d_slots = self._stage.to_device(slots)
            self._write(key, value, d_slots)
        self._publish_row(seq_id, row)
        return slots

    def prefill_chunk(self, seq_ids: Sequence[int], rows: Sequence[int], chunk_lens: Sequence[int],
                      key: torch.Tensor, value: torch.Tensor, q: torch.Tensor, scale: float,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """One prefill chunk per sequence: a sequence not yet live is admitted
        with its chunk as its prompt, a live one is extended by it
        (pkv_append_tokens); the chunks' K/V rows ([sum(chunk_lens), H_kv, D],
        concatenated in order) are written, then every chunk's query rows
        (q [sum(chunk_lens), H_q, D]) attend causally over their sequence
        (paged_prefill_attention; over an 8-bit pool paged_prefill_attention_fp8,
        bf16 or fp16 q); ``rows`` distinct.  The allocation is all or nothing
        (pkv_admit_batch).  Returns out [sum(chunk_lens), H_q, D]."""
        _check_distinct(rows)
        if not (len(seq_ids) == len(rows) == len(chunk_lens)):
            raise ValueError("one row and one chunk length per sequence")
        # all or nothing: a batch the free list cannot hold changes nothing
        slots, lens = self.manager.admit_batch(seq_ids, chunk_lens, extend_live=True)
        self._run_copies()
        if slots.size:
            self._write(key, value, self._stage.to_device(slots))
        self._publish_rows(seq_ids, rows)
        B = len(seq_ids)
        q_start = np.concatenate([[0], np.cumsum(np.asarray(chunk_lens, dtype=np.int64))]).astype(np.int32)
        d_qs = self._stage.to_device(q_start)
        d_lens = self._stage.to_device(lens)
        rows_np = np.asarray(list(rows), dtype=np.int32)
        if np.array_equal(rows_np, np.arange(B, dtype=np.int32)):
            tables = self.tables[:B]                 # the rows already in batch order: a view
        else:                                        # the batch's rows gathered in order
            tables = torch.empty((B, self.width), dtype=torch.int32, device=self.device)
            copy_table_rows(tables, self.tables, B, src_rows=self._stage.to_device(rows_np))
        max_q = int(max(chunk_lens)) if B else 0
        max_len = int(max(lens)) if B else 0
        if self.fp8:
            need = prefill_fp8_workspace_size(B, max_len, self.key_cache, self.value_cache)
            if self._pf_ws is None or self._pf_ws.numel() < need:
                self._pf_ws = torch.empty(max(need, 1), dtype=torch.uint8, device=self.device)
            return paged_prefill_attention_fp8(q, d_qs, self.key_cache, self.value_cache, self.key_scales,
                                               self.value_scales, tables, d_lens, scale, max_q_len=max_q,
                                               max_context_len=max_len, out=out, workspace=self._pf_ws)
        return paged_prefill_attention(q, d_qs, self.key_cache, self.value_cache, tables, d_lens, scale,
                                       max_q_len=max_q, max_context_len=max_len, out=out)

    def _run_copies(self):
        """Copy-on-write: the block copies the manager queued, on the stream,
        before anything writes into the new blocks."""
        if not self._sharing:
            return
        src, dst = self.manager.take_copies()
        if not len(src):
            return
        if self.fp8:
            copy_blocks_fp8(src, dst, self.key_cache, self.value_cache, self.key_scales, self.value_scales)
        else:
            copy_blocks(src, dst, self.key_cache, self.value_cache)

    def _write(self, key, value, d_slots):
        if self.fp8:
            paged_kv_write_fp8(key, value, d_slots, self.key_cache, self.value_cache,
                               self.key_scales, self.value_scales)
        else:
            paged_kv_write(key, value, d_slots, self.key_cache, self.value_cache)

    def prefill_many(self, seq_ids: Sequence[int], rows: Sequence[int], lengths: Sequence[int],
                     key: torch.Tensor, value: torch.Tensor) -> np.ndarray:
        """Admit several sequences whose prompt rows are concatenated in
        ``key``/``value`` ([sum(lengths), H_kv, D]) with one write launch and
        one table publication (``rows`` distinct).  The allocation is all or
        nothing (pkv_admit_batch): when one sequence cannot be admitted, no
        sequence is, and nothing is written or published."""
        _check_distinct(rows)
        if not (len(seq_ids) == len(rows) == len(lengths)):
            raise ValueError("one row and one length per sequence")
        # all or nothing: a batch the free list cannot hold changes nothing
        slots, _ = self.manager.admit_batch(seq_ids, lengths, extend_live=False)
        if slots.size:
            d_slots = self._stage.to_device(slots)
            self._write(key, value, d_slots)
        self._publish_rows(seq_ids, rows)
        return slots

    def share_prefix(self, donor_id: int, seq_id: int, row: int, num_tokens: int) -> None:
        """Admit ``seq_id`` into ``row`` holding the first ``num_tokens`` tokens
        of live ``donor_id`` on the donor's blocks, no copy
        ([impl-detail] "前缀共享"); its appends copy a shared block first."""
        self.manager.share_prefix(donor_id, seq_id, num_tokens)
        self._sharing = True
        self._publish_row(seq_id, row)

    def swap_out(self, seq_id: int) -> torch.Tensor:
        """Move a live sequence's blocks to pinned host memory and release
        them ([impl-detail] "异构内存支持" evict_to_cpu): gather on the device
        (on the current stream, so it reads the blocks before any later work
        there reuses them), then one device-to-host copy on the engine's copy
        stream, which overlaps the decode steps queued after it.  Returns the
        host copy, which swap_in takes back: one pinned tensor
        [n, 2, H_kv, bs, D], or for an 8-bit pool the pair (codes, scale bytes
        [n, 2, H_kv, bs]).  It holds the data once wait_swap(seq_id) has
        returned; swap_in waits for the copy by itself.  The sequence's row is
        left to the caller."""
        ids = self.manager.swap_out(seq_id)
        if self.fp8:
            staged = gather_blocks_fp8(ids, self.key_cache, self.value_cache, self.key_scales, self.value_scales)
        else:
            staged = (gather_blocks(ids, self.key_cache, self.value_cache),)
        host = tuple(torch.empty(t.shape, dtype=t.dtype, pin_memory=True) for t in staged)
        if self._copy_stream is None:
            self._copy_stream = torch.cuda.Stream(self.device)
        cs = self._copy_stream
        cs.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(cs):
            for h, t in zip(host, staged):
                h.copy_(t, non_blocking=True)
        for t in staged:
            t.record_stream(cs)        # its memory is not handed out again before the copy has read it
        self._swap_done[seq_id] = cs.record_event()
        for r, s in list(self.row_seq.items()):
            if s == seq_id:
                del self.row_seq[r]
        return host if self.fp8 else host[0]

    def wait_swap(self, seq_id: int) -> None:
        """Blocks the host until the device-to-host copy of seq_id's last
        swap_out has landed."""
        ev = self._swap_done.get(seq_id)
        if ev is not None:
            ev.synchronize()

    def swap_in(self, seq_id: int, row: int, host: torch.Tensor) -> None:
        """Bring a swapped sequence back into ``row`` on fresh blocks
        ([impl-detail] "异构内存支持" prefetch_to_gpu): one host-to-device
        copy, a scatter, and the table row published."""
        ids = self.manager.swap_in(seq_id)
        ev = self._swap_done.pop(seq_id, None)
        if ev is not None:             # the host copy is read after it has been written
            torch.cuda.current_stream(self.device).wait_event(ev)
        if self.fp8:
            codes, scales = (t.to(self.device, non_blocking=True) for t in host)
            scatter_blocks_fp8(codes, scales, ids, self.key_cache, self.value_cache, self.key_scales,
                               self.value_scales)
        else:
            scatter_blocks(host.to(self.device, non_blocking=True), ids, self.key_cache, self.value_cache)
        self._publish_row(seq_id, row)

    def _publish_row(self, seq_id: int, row: int):
        tab = self.manager.block_tables([seq_id], self.width, -1)
        self._stage.copy_into(self.tables[row], tab[0])
        self.row_seq[row] = seq_id

    def _publish_rows(self, seq_ids: Sequence[int], rows: Sequence[int]):
        """The table rows of several sequences at once (distinct rows): one
        table read from the manager, one staged copy, one row scatter
        (pkv_copy_table_rows)."""
        if len(rows) == 1:
            self._publish_row(int(seq_ids[0]), int(rows[0]))
            return
        if len(rows) == 0:
            return
        tab = self.manager.block_tables([int(x) for x in seq_ids], self.width, -1)
        d_rows = self._stage.to_device(np.asarray(rows, dtype=np.int32))
        copy_table_rows(self.tables, self._stage.to_device(tab).view(len(rows), self.width), len(rows),
                        dst_rows=d_rows)
        for sid, row in zip(seq_ids, rows):
            self.row_seq[int(row)] = int(sid)

    def free(self, seq_id: int) -> None:
        self.manager.free_sequence(seq_id)
        self._swap_done.pop(seq_id, None)
        for r, s in list(self.row_seq.items()):
            if s == seq_id:
                del self.row_seq[r]

    # -- decode ---------------------------------------------------------------
    def workspace(self, num_seqs: int, num_q_heads: int, max_context_len: int) -> Optional[torch.Tensor]:
        need = workspace_size(num_seqs, num_q_heads, self.num_kv_heads, self.head_dim,
                              max_context_len, self.partition_tokens)
        if need == 0:
            return None
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws

    def decode_step(self, seq_ids: np.ndarray, new_k: torch.Tensor, new_v: torch.Tensor,
                    q: torch.Tensor, scale: float, max_context_len: Optional[int] = None,
                    out: Optional[torch.Tensor] = None, events=None,
                    fused: bool = True, noalloc: bool = False) -> torch.Tensor:
        """One decode step for rows 0..n-1 holding ``seq_ids`` (int64).
        ``max_context_len`` defaults to the longest length after the append
        (known on the host from the manager, no device sync).  ``events``
        (three torch.cuda.Event) are recorded before the attention kernel
        (with the fused step: the write-and-attention kernel), between it and
        the merge, and after the merge; two are recorded around the whole
        step, a separate write launch included.  ``fused`` = False forces the
        separate write launch.  ``noalloc`` (16-bit pools, no events) runs the
        step through pkv_decode_step_noalloc: no workspace, the library's own
        per-GPU array instead."""
        n = len(seq_ids)
        if n > self.max_rows:
            raise ValueError("more sequences than the engine's rows")
        if noalloc and (self.fp8 or events is not None or self.partition_tokens != 0):
            raise ValueError("the no-allocation step covers 16-bit pools on the stream path, without events")
        self._ids[:n] = seq_ids
        self.manager._append_at(self._addr[0], n, self._addr[1], self._addr[2], self._addr[3])
        self._run_copies()
        if max_context_len is None:
            max_context_len = int(self.lens[:n].max()) if n else 0
        # two events bracket the whole step, the separate write launch included
        whole = events is not None and len(events) == 2
        if self.fp8 and not fused:
            if whole:
                events[0].record()
            decode_write_fp8(new_k, new_v, self.slots[:n], self.lens[:n], self.key_cache,
                             self.value_cache, self.key_scales, self.value_scales,
                             block_tables=self.tables, lens_out=self.d_lens)
            return self.attend(q, self.d_lens[:n], scale, max_context_len, out=out, events=events,
                               _started=whole)
        if self.fp8:
            ws = self.workspace(n, q.shape[1], max_context_len)
            if out is None:
                out = torch.empty(q.shape, dtype=torch.float32, device=self.device)
            args8 = (q, new_k, new_v, self.slots[:n], self.lens[:n], self.key_cache, self.value_cache,
                     self.key_scales, self.value_scales, self.tables, self.d_lens, scale, max_context_len)
            return decode_step_fp8(*args8, out=out, workspace=ws, events=events)
        if noalloc:
            if out is None:
                out = torch.empty(q.shape, dtype=torch.float32, device=self.device)
            return decode_step_noalloc(q, new_k, new_v, self.slots[:n], self.lens[:n], self.key_cache,
                                       self.value_cache, self.tables, self.d_lens, scale, max_context_len,
                                       out=out)
        if not (fused and self.partition_tokens == 0 and n > 0):
            if whole:
                events[0].record()
            decode_write(new_k, new_v, self.slots[:n], self.lens[:n], self.key_cache, self.value_cache,
                         block_tables=self.tables, lens_out=self.d_lens)
            return self.attend(q, self.d_lens[:n], scale, max_context_len, out=out, events=events,
                               _started=whole)
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=self.device)
        args = (q, new_k, new_v, self.slots[:n], self.lens[:n], self.key_cache, self.value_cache,
                self.tables, self.d_lens, scale, max_context_len)
        ws = self.workspace(n, q.shape[1], max_context_len)
        return decode_step(*args, out=out, workspace=ws, events=events)

    def attend(self, q: torch.Tensor, lens: torch.Tensor, scale: float, max_context_len: int,
               out: Optional[torch.Tensor] = None, events=None, _started: bool = False) -> torch.Tensor:
        """Attention of rows 0..B-1 over the current cache (no append/write).
        Two ``events`` bracket the launches, three also split them at the
        partial / merge boundary; ``_started`` says the first of two events
        was already recorded (before the step's write)."""
        n = q.shape[0]
        ws = self.workspace(n, q.shape[1], max_context_len)
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=self.device)
        if self.fp8:
            args = (q, self.key_cache, self.value_cache, self.key_scales, self.value_scales,
                    self.tables[:n], lens, scale)
            kw8 = dict(out=out, max_context_len=max_context_len, workspace=ws)
            if events is None:
                return paged_decode_attention_fp8(*args, **kw8)
            if len(events) == 2:
                if not _started:
                    events[0].record()
                paged_decode_attention_fp8(*args, **kw8)
                events[1].record()
                return out
            events[0].record()
            paged_decode_attention_fp8(*args, phase="partial", **kw8)
            events[1].record()
            paged_decode_attention_fp8(*args, phase="merge", **kw8)
            events[2].record()
            return out
        kw = dict(partition_tokens=self.partition_tokens, max_context_len=max_context_len,
                  workspace=ws)
        if events is not None and len(events) == 2:
            if not _started:
                events[0].record()
            paged_decode_attention(q, self.key_cache, self.value_cache, self.tables[:n], lens, scale,
                                   out=out, **kw)
            events[1].record()
            return out
        if events is None:
            return paged_decode_attention(q, self.key_cache, self.value_cache, self.tables[:n],
                                          lens, scale, out=out, **kw)
        events[0].record()
        paged_decode_attention(q, self.key_cache, self.value_cache, self.tables[:n], lens, scale,
                               out=out, phase="partial", **kw)
        events[1].record()
        paged_decode_attention(q, self.key_cache, self.value_cache, self.tables[:n], lens, scale,
                               out=out, phase="merge", **kw)
        events[2].record()
        return out
