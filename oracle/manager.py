"""Block manager (oracle, test infrastructure only).

The pages' manager, written out as a plain Python object:

* state: a pool of ``num_blocks`` physical ids, an ordered free list and, per
  live sequence, its length and block table ([MiniPaged-Qwen] §8.1, §8.2;
  [mini-vLLM BM] "Block Manager 要维护哪些东西").
* ``allocate_for_prefill`` takes ceil(n / block_size) blocks from the FRONT of
  the free list, all or nothing ([mini-vLLM BM] "prefill 时如何分配 block";
  [leetcode-22] Step 4 TODO 2, "Prefill 原子分配").
* ``append_slot_for_decode`` allocates one front block exactly when the
  position opens a new logical block (logical_block == len(block_table)),
  returns the slot and increments the length ([MiniPaged-Qwen] §5.2 and §9;
  [mini-vLLM BM] "decode 时如何追加 slot").  On an empty free list it fails
  and changes nothing ([leetcode-22] Step 2 table, decode rollback test).
* ``append_slots_for_decode`` is the batched form with the all-or-nothing
  pre-check the scheduler needs ([mini-vLLM BM] "Block Manager 和 Scheduler
  如何协作", can_append_slots).
* ``free_sequence`` drops the sequence's reference to each block of its
  table and appends the blocks no table holds any more onto the free list,
  in table order ([MiniPaged-Qwen] §5.3; [mini-vLLM BM] "释放 block";
  [impl-detail] "块池" ref_count).  With ``sort_on_release`` the free list
  is sorted afterwards, which is what [leetcode-22] reference answer
  ``release_request`` does.
* Prefix sharing and copy-on-write ([impl-detail] "Copy-on-Write共享"):
  every block carries a reference count, the number of tables holding it.
  ``share_prefix`` starts a sequence on the first ceil(n / bs) blocks of a
  live donor (count + 1 each, "前缀共享").  An append whose token lands in a
  block held by more than one table first takes a free block, queues a
  copy of the shared block into it, drops one reference from the shared
  block and puts the new block in the table ("Copy-on-Write机制").  The
  queued (source, destination) pairs are drained by ``take_copies``; the
  caller copies those blocks before it writes the step's rows.
* Swap to host ([impl-detail] "异构内存支持" evict_to_cpu / prefetch_to_gpu):
  ``swap_out`` gives a live sequence's blocks back to the free list (in
  table order) and keeps its length, so the caller can copy those blocks to
  host memory first; ``swap_in`` takes ceil(len / bs) blocks from the front
  of the free list, all or nothing, for the caller to copy back into.  A
  sequence holding a shared block cannot be swapped out (its blocks would
  stay in other tables).
* ``check_invariants`` tests the invariants of [MiniPaged-Qwen] §15 and
  [mini-vLLM BM] "正确性不变量", with I1 read for shared blocks as "each
  block's count equals the number of tables holding it".

Readings taken where the pages are open (each listed in the design notes):
allocation from the front of an ordered free list, release by appending in
table order; the boundary rule of [MiniPaged-Qwen] §9 (not leetcode-22's
``new_len % bs == 1``, which never allocates when block_size == 1); a prefill
of 0 tokens creates a live empty sequence; sequence ids are non-negative;
a shared prefix shares ceil(n / bs) blocks, its partial last block
included, as [impl-detail]'s ``share_prefix_blocks`` does; the copy takes
the whole block.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


class ManagerError(Exception):
    """Base of all manager errors.  Any error leaves the state unchanged."""


class InvalidArgument(ManagerError, ValueError):
    pass


class OutOfBlocks(ManagerError, RuntimeError):
    def __init__(self, msg: str = "OOM"):
        super().__init__(msg)


class NotLive(ManagerError, ValueError):
    """Unknown or already-freed sequence (covers double free)."""


class AlreadyPrefilled(ManagerError, ValueError):
    pass


def blocks_needed(num_tokens: int, block_size: int) -> int:
    """ceil(num_tokens / block_size) ([MiniPaged-Qwen] §4.3;
    [mini-vLLM BM] "prefill 时如何分配 block")."""
    return -(-num_tokens // block_size)


class _Seq:
    __slots__ = ("length", "table")

    def __init__(self):
        self.length = 0          # tokens written so far == next write position
        self.table: List[int] = []


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int,
                 initial_free_order: Optional[Sequence[int]] = None,
                 sort_on_release: bool = False):
        if num_blocks <= 0 or block_size <= 0:
            raise InvalidArgument("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        if initial_free_order is None:
            self.free: List[int] = list(range(self.num_blocks))
        else:
            order = [int(x) for x in initial_free_order]
            if sorted(order) != list(range(self.num_blocks)):
                raise InvalidArgument("initial free order must be a permutation of 0..N-1")
            self.free = order
        self.sort_on_release = bool(sort_on_release)
        self.seqs: Dict[int, _Seq] = {}
        self.ref: List[int] = [0] * self.num_blocks      # tables holding each block
        self.swapped: Dict[int, int] = {}                # swapped-out sequence -> length
        self.copies: List[Tuple[int, int]] = []          # queued (source, destination)

    # -- queries -----------------------------------------------------------
    def num_free_blocks(self) -> int:
        return len(self.free)

    def can_allocate(self, num_tokens: int) -> bool:
        """Enough free blocks for a prefill of ``num_tokens``
        ([mini-vLLM BM] "prefill 时如何分配 block", can_allocate)."""
        if num_tokens < 0:
            raise InvalidArgument("num_tokens must be >= 0")
        return blocks_needed(num_tokens, self.block_size) <= len(self.free)

    def is_live(self, seq_id: int) -> bool:
        return seq_id in self.seqs

    def block_table(self, seq_id: int) -> List[int]:
        return list(self._live(seq_id).table)

    def context_len(self, seq_id: int) -> int:
        return self._live(seq_id).length

    def block_tables(self, seq_ids: Sequence[int], width: int, pad: int = -1) -> np.ndarray:
        """Batch block-table tensor padded with ``pad`` ([MiniPaged-Qwen] §16.5)."""
        out = np.full((len(seq_ids), width), pad, dtype=np.int32)
        for row, sid in enumerate(seq_ids):
            table = self._live(sid).table
            if len(table) > width:
                raise InvalidArgument("table wider than requested width")
            out[row, :len(table)] = table
        return out

    def context_lens(self, seq_ids: Sequence[int]) -> np.ndarray:
        """Per-sequence lengths ([MiniPaged-Qwen] §16.6)."""
        return np.array([self._live(s).length for s in seq_ids], dtype=np.int32)

    def ref_count(self, block: int) -> int:
        """Number of tables holding ``block`` ([impl-detail] "块池" ref_count)."""
        if block < 0 or block >= self.num_blocks:
            raise InvalidArgument("block id out of range")
        return self.ref[block]

    def take_copies(self) -> List[Tuple[int, int]]:
        """The queued copy-on-write pairs (source, destination), oldest first;
        the queue is left empty."""
        out, self.copies = self.copies, []
        return out

    # -- operations --------------------------------------------------------
    def allocate_for_prefill(self, seq_id: int, num_tokens: int) -> List[int]:
        """Create ``seq_id`` with ``num_tokens`` prompt tokens and return their
        slots, token t at block_table[t // bs], offset t % bs
        ([mini-vLLM BM] "Block Manager 和 ModelRunner 如何协作")."""
        if seq_id < 0 or num_tokens < 0:
            raise InvalidArgument("seq_id and num_tokens must be >= 0")
        if seq_id in self.seqs or seq_id in self.swapped:
            raise AlreadyPrefilled(f"sequence {seq_id} is already live")
        need = blocks_needed(num_tokens, self.block_size)
        if need > len(self.free):
            raise OutOfBlocks()
        seq = _Seq()
        seq.table = self.free[:need]
        del self.free[:need]
        for pb in seq.table:
            self.ref[pb] = 1
        seq.length = num_tokens
        self.seqs[seq_id] = seq
        bs = self.block_size
        return [seq.table[t // bs] * bs + t % bs for t in range(num_tokens)]

    def share_prefix(self, donor_id: int, seq_id: int, num_tokens: int) -> None:
        """Create ``seq_id`` holding the first ``num_tokens`` tokens of live
        ``donor_id`` without copying: its table is the donor's first
        ceil(num_tokens / bs) blocks, each block's count + 1
        ([impl-detail] "前缀共享", share_prefix_blocks)."""
        if seq_id < 0 or num_tokens < 0:
            raise InvalidArgument("seq_id and num_tokens must be >= 0")
        donor = self._live(donor_id)
        if seq_id in self.seqs or seq_id in self.swapped:
            raise AlreadyPrefilled(f"sequence {seq_id} is already live")
        if num_tokens > donor.length:
            raise InvalidArgument("shared prefix longer than the donor")
        seq = _Seq()
        seq.table = donor.table[:blocks_needed(num_tokens, self.block_size)]
        for pb in seq.table:
            self.ref[pb] += 1
        seq.length = num_tokens
        self.seqs[seq_id] = seq

    def append_slot_for_decode(self, seq_id: int) -> int:
        """Slot of position len(seq); allocates one front block exactly when
        that position opens a new logical block; then len += 1
        ([MiniPaged-Qwen] §9, §9.1-§9.3)."""
        seq = self._live(seq_id)
        L = seq.length
        logical_block = L // self.block_size
        block_offset = L % self.block_size
        if logical_block == len(seq.table):
            if not self.free:
                raise OutOfBlocks()
            new = self.free.pop(0)
            self.ref[new] = 1
            seq.table.append(new)
        elif self.ref[seq.table[logical_block]] > 1:
            # the token lands in a block other tables hold: copy on write
            if not self.free:
                raise OutOfBlocks()
            old = seq.table[logical_block]
            new = self.free.pop(0)
            self.ref[old] -= 1
            self.ref[new] = 1
            seq.table[logical_block] = new
            self.copies.append((old, new))
        physical_block = seq.table[logical_block]
        seq.length = L + 1
        return physical_block * self.block_size + block_offset

    def append_slots_for_decode(self, seq_ids: Sequence[int]) -> List[int]:
        """Batched append, all or nothing: the blocks this round needs are
        counted first and the whole call fails with no change when the free
        list is short ([mini-vLLM BM] "Block Manager 和 Scheduler 如何协作")."""
        ids = [int(s) for s in seq_ids]
        if len(set(ids)) != len(ids):
            raise InvalidArgument("duplicate sequence ids in one append")
        for s in ids:
            self._live(s)
        # blocks this call takes: one per opened block, one per copy on
        # write, counting the references earlier copies in the call drop
        need = 0
        dropped: Dict[int, int] = {}
        for s in ids:
            seq = self.seqs[s]
            lb = seq.length // self.block_size
            if lb == len(seq.table):
                need += 1
            else:
                pb = seq.table[lb]
                if self.ref[pb] - dropped.get(pb, 0) > 1:
                    need += 1
                    dropped[pb] = dropped.get(pb, 0) + 1
        if need > len(self.free):
            raise OutOfBlocks()
        return [self.append_slot_for_decode(s) for s in ids]

    def append_tokens(self, seq_id: int, num_tokens: int) -> List[int]:
        """Slots of ``num_tokens`` new tokens at positions len .. len + n - 1
        (a prefill chunk of a live sequence), all or nothing: the blocks the
        n appends take (opened blocks, and a copy of a shared tail block) are
        counted first; then each token is appended as append_slot_for_decode
        does ([MiniPaged-Qwen] §9; [mini-vLLM BM] "prefill 时如何分配 block")."""
        seq = self._live(seq_id)
        if num_tokens < 0:
            raise InvalidArgument("num_tokens must be >= 0")
        L, bs = seq.length, self.block_size
        need = blocks_needed(L + num_tokens, bs) - len(seq.table)
        if num_tokens > 0 and L // bs < len(seq.table) and self.ref[seq.table[L // bs]] > 1:
            need += 1
        if need > len(self.free):
            raise OutOfBlocks()
        return [self.append_slot_for_decode(seq_id) for _ in range(num_tokens)]

    def admit_batch(self, seq_ids: Sequence[int], chunk_lens: Sequence[int],
                    extend_live: bool = False) -> List[List[int]]:
        """A batch of prefill chunks admitted all or nothing ([mini-vLLM BM]
        "Block Manager 和 Scheduler 如何协作": the scheduler admits only what
        the free blocks cover).  Sequence seq_ids[i] gets chunk_lens[i]
        tokens, in array order: a sequence not live is created as
        allocate_for_prefill creates it; a live one is extended as
        append_tokens extends it, when ``extend_live``.  Everything is
        checked before anything changes: ids >= 0 and distinct, lengths
        >= 0, no swapped id, no live id unless ``extend_live``, and the
        blocks of the whole batch (new tables, opened blocks, and a copy of
        each shared tail block a chunk writes into, counting the references
        earlier copies of the batch drop) against the free list.  Returns
        each sequence's slots."""
        ids = [int(x) for x in seq_ids]
        lens = [int(x) for x in chunk_lens]
        if len(ids) != len(lens):
            raise InvalidArgument("one chunk length per sequence")
        if any(x < 0 for x in ids) or any(n < 0 for n in lens):
            raise InvalidArgument("seq_ids and chunk lengths must be >= 0")
        if len(set(ids)) != len(ids):
            raise InvalidArgument("duplicate sequence ids in one batch")
        bs = self.block_size
        need = 0
        dropped: Dict[int, int] = {}
        for sid, n in zip(ids, lens):
            if sid in self.swapped or (sid in self.seqs and not extend_live):
                raise AlreadyPrefilled(f"sequence {sid} is already live")
            if sid not in self.seqs:
                need += blocks_needed(n, bs)
                continue
            seq = self.seqs[sid]
            L = seq.length
            need += blocks_needed(L + n, bs) - len(seq.table)
            if n > 0 and L // bs < len(seq.table):
                tail = seq.table[L // bs]
                if self.ref[tail] - dropped.get(tail, 0) > 1:
                    need += 1
                    dropped[tail] = dropped.get(tail, 0) + 1
        if need > len(self.free):
            raise OutOfBlocks()
        return [self.append_tokens(sid, n) if sid in self.seqs else self.allocate_for_prefill(sid, n)
                for sid, n in zip(ids, lens)]

    def swap_out(self, seq_id: int) -> List[int]:
        """Release the blocks of live ``seq_id`` (returned in table order, for
        the caller to copy out first) and keep its length; the sequence is
        then swapped, not live ([impl-detail] "异构内存支持" evict_to_cpu)."""
        seq = self._live(seq_id)
        if any(self.ref[pb] > 1 for pb in seq.table):
            raise InvalidArgument("a sequence holding a shared block cannot be swapped out")
        table = list(seq.table)
        for pb in table:
            self.ref[pb] = 0
            self.free.append(pb)
        if self.sort_on_release:
            self.free.sort()
        self.swapped[int(seq_id)] = seq.length
        del self.seqs[int(seq_id)]
        return table

    def swap_in(self, seq_id: int) -> List[int]:
        """Make swapped ``seq_id`` live again on ceil(len / bs) blocks from the
        front of the free list, all or nothing; returns its new table (for the
        caller to copy back into, [impl-detail] "异构内存支持" prefetch_to_gpu)."""
        seq_id = int(seq_id)
        if seq_id in self.seqs:
            raise AlreadyPrefilled(f"sequence {seq_id} is live")
        if seq_id not in self.swapped:
            raise NotLive(f"sequence {seq_id} is not swapped out")
        L = self.swapped[seq_id]
        need = blocks_needed(L, self.block_size)
        if need > len(self.free):
            raise OutOfBlocks()
        seq = _Seq()
        seq.table = self.free[:need]
        del self.free[:need]
        for pb in seq.table:
            self.ref[pb] = 1
        seq.length = L
        self.seqs[seq_id] = seq
        del self.swapped[seq_id]
        return list(seq.table)

    def free_sequence(self, seq_id: int) -> None:
        """Return every block of ``seq_id`` to the free list exactly once
        ([MiniPaged-Qwen] §5.3; [mini-vLLM BM] "释放 block").  A swapped-out
        sequence holds no blocks and is just forgotten."""
        if int(seq_id) in self.swapped:
            del self.swapped[int(seq_id)]
            return
        seq = self._live(seq_id)
        for pb in seq.table:
            self.ref[pb] -= 1
            if self.ref[pb] == 0:
                self.free.append(pb)
        if self.sort_on_release:
            self.free.sort()
        del self.seqs[seq_id]

    # -- invariants --------------------------------------------------------
    def check_invariants(self) -> List[str]:
        """Names of violated invariants (empty when all hold).

        I1 no physical id twice in one table, and each block's count equals
        the number of tables holding it (without sharing: no id in two
        tables); I2 tables and free list disjoint, free blocks count 0;
        I3 |distinct allocated| + |free| == N; I4 ids in [0, N);
        I5 len(table) == ceil(len / bs); I6 free list has no duplicates
        ([MiniPaged-Qwen] §15; [mini-vLLM BM] "正确性不变量";
        [leetcode-22] Step 3 table; [impl-detail] "Copy-on-Write共享").
        """
        bad = []
        allocated = [pb for s in self.seqs.values() for pb in s.table]
        holders: Dict[int, int] = {}
        for pb in allocated:
            holders[pb] = holders.get(pb, 0) + 1
        if any(len(s.table) != len(set(s.table)) for s in self.seqs.values()) or \
                any(self.ref[pb] != n for pb, n in holders.items()
                    if 0 <= pb < self.num_blocks):
            bad.append("I1")
        if set(allocated) & set(self.free) or \
                any(self.ref[pb] != 0 for pb in self.free if 0 <= pb < self.num_blocks):
            bad.append("I2")
        if len(holders) + len(self.free) != self.num_blocks:
            bad.append("I3")
        if any(pb < 0 or pb >= self.num_blocks for pb in allocated + self.free):
            bad.append("I4")
        if any(len(s.table) != blocks_needed(s.length, self.block_size)
               for s in self.seqs.values()):
            bad.append("I5")
        if len(self.free) != len(set(self.free)):
            bad.append("I6")
        return bad

    # -- helpers -----------------------------------------------------------
    def _live(self, seq_id: int) -> _Seq:
        seq = self.seqs.get(int(seq_id))
        if seq is None:
            raise NotLive(f"sequence {seq_id} is not live")
        return seq
