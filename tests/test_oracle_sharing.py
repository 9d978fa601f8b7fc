"""Pins of the oracle's prefix sharing and copy-on-write ([impl-detail]
"Copy-on-Write共享": share_prefix_blocks and copy_on_write) against a small
example worked by hand from those rules, against the invariants (with a
mistake planted in a copy of the oracle to show they catch it), and against
the data-level property copy-on-write exists for: a sequence's write never
changes what another sequence reads.  CPU only."""
import numpy as np
import pytest

import oracle
import synth
from oracle.manager import BlockManager


def _checked(m):
    assert m.check_invariants() == []
    return m


def test_share_then_copy_on_write_worked_by_hand():
    # N = 8, bs = 4, free list 0..7.  Sequence 0 holds 10 tokens in blocks
    # [0, 1, 2] (block 2 half full); sequence 1 shares that whole prefix.
    m = BlockManager(8, 4)
    m.allocate_for_prefill(0, 10)
    m.share_prefix(0, 1, 10)
    _checked(m)
    assert m.block_table(1) == [0, 1, 2] and m.context_len(1) == 10
    assert [m.ref_count(b) for b in range(4)] == [2, 2, 2, 0]
    assert m.take_copies() == []
    # Sequence 1's token 10 lands at offset 2 of shared block 2: it takes
    # block 3 (front of the free list), block 2 is copied into it, block 2
    # keeps one holder.
    assert m.append_slot_for_decode(1) == 3 * 4 + 2
    assert m.block_table(1) == [0, 1, 3] and m.block_table(0) == [0, 1, 2]
    assert [m.ref_count(b) for b in range(5)] == [2, 2, 1, 1, 0]
    assert m.take_copies() == [(2, 3)] and m.take_copies() == []
    # Sequence 0 now holds block 2 alone: it writes in place, no copy.
    assert m.append_slot_for_decode(0) == 2 * 4 + 2
    assert m.take_copies() == []
    assert m.free == [4, 5, 6, 7]
    # Sequence 1 fills block 3, then opens block 4.
    assert m.append_slot_for_decode(1) == 3 * 4 + 3
    assert m.append_slot_for_decode(1) == 4 * 4
    assert m.block_table(1) == [0, 1, 3, 4]
    _checked(m)
    # Freeing sequence 0 releases only the block nobody else holds.
    m.free_sequence(0)
    assert m.free == [5, 6, 7, 2]
    assert [m.ref_count(b) for b in range(5)] == [1, 1, 0, 1, 1]
    m.free_sequence(1)
    assert m.free == [5, 6, 7, 2, 0, 1, 3, 4]
    _checked(m)


def test_block_aligned_prefix_needs_no_copy():
    m = BlockManager(8, 4)
    m.allocate_for_prefill(0, 8)
    m.share_prefix(0, 1, 8)
    assert m.append_slot_for_decode(1) == 2 * 4      # opens block 2
    assert m.append_slot_for_decode(0) == 3 * 4      # opens block 3
    assert m.take_copies() == []
    assert m.block_table(0)[:2] == m.block_table(1)[:2] == [0, 1]
    _checked(m)


def test_shorter_prefix_and_empty_prefix():
    m = BlockManager(8, 4)
    m.allocate_for_prefill(0, 10)
    m.share_prefix(0, 1, 5)                          # blocks 0 and 1 (token 4 in block 1)
    assert m.block_table(1) == [0, 1] and m.context_len(1) == 5
    assert m.append_slot_for_decode(1) == 3 * 4 + 1  # position 5 lands in shared block 1
    assert m.take_copies() == [(1, 3)]
    m.share_prefix(0, 2, 0)
    assert m.block_table(2) == [] and m.context_len(2) == 0
    assert m.append_slot_for_decode(2) == 4 * 4
    _checked(m)


def test_share_errors_change_nothing():
    m = BlockManager(4, 4)
    m.allocate_for_prefill(0, 6)
    before = (list(m.free), m.block_table(0), list(m.ref))
    with pytest.raises(oracle.NotLive):
        m.share_prefix(9, 1, 2)
    with pytest.raises(oracle.AlreadyPrefilled):
        m.share_prefix(0, 0, 2)
    with pytest.raises(oracle.InvalidArgument):
        m.share_prefix(0, 1, 7)
    with pytest.raises(oracle.InvalidArgument):
        m.share_prefix(0, -1, 2)
    assert (list(m.free), m.block_table(0), list(m.ref)) == before
    assert not m.is_live(1)


def test_copy_on_write_out_of_blocks_is_atomic():
    m = BlockManager(2, 4)
    m.allocate_for_prefill(0, 6)                     # blocks 0, 1: pool exhausted
    m.share_prefix(0, 1, 6)
    state = (m.block_table(0), m.block_table(1), list(m.ref), list(m.free))
    with pytest.raises(oracle.OutOfBlocks):
        m.append_slot_for_decode(1)
    with pytest.raises(oracle.OutOfBlocks):
        m.append_slots_for_decode([0, 1])
    assert (m.block_table(0), m.block_table(1), list(m.ref), list(m.free)) == state
    assert m.context_len(0) == m.context_len(1) == 6 and m.take_copies() == []


def test_batched_append_counts_copies_in_order():
    # Two sharers of half-full block 1 in one batch: the first copies, which
    # leaves the second the only holder, so it writes in place.
    m = BlockManager(3, 4)
    m.allocate_for_prefill(0, 6)
    m.share_prefix(0, 1, 6)
    slots = m.append_slots_for_decode([1, 0])
    assert slots == [2 * 4 + 2, 1 * 4 + 2]
    assert m.take_copies() == [(1, 2)]
    # One free block short of two copies: three sharers, none free.
    m2 = BlockManager(3, 4)
    m2.allocate_for_prefill(0, 6)
    m2.share_prefix(0, 1, 6)
    m2.share_prefix(0, 2, 6)
    m2.allocate_for_prefill(3, 1)                   # takes the last free block
    with pytest.raises(oracle.OutOfBlocks):
        m2.append_slots_for_decode([0, 1, 2])
    _checked(m2)


@pytest.mark.parametrize("seed,n_blocks,bs", [(31, 40, 4), (32, 12, 1), (33, 64, 16), (34, 25, 3)])
def test_random_share_traces_keep_invariants(seed, n_blocks, bs):
    m = BlockManager(n_blocks, bs, np.random.default_rng(seed).permutation(n_blocks))
    for op in synth.manager_share_trace(seed, 2000):
        try:
            if op[0] == "prefill":
                m.allocate_for_prefill(op[1], op[2])
            elif op[0] == "share":
                m.share_prefix(op[1], op[2], op[3])
            elif op[0] == "append":
                slot = m.append_slot_for_decode(op[1])
                assert m.ref_count(slot // bs) == 1      # a write never lands in a shared block
            elif op[0] == "append_batch":
                for slot in m.append_slots_for_decode(list(op[1])):
                    assert m.ref_count(slot // bs) == 1
            elif op[0] == "free":
                m.free_sequence(op[1])
            else:
                m.can_allocate(op[1])
        except oracle.ManagerError:
            pass
        m.take_copies()
        assert m.check_invariants() == []
        assert sum(m.ref) == sum(len(s.table) for s in m.seqs.values())


class _ForgetsToRelease(BlockManager):
    """A planted mistake: release drops only the first reference."""

    def free_sequence(self, seq_id):
        seq = self._live(seq_id)
        for i, pb in enumerate(seq.table):
            if i == 0:
                self.ref[pb] -= 1
            if self.ref[pb] == 0:
                self.free.append(pb)
        del self.seqs[seq_id]


class _CopiesWithoutDrop(BlockManager):
    """A planted mistake: copy-on-write leaves the shared block's count."""

    def append_slot_for_decode(self, seq_id):
        seq = self._live(seq_id)
        lb = seq.length // self.block_size
        if lb < len(seq.table) and self.ref[seq.table[lb]] > 1:
            self.ref[seq.table[lb]] += 1                 # undone by the real path below
        return super().append_slot_for_decode(seq_id)


@pytest.mark.parametrize("bad", [_ForgetsToRelease, _CopiesWithoutDrop])
def test_invariants_catch_planted_mistakes(bad):
    m = bad(8, 4)
    m.allocate_for_prefill(0, 10)
    m.share_prefix(0, 1, 10)
    m.append_slot_for_decode(1)
    m.free_sequence(0)
    assert m.check_invariants() != []


def test_copy_on_write_isolates_sequences():
    """After a copy on write each sequence reads its own tokens: the sharer's
    write shows in its own gather and not in the donor's, and the shared
    positions read alike in both."""
    rng = np.random.default_rng(7)
    N, H, bs, D = 6, 2, 4, 8
    m = BlockManager(N, bs)
    kc, vc = oracle.new_pool(N, H, bs, D, synth.poison_array((), "f32"))
    slots = m.allocate_for_prefill(0, 6)
    k0 = rng.standard_normal((6, H, D)).astype(np.float32)
    v0 = rng.standard_normal((6, H, D)).astype(np.float32)
    oracle.write_kv(k0, v0, slots, kc, vc, bs)
    m.share_prefix(0, 1, 6)
    s1 = m.append_slot_for_decode(1)
    oracle.copy_blocks(m.take_copies(), kc, vc)
    k1 = rng.standard_normal((1, H, D)).astype(np.float32)
    v1 = rng.standard_normal((1, H, D)).astype(np.float32)
    oracle.write_kv(k1, v1, [s1], kc, vc, bs)
    s0 = m.append_slot_for_decode(0)
    k2 = rng.standard_normal((1, H, D)).astype(np.float32)
    oracle.write_kv(k2, k2, [s0], kc, vc, bs)
    g0 = oracle.gather_logical(kc, m.block_table(0), 7)
    g1 = oracle.gather_logical(kc, m.block_table(1), 7)
    v1g = oracle.gather_logical(vc, m.block_table(1), 7)
    assert np.array_equal(g0[:, :6], k0.transpose(1, 0, 2))
    assert np.array_equal(g1[:, :6], k0.transpose(1, 0, 2))
    assert np.array_equal(v1g[:, :6], v0.transpose(1, 0, 2))
    assert np.array_equal(g1[:, 6], k1[0]) and np.array_equal(v1g[:, 6], v1[0])
    assert np.array_equal(g0[:, 6], k2[0])
