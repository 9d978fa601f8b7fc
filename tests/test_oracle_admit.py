"""Pins of the oracle's all-or-nothing batch admission ([mini-vLLM BM]
"Block Manager 和 Scheduler 如何协作": a batch is admitted only when the
free blocks cover all of it), worked by hand.  CPU only."""
import pytest

import oracle
from oracle.manager import BlockManager


def test_batch_that_fits_equals_the_calls_one_by_one():
    m = BlockManager(8, 4)
    slots = m.admit_batch([0, 1, 2], [5, 3, 9])              # 2 + 1 + 3 blocks from the front
    assert [m.block_table(s) for s in (0, 1, 2)] == [[0, 1], [2], [3, 4, 5]]
    assert slots == [[0, 1, 2, 3, 4], [8, 9, 10], [12, 13, 14, 15, 16, 17, 18, 19, 20]]
    assert m.free == [6, 7]
    ref = BlockManager(8, 4)
    assert [ref.allocate_for_prefill(0, 5), ref.allocate_for_prefill(1, 3),
            ref.allocate_for_prefill(2, 9)] == slots
    assert ref.free == m.free


def test_kth_sequence_out_of_blocks_changes_nothing():
    m = BlockManager(8, 4)
    m.allocate_for_prefill(0, 20)                              # blocks 0..4, free [5, 6, 7]
    with pytest.raises(oracle.OutOfBlocks):                    # 1 + 3 > 3 free: the second does not fit
        m.admit_batch([1, 2], [4, 9])
    assert m.free == [5, 6, 7] and not m.is_live(1) and not m.is_live(2)
    with pytest.raises(oracle.AlreadyPrefilled):               # live id without extend_live
        m.admit_batch([3, 0], [1, 1])
    assert not m.is_live(3)
    with pytest.raises(oracle.InvalidArgument):                # repeated id
        m.admit_batch([3, 3], [1, 1])
    assert m.check_invariants() == []


def test_extension_counts_opened_blocks_and_one_copy_per_shared_tail():
    m = BlockManager(8, 4)
    m.allocate_for_prefill(0, 6)                               # table [0, 1], tail block 1 half full
    m.share_prefix(0, 1, 6)                                    # block 1 now held twice
    # seq 0 writes into the shared tail (copy: block 2) and opens one more
    # (block 3); seq 1 then holds block 1 alone, so its chunk copies nothing
    # and opens block 4; a new sequence takes block 5
    slots = m.admit_batch([0, 1, 7], [3, 3, 2], extend_live=True)
    assert m.block_table(0) == [0, 2, 3] and m.block_table(1) == [0, 1, 4] and m.block_table(7) == [5]
    assert m.take_copies() == [(1, 2)]
    assert slots == [[2 * 4 + 2, 2 * 4 + 3, 3 * 4 + 0], [1 * 4 + 2, 1 * 4 + 3, 4 * 4 + 0], [20, 21]]
    assert m.free == [6, 7]
    # the same batch with one free block too few fails whole
    m2 = BlockManager(5, 4)
    m2.allocate_for_prefill(0, 6)
    m2.share_prefix(0, 1, 6)
    with pytest.raises(oracle.OutOfBlocks):                    # needs 2 + 1 + 1 = 4, three free
        m2.admit_batch([0, 1, 7], [3, 3, 2], extend_live=True)
    assert m2.free == [2, 3, 4] and m2.context_len(0) == 6 and m2.context_len(1) == 6
    assert m2.ref_count(1) == 2 and m2.take_copies() == []
