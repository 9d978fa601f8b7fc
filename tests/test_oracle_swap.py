"""Pins of the oracle's swap to host ([impl-detail] "异构内存支持"
evict_to_cpu / prefetch_to_gpu): a worked-by-hand example (released ids,
free-list order, atomic OOM on swap-in, the new table), the error cases, and
the data round trip through gather / scatter; plus C++ parity on random
traces with swaps.  CPU only."""
import numpy as np
import pytest

import oracle
import synth
import paged_kv_cache_128_amd as pkv
from oracle.manager import BlockManager


def test_swap_worked_by_hand():
    m = BlockManager(8, 4)
    m.allocate_for_prefill(0, 10)              # blocks 0, 1, 2
    m.allocate_for_prefill(1, 5)               # blocks 3, 4
    assert m.swap_out(0) == [0, 1, 2]
    assert m.free == [5, 6, 7, 0, 1, 2] and not m.is_live(0)
    with pytest.raises(oracle.NotLive):
        m.append_slot_for_decode(0)
    with pytest.raises(oracle.AlreadyPrefilled):
        m.allocate_for_prefill(0, 3)
    m.allocate_for_prefill(2, 16)              # blocks 5, 6, 7, 0
    with pytest.raises(oracle.OutOfBlocks):    # needs 3, two free: stays swapped
        m.swap_in(0)
    assert m.free == [1, 2] and 0 in m.swapped
    m.free_sequence(2)
    assert m.free == [1, 2, 5, 6, 7, 0]
    assert m.swap_in(0) == [1, 2, 5]
    assert m.context_len(0) == 10 and m.block_table(0) == [1, 2, 5]
    assert m.append_slot_for_decode(0) == 5 * 4 + 2
    assert m.check_invariants() == []
    with pytest.raises(oracle.AlreadyPrefilled):
        m.swap_in(0)
    with pytest.raises(oracle.NotLive):
        m.swap_in(7)


def test_shared_sequences_do_not_swap_and_swapped_ones_free():
    m = BlockManager(8, 4)
    m.allocate_for_prefill(0, 6)
    m.share_prefix(0, 1, 6)
    with pytest.raises(oracle.InvalidArgument):
        m.swap_out(1)
    assert m.is_live(1) and m.ref_count(0) == 2
    m.free_sequence(1)
    m.swap_out(0)
    m.free_sequence(0)                         # forgets the swapped sequence
    with pytest.raises(oracle.NotLive):
        m.swap_in(0)
    assert len(m.free) == 8 and m.check_invariants() == []


def test_swap_round_trip_restores_the_data():
    rng = np.random.default_rng(3)
    N, H, bs, D = 10, 2, 4, 8
    m = BlockManager(N, bs, rng.permutation(N))
    kc, vc = oracle.new_pool(N, H, bs, D, synth.poison_array((), "bf16"))
    k = synth.normal(rng, (13, H, D), "bf16")
    v = synth.normal(rng, (13, H, D), "bf16")
    oracle.write_kv(k, v, m.allocate_for_prefill(0, 13), kc, vc, bs)
    before_k = oracle.gather_logical(kc, m.block_table(0), 13).copy()
    before_v = oracle.gather_logical(vc, m.block_table(0), 13).copy()
    staged = oracle.gather_blocks(m.swap_out(0), kc, vc)
    # another sequence overwrites the released blocks
    slots = m.allocate_for_prefill(1, 4 * 9)
    oracle.write_kv(synth.normal(rng, (36, H, D), "bf16"), synth.normal(rng, (36, H, D), "bf16"),
                    slots, kc, vc, bs)
    m.free_sequence(1)
    ids = m.swap_in(0)
    oracle.scatter_blocks(staged, ids, kc, vc)
    assert np.array_equal(oracle.gather_logical(kc, ids, 13), before_k)
    assert np.array_equal(oracle.gather_logical(vc, ids, 13), before_v)


def test_gather_blocks_layout_pinned_to_the_written_rows():
    """16-bit / fp32 swap staging, pinned to the rows that went in rather than
    to scatter_blocks: entry j of the staged array is [2, H, bs, D] with
    index 0 the K rows and index 1 the V rows of block ids[j] (the staging
    layout the C header states), token t of the prompt at block
    table[t // bs], row t % bs.  K and V carry different values (V = -K - 1),
    so swapped halves, a transposed head / row axis or a wrong block order
    all fail."""
    N, H, bs, D, n = 6, 2, 4, 8, 10
    m = BlockManager(N, bs, [4, 1, 5, 0, 3, 2])
    kc, vc = oracle.new_pool(N, H, bs, D, np.array(np.nan, dtype=np.float32))
    t_, h_, d_ = np.meshgrid(np.arange(n), np.arange(H), np.arange(D), indexing="ij")
    k = (1000.0 * t_ + 100.0 * h_ + d_).astype(np.float32)        # [n, H, D]
    v = -k - 1.0
    oracle.write_kv(k, v, m.allocate_for_prefill(0, n), kc, vc, bs)
    table = m.block_table(0)
    assert table == [4, 1, 5]
    ids = [5, 4, 1]
    staged = oracle.gather_blocks(ids, kc, vc)
    assert staged.shape == (3, 2, H, bs, D)
    for j, blk in enumerate(ids):
        lb = table.index(blk)
        for off in range(bs):
            t = lb * bs + off
            for h in range(H):
                if t < n:
                    assert np.array_equal(staged[j, 0, h, off], k[t, h]), (j, off, h)
                    assert np.array_equal(staged[j, 1, h, off], v[t, h]), (j, off, h)
                else:                                  # block 5's unused tail: untouched poison
                    assert np.all(np.isnan(staged[j, :, h, off]))
    assert oracle.gather_blocks([], kc, vc).shape == (0, 2, H, bs, D)


@pytest.mark.parametrize("seed,n_blocks,bs,sort", [(61, 30, 4, False), (62, 12, 1, True), (63, 20, 16, False)])
def test_swap_traces_match_c_manager(seed, n_blocks, bs, sort):
    rng = np.random.default_rng(seed)
    o = oracle.BlockManager(n_blocks, bs, sort_on_release=sort)
    c = pkv.KVBlockManager(n_blocks, bs, sort_on_release=sort)
    errs = {oracle.InvalidArgument: pkv.InvalidArgumentError, oracle.OutOfBlocks: pkv.OutOfBlocksError,
            oracle.NotLive: pkv.NotLiveError, oracle.AlreadyPrefilled: pkv.AlreadyPrefilledError}

    def run(mgr, op):
        try:
            name, args = op[0], op[1:]
            if name == "append":
                return ("ok", int(mgr.append_slot_for_decode(*args)))
            if name == "prefill":
                return ("ok", [int(x) for x in mgr.allocate_for_prefill(*args)])
            if name == "share":
                mgr.share_prefix(*args)
                return ("ok", None)
            if name == "free":
                mgr.free_sequence(*args)
                return ("ok", None)
            return ("ok", [int(x) for x in getattr(mgr, name)(*args)])
        except (oracle.ManagerError, pkv.PkvError) as e:
            return ("err", next(k.__name__ for k, v in errs.items() if isinstance(e, (k, v))))

    kinds = set()
    for _ in range(1500):
        u = rng.random()
        sid = int(rng.integers(10))
        if u < 0.2:
            op = ("prefill", sid, int(rng.integers(0, 14)))
        elif u < 0.3:
            op = ("share", int(rng.integers(10)), sid, int(rng.integers(0, 10)))
        elif u < 0.55:
            op = ("append", sid)
        elif u < 0.7:
            op = ("swap_out", sid)
        elif u < 0.85:
            op = ("swap_in", sid)
        else:
            op = ("free", sid)
        ro, rc = run(o, op), run(c, op)
        assert ro == rc, (op, ro, rc)
        o.take_copies()
        c.take_copies()
        kinds.add((op[0], ro[0]))
        assert c.free_list() == o.free and c.check_invariants() and o.check_invariants() == []
        for s in range(10):
            assert c.is_swapped(s) == (s in o.swapped)
    assert ("swap_out", "ok") in kinds and ("swap_in", "ok") in kinds
