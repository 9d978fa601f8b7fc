"""Pins of the oracle's block manager, slot map, write, gather and ledger
against the values the pages print (tests/golden/worked_examples.json) and
against invariants.  CPU only."""
import numpy as np
import pytest

import oracle
import synth
from oracle.manager import BlockManager, blocks_needed


def _mgr_with_front(n, bs, front, **kw):
    rest = [i for i in range(n) if i not in front]
    return BlockManager(n, bs, list(front) + rest, **kw)


def test_address_translation_worked_example(golden):
    g = golden["address_translation"]
    bs, table = g["block_size"], g["block_table"]
    assert oracle.slot_of(table, g["token_pos"], bs) == g["slot"]
    assert oracle.split_slot(g["slot"], bs) == (g["physical_block"], g["block_offset"])
    rows = g["position_rows"]
    for pos, lb, off in zip(rows["token_pos"], rows["logical_block"], rows["block_offset"]):
        slot = oracle.slot_of(table, pos, bs)
        assert oracle.split_slot(slot, bs) == (table[lb], off)


def test_append_token_walk(golden):
    g = golden["append_token_walk"]
    bs = g["block_size"]
    m = _mgr_with_front(16, bs, g["table_before"] + [g["new_block"]])
    m.allocate_for_prefill(7, 7)
    assert m.block_table(7) == g["table_before"]
    s7 = m.append_slot_for_decode(7)             # position 7
    assert oracle.split_slot(s7, bs) == (g["table_before"][g["len7"]["logical_block"]],
                                          g["len7"]["block_offset"])
    assert m.block_table(7) == g["table_before"]  # no allocation
    s8 = m.append_slot_for_decode(7)             # position 8 opens logical block 2
    assert m.block_table(7) == g["len8"]["table_after"]
    assert s8 == g["len8"]["slot"]
    assert m.context_len(7) == 9


def test_block_counts_and_waste(golden):
    g = golden["block_counts"]
    bs = g["block_size"]
    assert blocks_needed(7, bs) == g["len7_blocks"]
    assert blocks_needed(10, bs) == g["len10_blocks"]
    assert 10 - (g["len10_blocks"] - 1) * bs == g["len10_last_used"]
    assert oracle.tail_waste(10, bs) == g["len10_waste"]
    assert oracle.tail_waste(8, bs) == 0


def test_prefill_example(golden):
    g = golden["prefill_example"]
    bs = g["block_size"]
    m = _mgr_with_front(16, bs, g["free_before"])
    slots = m.allocate_for_prefill(0, g["prompt"])
    assert m.block_table(0) == g["table"]
    assert m.free[:2] == g["free_after"]
    assert len(m.block_table(0)) == g["blocks"]
    assert g["prompt"] - (g["blocks"] - 1) * bs == g["last_block_used"]
    assert oracle.split_slot(slots[39], bs) == (g["token39"]["block"], g["token39"]["offset"])
    assert oracle.split_slot(slots[15], bs) == (g["token15"]["block"], g["token15"]["offset"])
    assert oracle.split_slot(slots[16], bs) == (g["token16"]["block"], g["token16"]["offset"])


def test_decode_growth(golden):
    g = golden["decode_growth"]
    bs = g["block_size"]
    m = BlockManager(64, bs)
    m.allocate_for_prefill(1, g["len"])
    t = m.block_table(1)
    s40 = m.append_slot_for_decode(1)
    assert oracle.split_slot(s40, bs) == (t[g["token40"]["logical_block"]], g["token40"]["offset"])
    assert len(m.block_table(1)) == 3
    for _ in range(41, 48):
        m.append_slot_for_decode(1)
    s48 = m.append_slot_for_decode(1)
    assert len(m.block_table(1)) == 4
    assert oracle.split_slot(s48, bs) == (m.block_table(1)[g["token48"]["logical_block"]], 0)
    # a new block is opened exactly when the current length is 16, 32, 48
    m2 = BlockManager(64, bs)
    m2.allocate_for_prefill(2, 0)
    opened = []
    for L in range(0, 60):
        before = len(m2.block_table(2))
        m2.append_slot_for_decode(2)
        if len(m2.block_table(2)) > before and L > 0:
            opened.append(L)
    assert opened == g["allocating_lengths"]
    assert blocks_needed(100, bs) == g["prompt100_blocks"]


def test_lifecycle_example(golden):
    g = golden["lifecycle"]
    bs = g["block_size"]
    m = _mgr_with_front(16, bs, g["free_front"])
    slots = m.allocate_for_prefill(0, g["prompt"])
    assert m.block_table(0) == g["table_after_prefill"]
    assert [list(oracle.split_slot(s, bs)) for s in slots] == g["prompt_block_offsets"]
    for tok in "GHI":
        s = m.append_slot_for_decode(0)
        assert oracle.split_slot(s, bs) == (g[tok]["block"], g[tok]["offset"])
    assert m.block_table(0) == g["table_final"]


def test_leetcode22_cases(golden):
    g = golden["leetcode22_tests"]
    c = g["case1"]
    m = BlockManager(c["num_blocks"], c["block_size"], sort_on_release=True)
    m.allocate_for_prefill(1, c["prompt"])
    assert len(m.block_table(1)) == c["blocks_after_prefill"]
    assert m.num_free_blocks() == c["free_after_prefill"]
    with pytest.raises(oracle.AlreadyPrefilled):
        m.allocate_for_prefill(1, c["prompt"])
    m.append_slot_for_decode(1)
    assert len(m.block_table(1)) == c["blocks_after_1_decode"]
    m.append_slot_for_decode(1)
    m.append_slot_for_decode(1)
    assert len(m.block_table(1)) == c["blocks_after_3_decodes"]
    assert m.num_free_blocks() == c["free_after_3_decodes"]
    # reconstruction: one head, head_dim 64, each block filled with a value
    pool = np.zeros((c["num_blocks"], 1, c["block_size"], 64))
    for pb, val in zip(m.block_table(1), c["fill"]):
        pool[pb] = val
    rows = oracle.gather_logical(pool, m.block_table(1), m.context_len(1))[0]
    assert rows.shape == (c["rows"], 64)
    for lo, hi, val in c["row_values"]:
        assert np.all(rows[lo:hi] == val)

    c = g["case1b"]
    pool = np.zeros((c["num_blocks"], 1, c["block_size"], 2))
    pool[3] = 3.0
    pool[1] = 1.0
    rows = oracle.gather_logical(pool, c["table"], c["seq_len"])[0]
    assert rows.shape == (c["rows"], 2)
    for lo, hi, val in c["row_values"]:
        assert np.all(rows[lo:hi] == val)

    c = g["case2"]
    m = BlockManager(c["num_blocks"], c["block_size"], sort_on_release=True)
    m.allocate_for_prefill(2, c["prompt"])
    assert len(m.block_table(2)) == c["blocks"]
    m.append_slot_for_decode(2)
    assert len(m.block_table(2)) == c["blocks_after_decode"] and m.context_len(2) == c["rows"]
    pool = np.zeros((c["num_blocks"], 1, c["block_size"], 8))
    pool[m.block_table(2)[0]] = 7.0
    pool[m.block_table(2)[1]] = 8.0
    rows = oracle.gather_logical(pool, m.block_table(2), m.context_len(2))[0]
    assert rows.shape == (5, 8) and np.all(rows[:4] == 7.0) and np.all(rows[4:] == 8.0)

    for key in ("case3", "case4"):
        c = g[key]
        m = BlockManager(c["num_blocks"], c["block_size"], sort_on_release=True)
        free_before = list(m.free)
        with pytest.raises(oracle.OutOfBlocks, match="OOM"):
            m.allocate_for_prefill(3, c["prompt"])
        assert m.free == free_before and not m.is_live(3)

    c = g["ledger"]
    led = oracle.estimate_kv_cache_bytes(c["num_blocks"], c["block_size"], c["num_layers"],
                                         c["num_kv_heads"], c["head_dim"], c["dtype_bytes"])
    assert led["kv_bytes_per_token"] == c["kv_bytes_per_token"]
    assert led["total_cache_bytes"] == c["total_cache_bytes"]

    c = g["report"]
    m = BlockManager(c["num_blocks"], c["block_size"], sort_on_release=True)
    m.allocate_for_prefill(5, c["prompt"])
    rep = oracle.allocation_report(len(m.block_table(5)), m.context_len(5), c["block_size"])
    assert rep["allocated_tokens"] == c["allocated_tokens"]
    assert rep["unused_tail_tokens"] == c["unused_tail_tokens"]
    assert round(rep["utilization"], 3) == c["utilization"]
    m.free_sequence(5)
    assert m.free == c["free_after_release"]
    with pytest.raises(oracle.NotLive):
        m.free_sequence(5)

    c = g["decode_rollback"]
    m = BlockManager(c["num_blocks"], c["block_size"])
    m.allocate_for_prefill(6, c["prompt"])
    with pytest.raises(oracle.OutOfBlocks):
        m.append_slot_for_decode(6)
    assert m.context_len(6) == c["prompt"] and len(m.block_table(6)) == 1


def test_gqa_head_map_example(golden):
    g = golden["gqa_example"]
    for qh, kvh in g["q_to_kv"]:
        assert oracle.kv_head_of(qh, g["num_q_heads"], g["num_kv_heads"]) == kvh


def test_ledger_matches_size_formula(golden):
    # M_KV = 2 * layers * L * H_kv * D * 2 for fp16: L tokens of the ledger's per-token bytes
    led = oracle.estimate_kv_cache_bytes(1, 1, 3, 5, 7, 2)
    assert led["kv_bytes_per_token"] * 11 == 2 * 3 * 11 * 5 * 7 * 2


def test_batched_append_is_all_or_nothing():
    m = BlockManager(4, 4)
    m.allocate_for_prefill(0, 4)   # next append opens a block
    m.allocate_for_prefill(1, 4)
    m.allocate_for_prefill(2, 3)   # next append stays in its block
    assert m.num_free_blocks() == 1
    snapshot = (list(m.free), {s: (q.length, list(q.table)) for s, q in m.seqs.items()})
    with pytest.raises(oracle.OutOfBlocks):
        m.append_slots_for_decode([2, 0, 1])   # needs two new blocks, one free
    assert (list(m.free), {s: (q.length, list(q.table)) for s, q in m.seqs.items()}) == snapshot
    with pytest.raises(oracle.InvalidArgument):
        m.append_slots_for_decode([0, 0])
    with pytest.raises(oracle.NotLive):
        m.append_slots_for_decode([0, 9])
    assert (list(m.free), {s: (q.length, list(q.table)) for s, q in m.seqs.items()}) == snapshot
    slots = m.append_slots_for_decode([2, 0])
    assert slots[0] == m.block_table(2)[0] * 4 + 3 and slots[1] == m.block_table(0)[1] * 4


def test_release_appends_in_table_order():
    m = BlockManager(8, 2, [5, 1, 7, 0, 2, 3, 4, 6])
    m.allocate_for_prefill(0, 5)       # takes [5, 1, 7]
    assert m.block_table(0) == [5, 1, 7]
    m.free_sequence(0)
    assert m.free == [0, 2, 3, 4, 6, 5, 1, 7]


def test_block_size_one_allocates_every_token():
    m = BlockManager(8, 1)
    m.allocate_for_prefill(0, 2)
    for i in range(3):
        m.append_slot_for_decode(0)
    assert len(m.block_table(0)) == 5 and m.context_len(0) == 5
    assert not m.check_invariants()


def _state(m):
    return (list(m.free), sorted((s, q.length, tuple(q.table)) for s, q in m.seqs.items()))


@pytest.mark.parametrize("seed,n_blocks,bs", [(1, 32, 4), (2, 7, 1), (3, 12, 16), (4, 60, 3)])
def test_invariants_hold_on_random_traces(seed, n_blocks, bs):
    rng = np.random.default_rng(seed)
    order = rng.permutation(n_blocks)
    m = BlockManager(n_blocks, bs, order, sort_on_release=bool(seed % 2))
    errors = {"ok": 0}
    for op in synth.manager_op_trace(seed, 10_000, max_id=30, max_prefill=40):
        before = _state(m)
        try:
            if op[0] == "prefill":
                m.allocate_for_prefill(op[1], op[2])
            elif op[0] == "append":
                m.append_slot_for_decode(op[1])
            elif op[0] == "append_batch":
                m.append_slots_for_decode(list(op[1]))
            elif op[0] == "free":
                m.free_sequence(op[1])
            else:
                m.can_allocate(op[1])
            errors["ok"] += 1
        except oracle.ManagerError as e:
            errors[type(e).__name__] = errors.get(type(e).__name__, 0) + 1
            assert _state(m) == before, "a failed op changed state"
        assert m.check_invariants() == []
    # the trace exercises every failure kind
    for kind in ("OutOfBlocks", "NotLive", "AlreadyPrefilled"):
        assert errors.get(kind, 0) > 0, errors


def test_invariant_checker_catches_corruption():
    m = BlockManager(8, 4)
    m.allocate_for_prefill(0, 9)
    assert m.check_invariants() == []
    m.free.append(m.block_table(0)[0])
    assert {"I2", "I3", "I6"} <= set(m.check_invariants()) or {"I2", "I3"} <= set(m.check_invariants())
    m = BlockManager(8, 4)
    m.allocate_for_prefill(0, 9)
    m.seqs[0].length = 20
    assert "I5" in m.check_invariants()
    m = BlockManager(8, 4)
    m.allocate_for_prefill(0, 4)
    m.allocate_for_prefill(1, 4)
    m.seqs[1].table[0] = m.seqs[0].table[0]
    m.free.append(99)
    bad = set(m.check_invariants())
    assert {"I1", "I4"} <= bad


def test_write_round_trip_and_poison():
    """A write followed by the table-order gather returns exactly the written
    rows; slots no write touched keep the poison bits ([leetcode-22] TODO 4)."""
    cfg = synth.CONFIGS["tiny"]
    wl = synth.decode_workload(cfg)
    from oracle.replay import decode_state
    st = decode_state(wl)
    for b in wl.seq_ids:
        L = int(st.context_lens[b])
        table = st.manager.block_table(b)
        k = oracle.gather_logical(st.key_cache, table, L)
        v = oracle.gather_logical(st.value_cache, table, L)
        expect_k = np.concatenate([wl.hist_k[b], wl.new_k[b:b + 1]], axis=0).transpose(1, 0, 2)
        expect_v = np.concatenate([wl.hist_v[b], wl.new_v[b:b + 1]], axis=0).transpose(1, 0, 2)
        assert np.array_equal(k.view(np.uint32), expect_k.view(np.uint32))
        assert np.array_equal(v.view(np.uint32), expect_v.view(np.uint32))
    used = {pb for b in wl.seq_ids for pb in st.manager.block_table(b)}
    poison = synth.POISON_BITS["f32"]
    kbits = st.key_cache.view(np.uint32)
    for pb in range(cfg.num_blocks):
        if pb not in used:
            assert np.all(kbits[pb] == poison)
    # exactly sum(L) slots per head were written
    written = np.count_nonzero(kbits[:, 0, :, 0] != poison)
    assert written == int(st.context_lens.sum())
    # the tiny workload's step: positions 39, 16, 0, 63; 16 and 0 open blocks
    assert st.manager.context_lens(wl.seq_ids).tolist() == [40, 17, 1, 64]
    assert len(used) == 10


def test_write_skips_out_of_range_slots():
    k = np.zeros((2, 1, 4, 2), dtype=np.float32)
    v = np.zeros_like(k)
    key = np.ones((3, 1, 2), dtype=np.float32)
    oracle.write_kv(key, key, [-1, 8, 5], k, v, 4)
    assert k.sum() == 2.0 and k[1, 0, 1].tolist() == [1.0, 1.0]
