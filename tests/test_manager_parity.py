"""The C++ block manager (through the C ABI) against the oracle manager on
the pages' worked examples and on seeded random op traces: identical slots,
tables, lengths, free-list order and error kinds after every op.  CPU only
(host logic)."""
import numpy as np
import pytest

import oracle
import paged_kv_cache_128_amd as pkv
import synth

ERR = {oracle.InvalidArgument: pkv.InvalidArgumentError, oracle.OutOfBlocks: pkv.OutOfBlocksError,
       oracle.NotLive: pkv.NotLiveError, oracle.AlreadyPrefilled: pkv.AlreadyPrefilledError}


def _run(mgr, op, impl):
    """Apply op; returns ("ok", result) or ("err", kind)."""
    try:
        if op[0] == "prefill":
            r = mgr.allocate_for_prefill(op[1], op[2])
            return "ok", [int(x) for x in r]
        if op[0] == "append":
            return "ok", int(mgr.append_slot_for_decode(op[1]))
        if op[0] == "append_batch":
            r = mgr.append_slots_for_decode(list(op[1]))
            if impl == "c":
                slots, lens, newb = r
                return "ok", [int(x) for x in slots]
            return "ok", [int(x) for x in r]
        if op[0] == "free":
            mgr.free_sequence(op[1])
            return "ok", None
        return "ok", bool(mgr.can_allocate(op[1]))
    except (oracle.ManagerError, pkv.PkvError) as e:
        for o, c in ERR.items():
            if isinstance(e, o) or isinstance(e, c):
                return "err", o.__name__
        raise


def _same_state(o, c, ids):
    assert c.free_list() == o.free
    assert c.num_live_sequences() == len(o.seqs)
    for s in ids:
        if o.is_live(s):
            assert c.block_table(s) == o.block_table(s)
            assert c.context_len(s) == o.context_len(s)
        else:
            with pytest.raises(pkv.NotLiveError):
                c.context_len(s)
    assert c.check_invariants()


@pytest.mark.parametrize("seed,n_blocks,bs,sort", [(11, 48, 4, False), (12, 9, 1, True),
                                                   (13, 20, 16, False), (14, 100, 3, True),
                                                   (15, 33, 7, False)])
def test_random_traces_match_oracle(seed, n_blocks, bs, sort):
    order = np.random.default_rng(seed).permutation(n_blocks)
    o = oracle.BlockManager(n_blocks, bs, order, sort_on_release=sort)
    c = pkv.KVBlockManager(n_blocks, bs, order, sort_on_release=sort)
    ids = list(range(30))
    kinds = set()
    for op in synth.manager_op_trace(seed, 10_000, max_id=30, max_prefill=50):
        ro = _run(o, op, "o")
        rc = _run(c, op, "c")
        assert ro == rc, (op, ro, rc)
        kinds.add(ro[1] if ro[0] == "err" else "ok")
        _same_state(o, c, ids)
    assert {"ok", "OutOfBlocks", "NotLive", "AlreadyPrefilled", "InvalidArgument"} <= kinds


def test_worked_examples_through_c_abi(golden):
    g = golden["address_translation"]
    m = pkv.KVBlockManager(16, 4, [5, 2, 9, 1] + [i for i in range(16) if i not in (5, 2, 9, 1)])
    slots = m.allocate_for_prefill(0, 16)
    assert slots[g["token_pos"]] == g["slot"]
    g = golden["lifecycle"]
    m = pkv.KVBlockManager(16, 4, g["free_front"] + [i for i in range(16) if i not in g["free_front"]])
    slots = m.allocate_for_prefill(0, g["prompt"])
    assert [[s // 4, s % 4] for s in slots] == g["prompt_block_offsets"]
    for tok in "GHI":
        s = m.append_slot_for_decode(0)
        assert [s // 4, s % 4] == [g[tok]["block"], g[tok]["offset"]]
    assert m.block_table(0) == g["table_final"]
    g = golden["leetcode22_tests"]["report"]
    m = pkv.KVBlockManager(g["num_blocks"], g["block_size"], sort_on_release=True)
    m.allocate_for_prefill(5, g["prompt"])
    m.free_sequence(5)
    assert m.free_list() == g["free_after_release"]
    with pytest.raises(pkv.NotLiveError):
        m.free_sequence(5)


def test_batched_append_outputs_new_blocks():
    m = pkv.KVBlockManager(16, 4)
    m.allocate_for_prefill(0, 4)
    m.allocate_for_prefill(1, 3)
    slots, lens, newb = m.append_slots_for_decode([0, 1])
    assert lens.tolist() == [5, 4]
    assert newb[0] == m.block_table(0)[1] and newb[1] == -1
    assert slots.tolist() == [m.block_table(0)[1] * 4, m.block_table(1)[0] * 4 + 3]
    tabs = m.block_tables([0, 1], 3, -1)
    assert tabs.tolist() == [m.block_table(0) + [-1], m.block_table(1) + [-1, -1]]
    with pytest.raises(pkv.InvalidArgumentError):
        m.block_tables([0, 1], 1, -1)


def test_churn_replay_matches_oracle():
    cfg = synth.CONFIGS["qwen2_7b_b64"]
    rng = np.random.default_rng(cfg.seed)
    rng.integers(512, 8193, size=cfg.batch)
    events = synth.churn_events(rng, 120)
    o = oracle.BlockManager(cfg.num_blocks, cfg.block_size)
    c = pkv.KVBlockManager(cfg.num_blocks, cfg.block_size)
    from oracle.replay import replay_churn
    replay_churn(o, events)
    for ev in events:
        if ev[0] == "prefill":
            c.allocate_for_prefill(ev[1], ev[2], want_slots=False)
        elif ev[0] == "grow":
            for _ in range(ev[2]):
                c.append_slots_for_decode(list(ev[1]))
        else:
            c.free_sequence(ev[1])
    assert c.free_list() == o.free


def _run_share(mgr, op, impl):
    """Apply a sharing-trace op; returns (outcome, result, queued copies)."""
    try:
        if op[0] == "share":
            mgr.share_prefix(op[1], op[2], op[3])
            r = ("ok", None)
        else:
            r = _run(mgr, op, impl)
    except (oracle.ManagerError, pkv.PkvError) as e:
        r = None
        for o, c in ERR.items():
            if isinstance(e, o) or isinstance(e, c):
                r = ("err", o.__name__)
        if r is None:
            raise
    if impl == "c":
        src, dst = mgr.take_copies()
        copies = list(zip(src.tolist(), dst.tolist()))
    else:
        copies = mgr.take_copies()
    return r, copies


@pytest.mark.parametrize("seed,n_blocks,bs,sort", [(41, 40, 4, False), (42, 12, 1, True),
                                                   (43, 20, 16, False), (44, 25, 3, True)])
def test_random_share_traces_match_oracle(seed, n_blocks, bs, sort):
    """Prefix sharing and copy-on-write: identical outcomes, slots, tables,
    reference counts, copy queues and free-list order after every op."""
    order = np.random.default_rng(seed).permutation(n_blocks)
    o = oracle.BlockManager(n_blocks, bs, order, sort_on_release=sort)
    c = pkv.KVBlockManager(n_blocks, bs, order, sort_on_release=sort)
    ids = list(range(24))
    kinds, n_copies = set(), 0
    for op in synth.manager_share_trace(seed, 2000):
        ro = _run_share(o, op, "o")
        rc = _run_share(c, op, "c")
        assert ro == rc, (op, ro, rc)
        kinds.add(ro[0][1] if ro[0][0] == "err" else "ok")
        n_copies += len(ro[1])
        _same_state(o, c, ids)
        assert [c.ref_count(b) for b in range(n_blocks)] == o.ref
    assert {"ok", "OutOfBlocks", "NotLive", "AlreadyPrefilled", "InvalidArgument"} <= kinds
    assert n_copies > 0 or bs == 1       # with bs == 1 no block is ever partly filled


def test_batched_append_reports_copy_on_write_blocks():
    m = pkv.KVBlockManager(8, 4)
    m.allocate_for_prefill(0, 6)
    m.share_prefix(0, 1, 6)
    slots, lens, newb = m.append_slots_for_decode([1, 0])
    assert newb.tolist() == [2, -1] and lens.tolist() == [7, 7]
    assert slots.tolist() == [2 * 4 + 2, 1 * 4 + 2]
    src, dst = m.take_copies()
    assert src.tolist() == [1] and dst.tolist() == [2]
    assert m.block_table(1) == [0, 2] and m.ref_count(1) == 1


@pytest.mark.parametrize("seed,n_blocks,bs", [(51, 30, 4), (52, 16, 16), (53, 9, 1)])
def test_append_tokens_matches_oracle(seed, n_blocks, bs):
    """Multi-token appends (prefill chunks), with sharing so that a chunk can
    start in a shared tail block: identical slots, errors, tables, copies
    and free lists."""
    rng = np.random.default_rng(seed)
    o = oracle.BlockManager(n_blocks, bs)
    c = pkv.KVBlockManager(n_blocks, bs)
    kinds = set()
    for _ in range(600):
        u = rng.random()
        sid = int(rng.integers(8))
        if u < 0.2:
            op = ("prefill", sid, int(rng.integers(0, 12)))
        elif u < 0.35:
            op = ("share", int(rng.integers(8)), sid, int(rng.integers(0, 12)))
        elif u < 0.8:
            op = ("append_tokens", sid, int(rng.integers(0, 20)))
        else:
            op = ("free", sid)
        res = []
        for mgr, impl in ((o, "o"), (c, "c")):
            try:
                if op[0] == "append_tokens":
                    r = ("ok", [int(x) for x in mgr.append_tokens(op[1], op[2])])
                else:
                    r = _run_share(mgr, op, impl)[0]
            except (oracle.ManagerError, pkv.PkvError) as e:
                r = ("err", next(o_.__name__ for o_, c_ in ERR.items() if isinstance(e, (o_, c_))))
            copies = mgr.take_copies()
            if impl == "c":
                copies = list(zip(copies[0].tolist(), copies[1].tolist()))
            res.append((r, copies))
        assert res[0] == res[1], (op, res)
        kinds.add(res[0][0][0] if res[0][0][0] == "ok" else res[0][0][1])
        assert c.free_list() == o.free and c.check_invariants() and o.check_invariants() == []
    assert {"ok", "OutOfBlocks"} <= kinds


def _admit(mgr, ids, lens, extend, impl):
    try:
        r = mgr.admit_batch(ids, lens, extend_live=extend)
        if impl == "c":
            return "ok", [int(x) for x in r[0]]
        return "ok", [int(x) for chunk in r for x in chunk]
    except (oracle.ManagerError, pkv.PkvError) as e:
        for o, c in ERR.items():
            if isinstance(e, o) or isinstance(e, c):
                return "err", o.__name__
        raise


@pytest.mark.parametrize("seed,n_blocks,bs", [(21, 40, 4), (22, 12, 1), (23, 64, 16), (24, 30, 3)])
def test_admit_batch_traces_match_oracle(seed, n_blocks, bs):
    """All-or-nothing batch admission (pkv_admit_batch) interleaved with
    shares, appends and frees: same slots, error kinds and state as the
    oracle after every op; every failed batch leaves the state unchanged."""
    rng = np.random.default_rng(seed)
    o = oracle.BlockManager(n_blocks, bs, rng.permutation(n_blocks))
    c = pkv.KVBlockManager(n_blocks, bs, o.free[:])
    ids = list(range(12))
    kinds = set()
    for _ in range(1500):
        u = rng.random()
        if u < 0.45:
            k = int(rng.integers(0, 5))
            batch = [int(x) for x in rng.integers(0, 12, k)]
            if rng.random() < 0.2:
                batch.append(-1 if rng.random() < 0.5 else (batch[0] if batch else 3))
            lens = [int(x) for x in rng.integers(0, 3 * bs + 2, len(batch))]
            extend = bool(rng.random() < 0.6)
            before = (o.free[:], {s: (o.context_len(s), o.block_table(s)) for s in ids if o.is_live(s)})
            ro = _admit(o, batch, lens, extend, "o")
            rc = _admit(c, batch, lens, extend, "c")
            assert ro == rc, (batch, lens, extend, ro, rc)
            if ro[0] == "err":
                assert (o.free, {s: (o.context_len(s), o.block_table(s)) for s in ids if o.is_live(s)}) == before
            kinds.add(("admit", ro[1] if ro[0] == "err" else "ok"))
        elif u < 0.55:
            donor, sid = int(rng.integers(12)), int(rng.integers(12))
            n = int(rng.integers(0, 3 * bs))
            for mgr in (o, c):
                try:
                    mgr.share_prefix(donor, sid, n)
                except (oracle.ManagerError, pkv.PkvError):
                    pass
        elif u < 0.8:
            op = ("append", int(rng.integers(12)))
            assert _run(o, op, "o") == _run(c, op, "c")
        else:
            op = ("free", int(rng.integers(12)))
            assert _run(o, op, "o") == _run(c, op, "c")
        o.take_copies()
        c.take_copies()
        _same_state(o, c, ids)
    assert {("admit", "ok"), ("admit", "OutOfBlocks"), ("admit", "AlreadyPrefilled"),
            ("admit", "InvalidArgument")} <= kinds
