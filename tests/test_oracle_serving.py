"""Pin of the oracle's serving-trace replay: the order of a serving step
([mini-vLLM BM] "Block Manager 和 Scheduler 如何协作": append a slot for
every running row, write the step's rows, attend, then release the finished
sequences and admit their replacements), worked by hand on a tiny pool.
CPU only."""
from types import SimpleNamespace

import numpy as np

import synth
from oracle.replay import serving_replay


def _rows(rng, n):
    return rng.standard_normal((n, 1, 2)).astype(np.float32)


def test_serving_replay_worked_by_hand():
    rng = np.random.default_rng(4)
    cfg = SimpleNamespace(num_blocks=8, block_size=4, num_kv_heads=1, head_dim=2, dtype="f32")
    prompts = [3, 4, 1]
    hist = [(_rows(rng, n), _rows(rng, n)) for n in prompts]
    refill_k, refill_v = _rows(rng, 2), _rows(rng, 2)
    steps = [SimpleNamespace(new_k=_rows(rng, 3), new_v=_rows(rng, 3),
                             refills=[SimpleNamespace(row=1, old_id=1, new_id=3, prompt_len=2,
                                                      k=refill_k, v=refill_v)]),
             SimpleNamespace(new_k=_rows(rng, 3), new_v=_rows(rng, 3), refills=[])]
    trace = SimpleNamespace(cfg=cfg, prompt_lens=np.array(prompts), hist_k=[h[0] for h in hist],
                            hist_v=[h[1] for h in hist], steps=steps)
    seen = []
    for st, mgr, kc, vc, row_ids, slots in serving_replay(trace):
        seen.append((list(row_ids), [int(s) for s in slots], [list(mgr.block_table(i)) for i in row_ids],
                     list(mgr.free)))
        # the step's rows sit at its slots (block slot // 4, row slot % 4)
        for i, s in enumerate(slots):
            assert np.array_equal(kc[s // 4, :, s % 4], st.new_k[i])
            assert np.array_equal(vc[s // 4, :, s % 4], st.new_v[i])
    # identity free list: prompts take blocks 0, 1, 2 (slots 0-2, 4-7, 8).
    # Step 0: seq 0 at position 3 -> slot 3; seq 1 at position 4 opens block 3
    # -> slot 12; seq 2 at position 1 -> slot 9.
    assert seen[0] == ([0, 1, 2], [3, 12, 9], [[0], [1, 3], [2]], [4, 5, 6, 7])
    # then seq 1 finishes: blocks 1, 3 appended in table order; its
    # replacement (id 3, prompt 2) takes block 4, slots 16, 17.
    # Step 1: seq 0 at position 4 opens block 5 -> slot 20; seq 3 at
    # position 2 -> slot 18; seq 2 at position 2 -> slot 10.
    assert seen[1] == ([0, 3, 2], [20, 18, 10], [[0, 5], [4], [2]], [6, 7, 1, 3])
    # the refill's prompt rows sit at slots 16, 17 and the rest of the pool
    # that nothing wrote is still the poison value
    assert np.array_equal(kc[4, :, 0], refill_k[0]) and np.array_equal(kc[4, :, 1], refill_k[1])
    poison = synth.poison_array((), "f32")
    assert np.array_equal(kc[6].view(np.uint32), np.broadcast_to(poison.view(np.uint32), kc[6].shape))
