"""The seeded generators are deterministic and produce the documented shapes;
the churn trace never runs the oracle manager out of blocks.  CPU only."""
import numpy as np

import oracle
import synth
from oracle.replay import replay_churn


def test_decode_workload_is_deterministic_and_shaped():
    for name in ("tiny", "qwen2_1p5b_b32"):
        cfg = synth.CONFIGS[name]
        a = synth.decode_workload(cfg)
        b = synth.decode_workload(cfg)
        assert np.array_equal(a.context_lens, b.context_lens)
        assert np.array_equal(a.q.view(np.uint8), b.q.view(np.uint8))
        assert a.q.shape == (cfg.batch, cfg.num_q_heads, cfg.head_dim)
        assert a.new_k.shape == (cfg.batch, cfg.num_kv_heads, cfg.head_dim)
        for i, L in enumerate(a.context_lens):
            assert a.hist_k[i].shape == (int(L) - 1, cfg.num_kv_heads, cfg.head_dim)
    cfg = synth.CONFIGS["qwen2_1p5b_b32"]
    w = synth.decode_workload(cfg)
    assert w.context_lens.min() >= 128 and w.context_lens.max() <= 2048
    assert sorted(w.initial_free_order.tolist()) == list(range(cfg.num_blocks))


def test_truncated_batch_keeps_the_same_sequences():
    cfg = synth.CONFIGS["qwen2_1p5b_b32"]
    full = synth.decode_workload(cfg)
    part = synth.decode_workload(cfg, batch=5)
    assert np.array_equal(full.context_lens[:5], part.context_lens)
    assert np.array_equal(full.q[:5], part.q)
    assert np.array_equal(full.hist_v[4], part.hist_v[4])


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -9, 3.0], dtype=np.float32)
    got = synth.to_storage(x, "bf16")
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa -> 1.0 (0x3F80)
    # 1 + 3*2^-8 is a tie between 1+2^-7 and 1+2^-6: even -> 1 + 2^-6 (0x3F82)
    assert got.tolist() == [0x3F80, 0x3F82, 0xBF80, 0x4040]


def test_churn_trace_never_runs_out_of_blocks():
    cfg = synth.CONFIGS["qwen2_7b_b64"]
    rng = np.random.default_rng(cfg.seed)
    rng.integers(512, 8193, size=cfg.batch)
    events = synth.churn_events(rng, cfg.churn_priors)
    assert sum(1 for e in events if e[0] == "prefill") == cfg.churn_priors
    m = oracle.BlockManager(cfg.num_blocks, cfg.block_size)
    replay_churn(m, events)                   # raises on OOM
    assert m.num_free_blocks() == cfg.num_blocks and not m.seqs
    assert m.free != list(range(cfg.num_blocks))   # order scrambled
    assert m.check_invariants() == []


def test_serving_trace_shapes():
    cfg = synth.CONFIGS["serving_trace"]
    tr = synth.serving_trace(cfg, steps=3, batch=8)
    assert tr.prompt_lens.min() >= 16 and tr.prompt_lens.max() <= 4096
    steps = list(tr.steps)
    assert len(steps) == 3 and steps[0].q.shape == (8, 32, 128)
