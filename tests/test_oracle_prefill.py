"""Pins of the oracle's chunked-prefill attention (oracle.prefill_attention):
every query row equals the online-softmax oracle run over the sequence cut
at that row's position (a second route, itself pinned), a one-row chunk is
decode attention, uniform scores give the running mean of V (closed form),
one-hot V rows expose the causal weights exactly, and rows placed before
the first position give zeros.  CPU only."""
import numpy as np
import pytest

import oracle
import synth


def _case(rng, dtype, N, H, bs, D, lens):
    m = oracle.BlockManager(N, bs, rng.permutation(N))
    kc, vc = oracle.new_pool(N, H, bs, D, synth.poison_array((), dtype))
    for b, L in enumerate(lens):
        slots = m.allocate_for_prefill(b, L)
        oracle.write_kv(synth.normal(rng, (L, H, D), dtype), synth.normal(rng, (L, H, D), dtype),
                        slots, kc, vc, bs)
    width = max(-(-L // bs) for L in lens)
    return m, kc, vc, m.block_tables(list(range(len(lens))), width, -1)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rows_equal_online_oracle_cut_at_their_position(dtype):
    rng = np.random.default_rng(11)
    lens, nq = [9, 20, 5], [4, 20, 1]
    m, kc, vc, tabs = _case(rng, dtype, 12, 2, 4, 8, lens)
    qs = np.concatenate([[0], np.cumsum(nq)])
    q = synth.normal(rng, (int(qs[-1]), 6, 8), dtype)
    out = oracle.prefill_attention(q, qs, kc, vc, tabs, lens, 0.3, dtype)
    for b, (L, n) in enumerate(zip(lens, nq)):
        for i in range(n):
            p = L - n + i
            ref = oracle.decode_attention_online(q[qs[b] + i], kc, vc, m.block_table(b), p + 1, 0.3, dtype)
            assert np.abs(out[qs[b] + i] - ref).max() < 1e-12, (b, i)


def test_one_row_chunk_is_decode_attention():
    rng = np.random.default_rng(12)
    lens = [17, 3, 40]
    m, kc, vc, tabs = _case(rng, "f16", 16, 2, 8, 16, lens)
    q = synth.normal(rng, (3, 4, 16), "f16")
    out = oracle.prefill_attention(q, [0, 1, 2, 3], kc, vc, tabs, lens, 0.25, "f16")
    ref = oracle.decode_attention(q, kc, vc, tabs, lens, 0.25, "f16")
    assert np.abs(out - ref).max() < 1e-12


def test_uniform_scores_give_running_means_and_one_hot_values_show_the_mask():
    N, H, bs, D, L = 4, 1, 4, 16, 12
    m = oracle.BlockManager(N, bs, [2, 0, 3, 1])
    kc, vc = oracle.new_pool(N, H, bs, D, synth.poison_array((), "f32"))
    slots = m.allocate_for_prefill(0, L)
    k = np.zeros((L, H, D), np.float32)                  # every score 0: uniform weights
    v = np.zeros((L, H, D), np.float32)
    v[np.arange(L), 0, np.arange(L)] = 1.0               # V row t = e_t
    oracle.write_kv(k, v, slots, kc, vc, bs)
    tabs = m.block_tables([0], 3, -1)
    q = np.ones((L, 1, D), np.float32)
    out = oracle.prefill_attention(q, [0, L], kc, vc, tabs, [L], 1.0, "f32")
    for i in range(L):
        expect = np.zeros(D)
        expect[:i + 1] = 1.0 / (i + 1)                   # mean of e_0 .. e_i
        assert np.allclose(out[i, 0], expect, rtol=0, atol=1e-15)


def test_rows_before_the_first_position_are_zero():
    rng = np.random.default_rng(13)
    m, kc, vc, tabs = _case(rng, "f32", 4, 1, 4, 8, [3])
    q = synth.normal(rng, (5, 2, 8), "f32")
    out = oracle.prefill_attention(q, [0, 5], kc, vc, tabs, [3], 0.5, "f32")
    assert np.all(out[:2] == 0.0) and np.all(np.isfinite(out[2:]))
