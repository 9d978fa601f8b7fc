"""Pins of the oracle's decode attention against closed forms, a library
routine (torch's scaled_dot_product_attention in float64 on the CPU, and
scipy's softmax), a second independent route (position-by-position online
softmax) and brute force on tiny inputs.  CPU only."""
import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth
from oracle.replay import decode_state


def _tiny_state():
    wl = synth.decode_workload(synth.CONFIGS["tiny"])
    return wl, decode_state(wl)


def _contiguous_inputs(wl, b):
    """Pre-scatter K/V of sequence b straight from the generator: history
    then the new token, as [L, H_kv, D] float64 (an independent route that
    never touches the pool or a block table)."""
    k = np.concatenate([wl.hist_k[b], wl.new_k[b:b + 1]], axis=0)
    v = np.concatenate([wl.hist_v[b], wl.new_v[b:b + 1]], axis=0)
    return (oracle.widen(k, wl.cfg.dtype), oracle.widen(v, wl.cfg.dtype))


def test_paged_matches_torch_sdpa_on_prescatter_kv():
    wl, st = _tiny_state()
    cfg = wl.cfg
    out = oracle.decode_attention(wl.q, st.key_cache, st.value_cache, st.block_tables,
                                  st.context_lens, cfg.scale, cfg.dtype)
    for b in wl.seq_ids:
        k, v = _contiguous_inputs(wl, b)
        q = torch.from_numpy(oracle.widen(wl.q[b], cfg.dtype))[None, :, None, :]
        kt = torch.from_numpy(k.transpose(1, 0, 2).copy())[None]
        vt = torch.from_numpy(v.transpose(1, 0, 2).copy())[None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q, kt, vt, scale=cfg.scale, enable_gqa=True)[0, :, 0, :].numpy()
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def test_gqa_against_sdpa_with_grouped_heads():
    """H_q = 12, H_kv = 2 (group 6): the library's GQA grouping (query head i
    reads kv head i // 6) agrees with the oracle's head map."""
    rng = np.random.default_rng(7)
    L, D = 37, 16
    q = rng.standard_normal((12, D))
    k = rng.standard_normal((2, L, D))
    v = rng.standard_normal((2, L, D))
    ours = oracle.contiguous_attention(q, k, v, 0.3)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        scale=0.3, enable_gqa=True)[0, :, 0].numpy()
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-12)
    for qh in range(12):
        s = scipy.special.softmax(0.3 * (k[qh // 6] @ q[qh]))
        np.testing.assert_allclose(ours[qh], s @ v[qh // 6], rtol=0, atol=1e-12)


def test_online_walk_agrees_with_gather_route():
    wl, st = _tiny_state()
    cfg = wl.cfg
    out = oracle.decode_attention(wl.q, st.key_cache, st.value_cache, st.block_tables,
                                  st.context_lens, cfg.scale, cfg.dtype)
    for b in wl.seq_ids:
        walk = oracle.decode_attention_online(wl.q[b], st.key_cache, st.value_cache,
                                              st.manager.block_table(b), int(st.context_lens[b]),
                                              cfg.scale, cfg.dtype)
        np.testing.assert_allclose(out[b], walk, rtol=0, atol=1e-12)


def test_single_token_returns_its_value_row_exactly():
    wl, st = _tiny_state()
    cfg = wl.cfg
    b = 2                                          # context length 1
    assert int(st.context_lens[b]) == 1
    out = oracle.decode_attention(wl.q, st.key_cache, st.value_cache, st.block_tables,
                                  st.context_lens, cfg.scale, cfg.dtype, seqs=[b])
    for qh in range(cfg.num_q_heads):
        assert np.array_equal(out[b, qh], oracle.widen(wl.new_v[b, qh], cfg.dtype))


def test_closed_forms():
    rng = np.random.default_rng(3)
    L, D = 29, 8
    q = rng.standard_normal((4, D))
    v = rng.standard_normal((2, L, D))
    # all keys equal -> uniform weights -> mean of V
    k_same = np.repeat(rng.standard_normal((2, 1, D)), L, axis=1)
    np.testing.assert_allclose(oracle.contiguous_attention(q, k_same, v, 0.7),
                               np.repeat(v.mean(axis=1), 2, axis=0), rtol=0, atol=1e-13)
    # scale 0 -> mean of V whatever the keys
    k = rng.standard_normal((2, L, D))
    np.testing.assert_allclose(oracle.contiguous_attention(q, k, v, 0.0),
                               np.repeat(v.mean(axis=1), 2, axis=0), rtol=0, atol=1e-13)
    # constant V rows -> that constant
    c = rng.standard_normal((2, 1, D))
    v_const = np.repeat(c, L, axis=1)
    out = oracle.contiguous_attention(q, k, v_const, 0.5)
    np.testing.assert_allclose(out, np.repeat(c[:, 0], 2, axis=0), rtol=0, atol=1e-13)
    # one dominant key -> its V row
    kd = np.zeros((2, L, D))
    kd[:, 11] = 50.0
    qd = np.abs(q) + 0.1
    out = oracle.contiguous_attention(qd, kd, v, 1.0)
    np.testing.assert_allclose(out, np.repeat(v[:, 11], 2, axis=0), rtol=0, atol=1e-12)
    # two keys: weights are the logistic function of the score gap
    q2 = np.array([[1.0, 0.0]])
    k2 = np.array([[[0.5, 0.0], [2.0, 0.0]]])
    v2 = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    w1 = 1.0 / (1.0 + np.exp(-(2.0 - 0.5) * 0.9))
    np.testing.assert_allclose(oracle.contiguous_attention(q2, k2, v2, 0.9)[0],
                               [1.0 - w1, w1], rtol=0, atol=1e-15)


def test_kv_head_signature():
    """Each KV head's V rows hold the head index; query head qh must return
    qh // G, which a wrong head map (for instance qh % H_kv) would not."""
    rng = np.random.default_rng(5)
    h_q, h_kv, L, D = 12, 4, 9, 4
    q = rng.standard_normal((h_q, D))
    k = rng.standard_normal((h_kv, L, D))
    v = np.zeros((h_kv, L, D)) + np.arange(h_kv)[:, None, None]
    out = oracle.contiguous_attention(q, k, v, 1.0)
    for qh in range(h_q):
        np.testing.assert_allclose(out[qh], qh // 3, rtol=0, atol=1e-13)


def test_empty_context_gives_zeros():
    q = np.ones((2, 4))
    k = np.zeros((1, 0, 4))
    assert np.array_equal(oracle.contiguous_attention(q, k, k, 1.0), np.zeros((2, 4)))


def test_physical_relabelling_and_contiguous_placement():
    """The output depends only on the logical sequence: a permuted placement
    and an identity (contiguous) placement of the same K/V agree exactly."""
    wl, st = _tiny_state()
    cfg = wl.cfg
    base = oracle.decode_attention(wl.q, st.key_cache, st.value_cache, st.block_tables,
                                   st.context_lens, cfg.scale, cfg.dtype)
    perm = np.random.default_rng(11).permutation(cfg.num_blocks)
    inv = np.argsort(perm)
    # new pool position j holds old block inv[j], so old block pb now lives at perm[pb]
    kc = st.key_cache[inv]
    vc = st.value_cache[inv]
    tables = np.where(st.block_tables >= 0, perm[np.maximum(st.block_tables, 0)], -1)
    moved = oracle.decode_attention(wl.q, kc, vc, tables, st.context_lens, cfg.scale, cfg.dtype)
    assert np.array_equal(base, moved)


def test_poison_in_tail_and_padding_is_never_read():
    """Unwritten tail slots hold NaN poison; a result with no NaN shows the
    read stopped at L (reading whole blocks would pick up the poison)."""
    wl, st = _tiny_state()
    cfg = wl.cfg
    out = oracle.decode_attention(wl.q, st.key_cache, st.value_cache, st.block_tables,
                                  st.context_lens, cfg.scale, cfg.dtype)
    assert np.isfinite(out).all()
    # sanity: the tail of sequence 1 (L = 17 -> second block holds 1 token) is poisoned
    table1 = st.manager.block_table(1)
    assert np.isnan(st.key_cache[table1[1], 0, 1:]).all()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_half_precision_widening(dtype):
    x = np.array([1.0, -2.5, 3.140625, 1e-3, 65504.0 if dtype == "f16" else 1e30], dtype=np.float32)
    s = synth.to_storage(x, dtype)
    w = oracle.widen(s, dtype)
    ref = torch.from_numpy(x).to(torch.bfloat16 if dtype == "bf16" else torch.float16).double().numpy()
    assert np.array_equal(w, ref)
