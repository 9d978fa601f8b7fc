"""GPU parity of chunked-prefill attention (paged_prefill_attention) against
the oracle's causal multi-query attention through block tables: sequences
admitted with a first chunk and extended by a second (so later chunks attend
over history written by earlier launches), ragged chunk lengths spanning
several 64-row workgroups and a ragged tail, GQA groups 7 and 4, both 16-bit
types and both output types; plus rows placed before the first position
(zeros), empty chunks, and a one-row chunk against the decode kernel."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
import paged_kv_cache_128_amd as pkv

from gpu_harness import to_device, TORCH_DTYPE

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(f"[gpu] {msg}", flush=True)


@pytest.mark.parametrize("dtype,hq,hkv,out_dtype,bs,D", [
    ("bf16", 28, 4, None, 16, 128), ("f16", 32, 8, None, 16, 128), ("bf16", 12, 2, "bf16", 16, 128),
    # shapes the matrix-core kernel does not take: the generic kernel
    ("f32", 4, 4, None, 16, 64), ("bf16", 8, 2, None, 8, 128), ("f16", 12, 2, "f16", 16, 64)])
def test_chunked_prefill_matches_oracle(dtype, hq, hkv, out_dtype, bs, D):
    from paged_kv_cache_128_amd.engine import PagedKVEngine
    rng = np.random.default_rng({"bf16": 81, "f16": 82, "f32": 83}[dtype] + hq + D + bs)
    first = [1, 37, 64, 130, 200, 5]
    second = [3, 64, 1, 77, 0, 150]
    B = len(first)
    tot = [a + b for a, b in zip(first, second)]
    N = sum(-(-t // bs) for t in tot) + 8
    order = rng.permutation(N)
    width = max(-(-t // bs) for t in tot)
    eng = PagedKVEngine(N, hkv, bs, D, TORCH_DTYPE[dtype], B, width, order,
                        fill_bits=synth.POISON_BITS[dtype], num_q_heads=hq)
    om = oracle.BlockManager(N, bs, order)
    okc, ovc = oracle.new_pool(N, hkv, bs, D, synth.poison_array((), dtype))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    od = None if out_dtype is None else TORCH_DTYPE[out_dtype]
    for chunk in (first, second):
        T = sum(chunk)
        k = synth.normal(rng, (T, hkv, D), dtype)
        v = synth.normal(rng, (T, hkv, D), dtype)
        q = synth.normal(rng, (T, hq, D), dtype)
        slots = []
        for b, n in enumerate(chunk):
            slots += (om.append_tokens(b, n) if om.is_live(b) else om.allocate_for_prefill(b, n))
        oracle.write_kv(k, v, slots, okc, ovc, bs)
        qs = np.concatenate([[0], np.cumsum(chunk)])
        lens = om.context_lens(list(range(B)))
        ref = oracle.prefill_attention(q, qs, okc, ovc, om.block_tables(list(range(B)), width, -1), lens,
                                       scale, dtype)
        out = None if od is None else torch.empty((T, hq, D), dtype=od, device="cuda")
        got = eng.prefill_chunk(list(range(B)), list(range(B)), chunk, to_device(k, dtype),
                                to_device(v, dtype), to_device(q, dtype), scale, out=out)
        torch.cuda.synchronize()
        err = np.abs(got.double().cpu().numpy() - ref).max()
        tol = (1e-5 if dtype == "f32" else 2e-3) if od is None else 2e-3 + np.abs(ref).max() * 2.0 ** -8
        _banner(f"prefill {dtype} hq={hq} bs={bs} D={D} chunk {chunk}: max abs err {err:.3e}")
        assert err <= tol, err


def test_prefill_edge_cases():
    """Rows before the first position give zeros, empty chunks write
    nothing, and a one-row chunk agrees with the decode kernel."""
    rng = np.random.default_rng(90)
    N, hkv, hq, bs, D = 16, 4, 28, 16, 128
    pool, kc, vc = pkv.new_pool(N, hkv, bs, D, torch.bfloat16, "cuda")
    kc.copy_(to_device(synth.normal(rng, (N, hkv, bs, D), "bf16"), "bf16"))
    vc.copy_(to_device(synth.normal(rng, (N, hkv, bs, D), "bf16"), "bf16"))
    tables = torch.tensor([[3, 7, 1], [0, 2, 4], [5, 6, 8]], dtype=torch.int32, device="cuda")
    lens = torch.tensor([10, 40, 33], dtype=torch.int32, device="cuda")
    chunk = [14, 0, 1]                          # 14 rows over 10 keys: the first 4 see nothing
    qs = torch.tensor([0, 14, 14, 15], dtype=torch.int32, device="cuda")
    q = torch.randn((15, hq, D), device="cuda").to(torch.bfloat16)
    out = pkv.paged_prefill_attention(q, qs, kc, vc, tables, lens, 0.088, max_q_len=14, max_context_len=48)
    torch.cuda.synchronize()
    ref = oracle.prefill_attention(q.view(torch.int16).cpu().numpy().view(np.uint16), [0, 14, 14, 15],
                                   kc.contiguous().view(torch.int16).cpu().numpy().view(np.uint16),
                                   vc.contiguous().view(torch.int16).cpu().numpy().view(np.uint16),
                                   tables.cpu().numpy(), [10, 40, 33], 0.088, "bf16")
    got = out.double().cpu().numpy()
    assert np.all(got[:4] == 0.0)
    assert np.abs(got - ref).max() <= 2e-3
    dec = pkv.paged_decode_attention(q[14:15].contiguous(), kc, vc, tables[2:3].contiguous(), lens[2:3].contiguous(),
                                     0.088, max_context_len=48)
    torch.cuda.synchronize()
    assert (dec[0] - out[14]).abs().max().item() <= 2e-3


@pytest.mark.parametrize("hq,hkv,bs,out_dtype,dt,D", [(28, 4, 16, None, "bf16", 128), (12, 2, 32, "bf16", "bf16", 128),
                                                     (28, 4, 16, None, "f16", 128), (12, 2, 32, "f16", "f16", 128),
                                                     (8, 2, 16, None, "bf16", 64), (8, 4, 8, "bf16", "bf16", 128)])
def test_fp8_chunked_prefill_matches_oracle(hq, hkv, bs, out_dtype, dt, D):
    """Chunked prefill over an 8-bit pool (paged_prefill_attention_fp8:
    with bf16 queries, head_dim 128 and block_size a multiple of 16 the
    blocks dequantised into a bf16 staging, then the matrix-core kernel;
    otherwise the codes read in place by the generic kernel): the quantising
    writes bit for bit (codes and scale bytes, poison included) and the
    attention within 2e-3 of the oracle's 8-bit prefill attention, over two
    chunks per sequence, with bf16 and with fp16 rows and queries."""
    from oracle import quant
    from paged_kv_cache_128_amd.engine import PagedKVEngine
    _banner(f"fp8 prefill hq={hq} hkv={hkv} bs={bs} D={D} out={out_dtype} {dt}")
    rng = np.random.default_rng(90 + hq + D + bs)
    first = [1, 37, 64, 130, 200, 5]
    second = [3, 64, 1, 77, 0, 150]
    B = len(first)
    tot = [a + b for a, b in zip(first, second)]
    N = sum(-(-t // bs) for t in tot) + 8
    order = rng.permutation(N)
    width = max(-(-t // bs) for t in tot)
    eng = PagedKVEngine(N, hkv, bs, D, torch.float8_e4m3fn, B, width, order, fill_bits=0, num_q_heads=hq)
    om = oracle.BlockManager(N, bs, order)
    o = quant.new_fp8_pool(N, hkv, bs, D)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    od = None if out_dtype is None else TORCH_DTYPE[out_dtype]
    for chunk in (first, second):
        T = sum(chunk)
        k = synth.normal(rng, (T, hkv, D), dt)
        v = synth.normal(rng, (T, hkv, D), dt)
        q = synth.normal(rng, (T, hq, D), dt)
        slots = []
        for b, n in enumerate(chunk):
            slots += (om.append_tokens(b, n) if om.is_live(b) else om.allocate_for_prefill(b, n))
        quant.write_kv_fp8(oracle.widen(k, dt).astype(np.float32), oracle.widen(v, dt).astype(np.float32),
                           slots, *o, bs)
        qs = np.concatenate([[0], np.cumsum(chunk)])
        ref = quant.prefill_attention_fp8(q, dt, qs, *o, om.block_tables(list(range(B)), width, -1),
                                          om.context_lens(list(range(B))), scale)
        out = None if od is None else torch.empty((T, hq, D), dtype=od, device="cuda")
        got = eng.prefill_chunk(list(range(B)), list(range(B)), chunk, to_device(k, dt),
                                to_device(v, dt), to_device(q, dt), scale, out=out)
        torch.cuda.synchronize()
        for g, w in zip((eng.key_cache, eng.value_cache, eng.key_scales, eng.value_scales), o):
            assert np.array_equal(g.contiguous().view(torch.uint8).cpu().numpy(), w)
        err = np.abs(got.double().cpu().numpy() - ref).max()
        tol = 2e-3 if od is None else 2e-3 + np.abs(ref).max() * 2.0 ** (-8 if dt == "bf16" else -11)
        _banner(f"fp8 prefill chunk {chunk}: max abs err {err:.3e}")
        assert err <= tol, err


def test_fp8_prefill_with_fp16_queries_keeps_rows_beyond_fp16_range():
    """8-bit rows written from fp32 tensors can carry scales no 16-bit fp16
    value holds (V rows near 1e6, K rows near 2^-18); an fp16-query prefill
    reads them in place with the row scale applied in fp32, so it agrees
    with the oracle's read-back values as the 8-bit decode does."""
    from oracle import quant
    from paged_kv_cache_128_amd.engine import PagedKVEngine
    rng = np.random.default_rng(97)
    hq, hkv, bs, D = 8, 2, 16, 128
    chunk = [40, 25]
    B, T = len(chunk), sum(chunk)
    N = sum(-(-n // bs) for n in chunk) + 4
    order = rng.permutation(N)
    width = max(-(-n // bs) for n in chunk)
    eng = PagedKVEngine(N, hkv, bs, D, torch.float8_e4m3fn, B, width, order, fill_bits=0, num_q_heads=hq)
    k = (rng.standard_normal((T, hkv, D)) * 2.0 ** -18).astype(np.float32)
    v = (rng.standard_normal((T, hkv, D)) * 1.0e6).astype(np.float32)
    q = synth.normal(rng, (T, hq, D), "f16")
    scale = float(np.float32(1.0 / np.sqrt(D)))
    got = eng.prefill_chunk([0, 1], [0, 1], chunk, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                            to_device(q, "f16"), scale)
    torch.cuda.synchronize()
    om = oracle.BlockManager(N, bs, order)
    o = quant.new_fp8_pool(N, hkv, bs, D)
    slots = om.allocate_for_prefill(0, chunk[0]) + om.allocate_for_prefill(1, chunk[1])
    quant.write_kv_fp8(k, v, slots, *o, bs)
    assert int(o[2][o[2] != 0xFF].max()) - 127 < -15 and int(o[3][o[3] != 0xFF].min()) - 127 > 7
    ref = quant.prefill_attention_fp8(q, "f16", [0, chunk[0], T], *o, om.block_tables([0, 1], width, -1),
                                      om.context_lens([0, 1]), scale)
    err = np.abs(got.double().cpu().numpy() - ref).max()
    _banner(f"fp8 prefill, fp16 queries, rows beyond fp16: max abs err {err:.3e} of max |out| {np.abs(ref).max():.3e}")
    assert err <= 2e-3 + 1e-6 * np.abs(ref).max()


def test_fp8_prefill_refuses_bad_types_and_small_workspace():
    """Host-side checks of paged_prefill_attention_fp8: fp32 queries are
    UNSUPPORTED, an output type other than fp32 or the queries' is INVALID,
    a short workspace for the bf16 staging path is a WORKSPACE error;
    nothing is launched."""
    lib = pkv.load_library()
    N, H, bs, D = 8, 2, 16, 128
    g = pkv.new_fp8_pool(N, H, bs, D, "cuda")
    lay = pkv.cache_layout(g[1], g[2])
    fake = g[0].data_ptr()
    need = lib.paged_prefill_attention_fp8_workspace_size(2, 64, ctypes.byref(lay))
    assert need >= 2 * 4 * 2 * H * bs * D * 2
    args = lambda qd, od, ws, wsb: lib.paged_prefill_attention_fp8(
        fake, od, fake, qd, fake, fake, 2, 16, g[1].data_ptr(), g[2].data_ptr(), g[4].data_ptr(),
        g[5].data_ptr(), ctypes.byref(lay), fake, 4, 4, 64, 0.1, ws, wsb, None)
    assert args(pkv.PKV_F32, pkv.PKV_F32, fake, need) == -5
    assert args(pkv.PKV_F16, pkv.PKV_BF16, fake, need) == -1
    assert args(pkv.PKV_BF16, pkv.PKV_F16, fake, need) == -1
    assert args(pkv.PKV_BF16, pkv.PKV_F32, fake, need - 1) == -7
    # (fp16 queries read the codes in place and take no workspace: not called
    # here, where the pointers are stand-ins)


def _prefill_sweep_shape(i):
    rng = np.random.default_rng(11000 + i)
    dtype = ["bf16", "f16", "f32"][int(rng.integers(0, 3))]
    D = 128 if rng.random() < 0.7 else 64
    bs = [8, 16, 32, 64][int(rng.integers(0, 4))]
    hkv = [1, 2, 4, 8][int(rng.integers(0, 4))]
    hq = hkv * int(rng.integers(1, 9))
    B = int(rng.integers(1, 7))
    rounds = [[int(rng.integers(0, 300)) if rng.random() > 0.15 else int(rng.integers(0, 2)) for _ in range(B)]
              for _ in range(int(rng.integers(1, 4)))]
    return dtype, D, bs, hkv, hq, rounds


@pytest.mark.parametrize("i", range(12))
def test_prefill_seeded_shape_sweep(i):
    """12 seeded prefill shapes (bf16 / fp16 / fp32 KV, D 64 or 128, block
    size 8 to 64, H_kv 1-8, G 1-8, up to 6 sequences admitted and extended
    over one to three rounds of chunks of 0 to 300 rows, fp32 output): the
    pool bit for bit as the oracle's write and every query row against the
    oracle's causal prefill, whichever kernel the shape goes to."""
    from paged_kv_cache_128_amd.engine import PagedKVEngine
    dtype, D, bs, hkv, hq, rounds = _prefill_sweep_shape(i)
    _banner(f"prefill sweep {i}: {dtype} D={D} bs={bs} hkv={hkv} hq={hq} chunks {rounds}")
    rng = np.random.default_rng(12000 + i)
    B = len(rounds[0])
    tot = [sum(r[b] for r in rounds) for b in range(B)]
    N = sum(-(-t // bs) for t in tot) + 8
    order = rng.permutation(N)
    width = max(1, max(-(-t // bs) for t in tot))
    eng = PagedKVEngine(N, hkv, bs, D, TORCH_DTYPE[dtype], B, width, order,
                        fill_bits=synth.POISON_BITS[dtype], num_q_heads=hq)
    om = oracle.BlockManager(N, bs, order)
    okc, ovc = oracle.new_pool(N, hkv, bs, D, synth.poison_array((), dtype))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    tol = 1e-5 if dtype == "f32" else 2e-3
    for chunk in rounds:
        T = sum(chunk)
        k = synth.normal(rng, (T, hkv, D), dtype)
        v = synth.normal(rng, (T, hkv, D), dtype)
        q = synth.normal(rng, (T, hq, D), dtype)
        slots = []
        for b, n in enumerate(chunk):
            slots += (om.append_tokens(b, n) if om.is_live(b) else om.allocate_for_prefill(b, n))
        oracle.write_kv(k, v, slots, okc, ovc, bs)
        qs = np.concatenate([[0], np.cumsum(chunk)])
        lens = om.context_lens(list(range(B)))
        ref = oracle.prefill_attention(q, qs, okc, ovc, om.block_tables(list(range(B)), width, -1), lens,
                                       scale, dtype)
        got = eng.prefill_chunk(list(range(B)), list(range(B)), chunk, to_device(k, dtype),
                                to_device(v, dtype), to_device(q, dtype), scale)
        torch.cuda.synchronize()
        for half, oc in ((0, okc), (1, ovc)):
            g = eng.pool[:, half].contiguous().cpu()
            u = np.uint16 if g.element_size() == 2 else np.uint32
            g = (g.view(torch.int16) if g.element_size() == 2 else g.view(torch.int32)).numpy().view(u)
            assert np.array_equal(g, oc.view(u)), half
        got = got.double().cpu().numpy()
        assert np.all(np.isfinite(got))
        err = float(np.abs(got - ref).max()) if T else 0.0
        _banner(f"  chunk {chunk}: max abs err {err:.3e}")
        assert err <= tol, err


@pytest.mark.parametrize("scale", [1e-3, 4.0, 64.0])
@pytest.mark.parametrize("dtype,bs", [("bf16", 16), ("f16", 32), ("bf16", 8)])
def test_prefill_extreme_score_ranges(scale, dtype, bs):
    """Causal prefill with softmax scales far from 1/sqrt(D): near-uniform
    weights, and scores hundreds of units apart (the running maximum jumping
    past the rescale slack), on the matrix-core kernel (block sizes 16, 32)
    and the generic one (block size 8), against the oracle."""
    from paged_kv_cache_128_amd.engine import PagedKVEngine
    rng = np.random.default_rng(5150 + bs)
    hq, hkv, D = 28, 4, 128
    chunk = [1, 45, 300, 129]
    B = len(chunk)
    N = sum(-(-c // bs) for c in chunk) + 4
    order = rng.permutation(N)
    width = max(-(-c // bs) for c in chunk)
    eng = PagedKVEngine(N, hkv, bs, D, TORCH_DTYPE[dtype], B, width, order,
                        fill_bits=synth.POISON_BITS[dtype], num_q_heads=hq)
    om = oracle.BlockManager(N, bs, order)
    okc, ovc = oracle.new_pool(N, hkv, bs, D, synth.poison_array((), dtype))
    T = sum(chunk)
    k = synth.normal(rng, (T, hkv, D), dtype)
    v = synth.normal(rng, (T, hkv, D), dtype)
    q = synth.normal(rng, (T, hq, D), dtype)
    slots = []
    for b, n in enumerate(chunk):
        slots += om.allocate_for_prefill(b, n)
    oracle.write_kv(k, v, slots, okc, ovc, bs)
    s = float(np.float32(scale))
    ref = oracle.prefill_attention(q, np.concatenate([[0], np.cumsum(chunk)]), okc, ovc,
                                   om.block_tables(list(range(B)), width, -1), om.context_lens(list(range(B))),
                                   s, dtype)
    got = eng.prefill_chunk(list(range(B)), list(range(B)), chunk, to_device(k, dtype), to_device(v, dtype),
                            to_device(q, dtype), s).double().cpu().numpy()
    assert np.all(np.isfinite(got))
    err = float(np.abs(got - ref).max())
    _banner(f"prefill extreme scores {dtype} bs={bs} scale {scale}: max abs err {err:.3e}")
    assert err <= 2e-3, err
