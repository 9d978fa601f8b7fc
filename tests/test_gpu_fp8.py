"""GPU parity of 8-bit KV blocks (PKV_FP8_E4M3) against the oracle
(oracle/quant.py): the quantising writes bit for bit over the whole pool
(codes and scale bytes, poison included), every E4M3 code read back exactly
(one-token attention returns the read-back V row), and 8-bit paged
attention within 2e-3 of the float64 oracle on the read-back values, for
the paired (H_kv <= 4) and unpaired (H_kv = 8) stream layouts and both
query types."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import quant
import paged_kv_cache_128_amd as pkv

from gpu_harness import to_device, TORCH_DTYPE

pytestmark = pytest.mark.gpu


def _banner(msg):
    print(f"[gpu] {msg}", flush=True)


def _f32(a, dtype):
    """Storage array -> the float32 values the write widens it to."""
    return oracle.widen(a, dtype).astype(np.float32)


def _u8(t):
    return t.contiguous().view(torch.uint8).cpu().numpy()


def _special_rows(rng, D):
    rows = [np.zeros(D, np.float32), np.full(D, -0.0, np.float32)]
    r = rng.standard_normal(D).astype(np.float32)
    r[0] = 448.0 * 8.0                               # amax exactly 448 * 2^3
    rows.append(r)
    rows.append((rng.standard_normal(D) * 2.0 ** 20).astype(np.float32))
    rows.append((rng.standard_normal(D) * 2.0 ** -20).astype(np.float32))
    t = np.array([(quant.e4m3_decode(c) + quant.e4m3_decode(c + 1)) / 2 for c in range(0x40, 0x40 + D // 2)],
                 np.float32)
    rows.append(np.concatenate([t, -t])[:D])         # ties at scale 2^0 (amax < 448)
    return np.stack(rows)


@pytest.mark.parametrize("src,H,bs,D,T", [("bf16", 4, 16, 128, 200), ("f16", 2, 16, 128, 37),
                                          ("f32", 8, 32, 64, 50)])
def test_fp8_write_bit_exact(src, H, bs, D, T):
    _banner(f"fp8 write {src} H={H} bs={bs} D={D} T={T}")
    rng = np.random.default_rng(T)
    N = T // bs + 6
    k = synth.normal(rng, (T, H, D), src)
    v = synth.normal(rng, (T, H, D), src)
    if src == "f32":                                 # special rows go through exactly as written
        sp = _special_rows(rng, D)
        k[:len(sp), 0] = sp
        v[:len(sp), H - 1] = -sp
    slots = rng.permutation(N * bs)[:T].astype(np.int64)
    slots[3] = N * bs + 5                            # outside the pool: skipped
    codes, kc, vc, scales, ks, vs = pkv.new_fp8_pool(N, H, bs, D, "cuda", poison=True)
    pkv.paged_kv_write_fp8(to_device(k, src), to_device(v, src), torch.from_numpy(slots).cuda(),
                           kc, vc, ks, vs)
    torch.cuda.synchronize()
    okc, ovc, oks, ovs = quant.new_fp8_pool(N, H, bs, D)
    quant.write_kv_fp8(_f32(k, src), _f32(v, src), slots, okc, ovc, oks, ovs, bs)
    assert np.array_equal(_u8(kc), okc) and np.array_equal(_u8(vc), ovc)
    assert np.array_equal(_u8(ks), oks) and np.array_equal(_u8(vs), ovs)


def test_fp8_decode_write_publishes_tables_and_lens():
    rng = np.random.default_rng(2)
    N, H, bs, D, n = 40, 4, 16, 128, 9
    k = synth.normal(rng, (n, H, D), "bf16")
    v = synth.normal(rng, (n, H, D), "bf16")
    slots = (rng.permutation(N)[:n] * bs + rng.integers(0, bs, n)).astype(np.int64)
    lens = rng.integers(1, 200, n).astype(np.int32)
    codes, kc, vc, scales, ks, vs = pkv.new_fp8_pool(N, H, bs, D, "cuda", poison=True)
    tables = torch.full((n, 16), -1, dtype=torch.int32, device="cuda")
    lens_out = torch.zeros(n, dtype=torch.int32, device="cuda")
    pkv.decode_write_fp8(to_device(k, "bf16"), to_device(v, "bf16"), slots, lens, kc, vc, ks, vs,
                         block_tables=tables, lens_out=lens_out)
    torch.cuda.synchronize()
    okc, ovc, oks, ovs = quant.new_fp8_pool(N, H, bs, D)
    quant.write_kv_fp8(_f32(k, "bf16"), _f32(v, "bf16"), slots, okc, ovc, oks, ovs, bs)
    assert np.array_equal(_u8(kc), okc) and np.array_equal(_u8(vs), ovs)
    assert np.array_equal(lens_out.cpu().numpy(), lens)
    tab = tables.cpu().numpy()
    for i in range(n):
        assert tab[i, (lens[i] - 1) // bs] == slots[i] // bs


def test_every_code_reads_back_exactly():
    """A sequence of one token attends to itself with weight 1: the output is
    its read-back V row.  Rows built from every finite E4M3 value (row max
    448, so the scale is 2^0 and each value is its own code) check the
    kernel's decoding of every code against the E4M3 definition."""
    H, bs, D, hq = 4, 16, 128, 28
    vals = np.array([quant.e4m3_decode(c) for c in range(0x7F)], np.float32)   # 0 .. 448
    row_pos = np.concatenate([vals, [448.0]])[:D].astype(np.float32)
    row_neg = -np.concatenate([vals[1:], [448.0, 448.0]])[:D].astype(np.float32)
    B = 2
    v = np.zeros((B, H, D), np.float32)
    v[0, :] = row_pos
    v[1, :] = row_neg
    k = np.ones((B, H, D), np.float32)
    N = 4
    codes, kc, vc, scales, ks, vs = pkv.new_fp8_pool(N, H, bs, D, "cuda", poison=True)
    slots = np.array([0, 2 * bs], np.int64)
    pkv.paged_kv_write_fp8(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                           torch.from_numpy(slots).cuda(), kc, vc, ks, vs)
    q = torch.randn((B, hq, D), device="cuda").to(torch.bfloat16)
    tables = torch.tensor([[0], [2]], dtype=torch.int32, device="cuda")
    lens = torch.ones(B, dtype=torch.int32, device="cuda")
    out = pkv.paged_decode_attention_fp8(q, kc, vc, ks, vs, tables, lens, 0.1, max_context_len=bs)
    torch.cuda.synchronize()
    okc, ovc, oks, ovs = quant.new_fp8_pool(N, H, bs, D)
    quant.write_kv_fp8(k, v, slots, okc, ovc, oks, ovs, bs)
    assert set(np.unique(ovc[0, 0, 0]).tolist()) | set(np.unique(ovc[2, 0, 0]).tolist()) >= \
        set(range(0x7F)) | set(range(0x81, 0xFF))
    got = out.cpu().numpy()
    for b, pb in enumerate((0, 2)):
        ref = quant.dequantize(ovc[pb, :, 0], ovs[pb, :, 0])
        for qh in range(hq):
            assert np.array_equal(got[b, qh].astype(np.float64), ref[qh // (hq // H)]), (b, qh)


def _fp8_case(q_dtype, hq, hkv, B, max_len, seed):
    rng = np.random.default_rng(seed)
    bs, D = 16, 128
    lens = rng.integers(1, max_len + 1, B)
    lens[0] = 1
    lens[1] = max_len
    N = int(np.ceil(lens / bs).sum()) + 8
    m = oracle.BlockManager(N, bs, rng.permutation(N))
    okc, ovc, oks, ovs = quant.new_fp8_pool(N, hkv, bs, D)
    codes, kc, vc, scales, ks, vs = pkv.new_fp8_pool(N, hkv, bs, D, "cuda", poison=True)
    for b, L in enumerate(lens):
        slots = np.array(m.allocate_for_prefill(b, int(L)), np.int64)
        k = synth.normal(rng, (L, hkv, D), "bf16")
        v = synth.normal(rng, (L, hkv, D), "bf16")
        quant.write_kv_fp8(_f32(k, "bf16"), _f32(v, "bf16"), slots, okc, ovc, oks, ovs, bs)
        pkv.paged_kv_write_fp8(to_device(k, "bf16"), to_device(v, "bf16"), torch.from_numpy(slots).cuda(),
                               kc, vc, ks, vs)
    width = int(np.ceil(lens.max() / bs))
    tabs = m.block_tables(list(range(B)), width, -1)
    q = synth.normal(rng, (B, hq, D), q_dtype)
    return lens, tabs, q, (okc, ovc, oks, ovs), (kc, vc, ks, vs)


@pytest.mark.parametrize("q_dtype,hq,hkv,B,max_len", [("bf16", 28, 4, 24, 700), ("f16", 12, 2, 32, 300),
                                                      ("bf16", 32, 8, 16, 500), ("bf16", 8, 1, 5, 2000)])
def test_fp8_attention_matches_oracle(q_dtype, hq, hkv, B, max_len):
    _banner(f"fp8 attention q={q_dtype} hq={hq} hkv={hkv} B={B} max_len={max_len}")
    lens, tabs, q, o, g = _fp8_case(q_dtype, hq, hkv, B, max_len, 60 + hq + B)
    scale = float(np.float32(1.0 / np.sqrt(128)))
    ref = quant.decode_attention_fp8(q, q_dtype, *o, tabs, lens, scale)
    out = pkv.paged_decode_attention_fp8(to_device(q, q_dtype), *g, torch.from_numpy(tabs).cuda(),
                                         torch.from_numpy(lens.astype(np.int32)).cuda(), scale,
                                         max_context_len=int(lens.max()))
    torch.cuda.synchronize()
    err = np.abs(out.double().cpu().numpy() - ref).max()
    _banner(f"max abs err {err:.3e}")
    assert err <= 2e-3, err
    # the two launches one by one give the same bits
    ws = torch.empty(pkv.workspace_size(B, hq, hkv, 128, int(lens.max())), dtype=torch.uint8, device="cuda")
    out2 = torch.empty_like(out)
    for ph in ("partial", "merge"):
        pkv.paged_decode_attention_fp8(to_device(q, q_dtype), *g, torch.from_numpy(tabs).cuda(),
                                       torch.from_numpy(lens.astype(np.int32)).cuda(), scale, out=out2,
                                       max_context_len=int(lens.max()), workspace=ws, phase=ph)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), out2.view(torch.int32))


def test_fp8_engine_decode_steps_match_oracle():
    """The engine with an 8-bit pool: prefill, then three decode steps
    (append, quantising step write with table and length publication,
    attention), against the oracle replay of the same ops."""
    from paged_kv_cache_128_amd.engine import PagedKVEngine
    rng = np.random.default_rng(77)
    B, hq, hkv, bs, D = 12, 28, 4, 16, 128
    lens = rng.integers(1, 300, B)
    lens[::4] = 16 * rng.integers(1, 10, len(lens[::4]))
    N = int(np.ceil((lens + 4) / bs).sum()) + 8
    order = rng.permutation(N)
    width = int(np.ceil((lens.max() + 4) / bs))
    eng = PagedKVEngine(N, hkv, bs, D, torch.float8_e4m3fn, B, width, order, fill_bits=0,
                        partition_tokens=0, num_q_heads=hq)
    om = oracle.BlockManager(N, bs, order)
    okc, ovc, oks, ovs = quant.new_fp8_pool(N, hkv, bs, D)
    k0 = synth.normal(rng, (int(lens.sum()), hkv, D), "bf16")
    v0 = synth.normal(rng, (int(lens.sum()), hkv, D), "bf16")
    at = 0
    for b, L in enumerate(lens):
        sl = om.allocate_for_prefill(b, int(L))
        quant.write_kv_fp8(_f32(k0[at:at + L], "bf16"), _f32(v0[at:at + L], "bf16"), sl, okc, ovc, oks, ovs, bs)
        at += L
    eng.prefill_many(list(range(B)), list(range(B)), [int(x) for x in lens], to_device(k0, "bf16"),
                     to_device(v0, "bf16"))
    ids = list(range(B))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    for step in range(3):
        nk = synth.normal(rng, (B, hkv, D), "bf16")
        nv = synth.normal(rng, (B, hkv, D), "bf16")
        q = synth.normal(rng, (B, hq, D), "bf16")
        slots = om.append_slots_for_decode(ids)
        quant.write_kv_fp8(_f32(nk, "bf16"), _f32(nv, "bf16"), slots, okc, ovc, oks, ovs, bs)
        ref = quant.decode_attention_fp8(q, "bf16", okc, ovc, oks, ovs, om.block_tables(ids, width, -1),
                                         om.context_lens(ids), scale)
        out = eng.decode_step(np.array(ids, np.int64), to_device(nk, "bf16"), to_device(nv, "bf16"),
                              to_device(q, "bf16"), scale)
        torch.cuda.synchronize()
        assert np.array_equal(_u8(eng.key_cache), okc) and np.array_equal(_u8(eng.value_cache), ovc)
        assert np.array_equal(_u8(eng.key_scales), oks) and np.array_equal(_u8(eng.value_scales), ovs)
        assert np.array_equal(eng.tables.cpu().numpy(), om.block_tables(ids, width, -1))
        err = np.abs(out.double().cpu().numpy() - ref).max()
        _banner(f"fp8 engine step {step}: max abs err {err:.3e}")
        assert err <= 2e-3, (step, err)


@pytest.mark.parametrize("hq,hkv,B", [(28, 4, 24), (32, 8, 9), (12, 2, 40)])
def test_fp8_fused_step_equals_separate_launches_and_oracle(hq, hkv, B):
    """pkv_decode_step_fp8 (the quantising write inside the 8-bit attention
    launch) gives bit for bit the pool, scales, tables, lengths and outputs
    of pkv_decode_write_fp8 followed by the 8-bit attention, over three
    steps that open blocks, and stays within 2e-3 of the oracle."""
    from paged_kv_cache_128_amd.engine import PagedKVEngine
    print(f"[gpu] fp8 fused step hq={hq} hkv={hkv} B={B}", flush=True)
    rng = np.random.default_rng(40 + B)
    bs, D = 16, 128
    lens = rng.integers(1, 300, size=B)
    lens[::4] = 16 * rng.integers(1, 12, size=len(lens[::4]))
    N = int(np.ceil((lens + 4) / bs).sum()) + 16
    order = rng.permutation(N)
    width = int(np.ceil((lens.max() + 4) / bs))
    engs = [PagedKVEngine(N, hkv, bs, D, torch.float8_e4m3fn, B, width, order, fill_bits=0,
                          partition_tokens=0, num_q_heads=hq) for _ in range(2)]
    om = oracle.BlockManager(N, bs, order)
    okc, ovc, oks, ovs = quant.new_fp8_pool(N, hkv, bs, D)
    k0 = synth.normal(rng, (int(lens.sum()), hkv, D), "bf16")
    v0 = synth.normal(rng, (int(lens.sum()), hkv, D), "bf16")
    at = 0
    for b, L in enumerate(lens):
        sl = om.allocate_for_prefill(b, int(L))
        quant.write_kv_fp8(_f32(k0[at:at + L], "bf16"), _f32(v0[at:at + L], "bf16"), sl, okc, ovc, oks, ovs, bs)
        at += L
    for e in engs:
        e.prefill_many(list(range(B)), list(range(B)), [int(x) for x in lens], to_device(k0, "bf16"),
                       to_device(v0, "bf16"))
    ids = np.arange(B, dtype=np.int64)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    for step in range(3):
        nk = synth.normal(rng, (B, hkv, D), "bf16")
        nv = synth.normal(rng, (B, hkv, D), "bf16")
        q = synth.normal(rng, (B, hq, D), "bf16")
        slots = om.append_slots_for_decode(list(range(B)))
        quant.write_kv_fp8(_f32(nk, "bf16"), _f32(nv, "bf16"), slots, okc, ovc, oks, ovs, bs)
        ref = quant.decode_attention_fp8(q, "bf16", okc, ovc, oks, ovs, om.block_tables(list(range(B)), width, -1),
                                         om.context_lens(list(range(B))), scale)
        oa = engs[0].decode_step(ids, to_device(nk, "bf16"), to_device(nv, "bf16"), to_device(q, "bf16"), scale,
                                 fused=True)
        ob = engs[1].decode_step(ids, to_device(nk, "bf16"), to_device(nv, "bf16"), to_device(q, "bf16"), scale,
                                 fused=False)
        torch.cuda.synchronize()
        for x, y in ((engs[0].pool, engs[1].pool), (engs[0].scales, engs[1].scales)):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), step
        assert np.array_equal(_u8(engs[0].key_cache), okc) and np.array_equal(_u8(engs[0].value_scales), ovs)
        assert torch.equal(engs[0].tables, engs[1].tables) and torch.equal(engs[0].d_lens, engs[1].d_lens)
        assert torch.equal(oa.view(torch.int32), ob.view(torch.int32)), step
        err = np.abs(oa.double().cpu().numpy() - ref).max()
        print(f"[gpu] fp8 fused step {step}: max abs err {err:.3e}", flush=True)
        assert err <= 2e-3, err
