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


_NON_FINITE = {"bf16": (0x7F80, 0xFF80, 0x7FC0), "f16": (np.inf, -np.inf, np.nan),
               "f32": (np.inf, -np.inf, np.nan)}


def _plant_non_finite(a, dtype, t):
    """+inf, -inf and NaN (in a's storage format) into token t's first head:
    its row scale then comes from the finite elements, and those three take
    the NaN code with their sign."""
    a[t, 0, 1], a[t, 0, 4], a[t, 0, 9] = _NON_FINITE[dtype]


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
    _plant_non_finite(k, src, 5)
    _plant_non_finite(v, src, 7)
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


@pytest.mark.parametrize("hq,hkv,B,outliers", [(28, 4, 24, False), (32, 8, 9, False), (12, 2, 40, False),
                                               (28, 4, 24, True)])
def test_fp8_fused_step_equals_separate_launches_and_oracle(hq, hkv, B, outliers):
    """pkv_decode_step_fp8 (the quantising write inside the 8-bit attention
    launch) gives bit for bit the pool, scales, tables, lengths and outputs
    of pkv_decode_write_fp8 followed by the 8-bit attention, over three
    steps that open blocks, and stays within 2e-3 of the oracle.  With
    `outliers`, the last step's new row of every third sequence has its V
    times 2^24 and a key of -4 times the sum of its group's queries (a
    weight of about e^-40 for that step's queries): the row the fused
    launch quantises and places itself then carries the largest V scale of
    its segment."""
    from paged_kv_cache_128_amd.engine import PagedKVEngine
    print(f"[gpu] fp8 fused step hq={hq} hkv={hkv} B={B} outliers={outliers}", flush=True)
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
        if outliers and step == 2:
            qg = _f32(q, "bf16").reshape(B, hkv, hq // hkv, D).sum(axis=2)
            nk[::3] = synth.to_storage(-4.0 * qg[::3], "bf16")
            nv[::3] = synth.to_storage(_f32(nv[::3], "bf16") * np.float32(2.0 ** 24), "bf16")
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


def _fp8_pools(rng, N, H, bs, D, T):
    """Oracle and GPU 8-bit pools, poisoned, then T random rows written at
    random slots by each side's quantising write (bit-exact, tested above)."""
    okc, ovc, oks, ovs = quant.new_fp8_pool(N, H, bs, D)
    g = pkv.new_fp8_pool(N, H, bs, D, "cuda", poison=True)
    k = synth.normal(rng, (T, H, D), "bf16")
    v = synth.normal(rng, (T, H, D), "bf16")
    slots = rng.permutation(N * bs)[:T].astype(np.int64)
    quant.write_kv_fp8(_f32(k, "bf16"), _f32(v, "bf16"), slots, okc, ovc, oks, ovs, bs)
    pkv.paged_kv_write_fp8(to_device(k, "bf16"), to_device(v, "bf16"), torch.from_numpy(slots).cuda(),
                           g[1], g[2], g[4], g[5])
    return (okc, ovc, oks, ovs), g


def _same_pool(g, o):
    okc, ovc, oks, ovs = o
    return (np.array_equal(_u8(g[1]), okc) and np.array_equal(_u8(g[2]), ovc)
            and np.array_equal(_u8(g[4]), oks) and np.array_equal(_u8(g[5]), ovs))


@pytest.mark.parametrize("H,bs,D,npairs", [(4, 16, 128, 300), (2, 32, 64, 3), (8, 8, 128, 1)])
def test_fp8_copy_blocks_bit_exact(H, bs, D, npairs):
    """pkv_copy_blocks_fp8 against the oracle's copy of codes and scale
    bytes, over the whole pool (poison included); an out-of-range pair is
    skipped."""
    _banner(f"fp8 copy_blocks H={H} bs={bs} D={D} pairs={npairs}")
    rng = np.random.default_rng(300 + npairs)
    N = 2 * npairs + 8
    o, g = _fp8_pools(rng, N, H, bs, D, (N * bs * 3) // 4)
    perm = rng.permutation(N)
    src = np.append(perm[:npairs], [N + 5]).astype(np.int32)
    dst = np.append(perm[npairs:2 * npairs], [perm[-1]]).astype(np.int32)
    pkv.copy_blocks_fp8(src, dst, g[1], g[2], g[4], g[5])
    torch.cuda.synchronize()
    quant.copy_blocks_fp8(list(zip(src.tolist(), dst.tolist())), *o)
    assert _same_pool(g, o)


@pytest.mark.parametrize("H,bs,D,n", [(4, 16, 128, 300), (2, 8, 64, 5)])
def test_fp8_gather_scatter_bit_exact(H, bs, D, n):
    """pkv_gather_blocks_fp8 / pkv_scatter_blocks_fp8 against the oracle's
    staging of codes and scale bytes."""
    _banner(f"fp8 gather/scatter H={H} bs={bs} D={D} n={n}")
    rng = np.random.default_rng(400 + n)
    N = n + 20
    o, g = _fp8_pools(rng, N, H, bs, D, N * bs - 7)
    ids = rng.permutation(N)[:n].astype(np.int32)
    codes, scales = pkv.gather_blocks_fp8(ids, g[1], g[2], g[4], g[5])
    torch.cuda.synchronize()
    rc, rs = quant.gather_blocks_fp8(ids, *o)
    assert np.array_equal(_u8(codes), rc) and np.array_equal(scales.cpu().numpy(), rs)
    dst = rng.permutation(N)[:n].astype(np.int32)
    pkv.scatter_blocks_fp8(codes, scales, dst, g[1], g[2], g[4], g[5])
    torch.cuda.synchronize()
    quant.scatter_blocks_fp8(rc, rs, dst, *o)
    assert _same_pool(g, o)


@pytest.mark.parametrize("fused", [True, False])
def test_fp8_shared_prefix_decode_matches_oracle(fused):
    """Prefix sharing on an 8-bit pool through the engine: forks and shorter
    shares, then decode steps whose appends copy shared blocks (codes and
    scales) first; against the oracle replay: the whole pool bit for bit,
    tables, reference counts, and attention within 2e-3."""
    from paged_kv_cache_128_amd.engine import PagedKVEngine
    _banner(f"fp8 sharing decode fused={fused}")
    rng = np.random.default_rng(61 + int(fused))
    hq, hkv, bs, D = 28, 4, 16, 128
    donors = [int(x) for x in rng.integers(1, 300, size=5)]
    donors[1] = 6 * bs
    shares = [(0, donors[0]), (1, donors[1]), (2, max(1, donors[2] // 2)), (3, (donors[3] // bs) * bs),
              (4, donors[4] - 1), (0, 0)]
    steps = 3
    ids = list(range(len(donors) + len(shares)))
    width = int(np.ceil((max(donors) + steps + 1) / bs))
    N = sum(int(np.ceil((L + steps) / bs)) for L in donors) + len(shares) * 2 + 16
    order = rng.permutation(N)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    om = oracle.BlockManager(N, bs, order)
    o = quant.new_fp8_pool(N, hkv, bs, D)
    eng = PagedKVEngine(N, hkv, bs, D, torch.float8_e4m3fn, len(ids), width, order, fill_bits=0,
                        partition_tokens=0, num_q_heads=hq)
    pk = [synth.normal(rng, (L, hkv, D), "bf16") for L in donors]
    pv = [synth.normal(rng, (L, hkv, D), "bf16") for L in donors]
    for sid, L in enumerate(donors):
        quant.write_kv_fp8(_f32(pk[sid], "bf16"), _f32(pv[sid], "bf16"), om.allocate_for_prefill(sid, L), *o, bs)
    eng.prefill_many(list(range(len(donors))), list(range(len(donors))), donors,
                     to_device(np.concatenate(pk), "bf16"), to_device(np.concatenate(pv), "bf16"))
    for j, (donor, n) in enumerate(shares):
        sid = len(donors) + j
        om.share_prefix(donor, sid, n)
        eng.share_prefix(donor, sid, sid, n)
    copies_seen = 0
    for step in range(steps):
        nk = synth.normal(rng, (len(ids), hkv, D), "bf16")
        nv = synth.normal(rng, (len(ids), hkv, D), "bf16")
        q = synth.normal(rng, (len(ids), hq, D), "bf16")
        slots = om.append_slots_for_decode(ids)
        pairs = om.take_copies()
        copies_seen += len(pairs)
        quant.copy_blocks_fp8(pairs, *o)
        quant.write_kv_fp8(_f32(nk, "bf16"), _f32(nv, "bf16"), slots, *o, bs)
        tabs = om.block_tables(ids, width, -1)
        ref = quant.decode_attention_fp8(q, "bf16", *o, tabs, om.context_lens(ids), scale)
        out = eng.decode_step(np.array(ids, np.int64), to_device(nk, "bf16"), to_device(nv, "bf16"),
                              to_device(q, "bf16"), scale, fused=fused)
        torch.cuda.synchronize()
        assert [eng.manager.ref_count(b) for b in range(N)] == om.ref, step
        assert np.array_equal(eng.tables.cpu().numpy(), tabs), step
        assert _same_pool((eng.pool, eng.key_cache, eng.value_cache, eng.scales, eng.key_scales,
                           eng.value_scales), o), step
        err = np.abs(out.double().cpu().numpy() - ref).max()
        _banner(f"fp8 sharing step {step}: copies {len(pairs)}, max abs err {err:.3e}")
        assert err <= 2e-3, (step, err)
    assert copies_seen > 0


def test_fp8_engine_swap_round_trip_is_bit_exact():
    """Swap of an 8-bit sequence through pinned host memory: after its
    blocks are reused by another sequence and it comes back on other
    blocks, its attention output is bit for bit what it was."""
    from paged_kv_cache_128_amd.engine import PagedKVEngine
    _banner("fp8 engine swap round trip")
    rng = np.random.default_rng(72)
    B, hq, hkv, bs, D = 6, 28, 4, 16, 128
    lens = rng.integers(20, 400, B)
    N = int(np.ceil(lens / bs).sum()) + 40
    eng = PagedKVEngine(N, hkv, bs, D, torch.float8_e4m3fn, B + 1, N, rng.permutation(N), num_q_heads=hq)
    k = to_device(synth.normal(rng, (int(lens.sum()), hkv, D), "bf16"), "bf16")
    v = to_device(synth.normal(rng, (int(lens.sum()), hkv, D), "bf16"), "bf16")
    eng.prefill_many(list(range(B)), list(range(B)), [int(x) for x in lens], k, v)
    q = to_device(synth.normal(rng, (B, hq, D), "bf16"), "bf16")
    d_lens = torch.from_numpy(lens.astype(np.int32)).cuda()
    before = eng.attend(q, d_lens, 0.088, int(lens.max())).clone()
    old_table = eng.manager.block_table(2)
    host = eng.swap_out(2)
    assert isinstance(host, tuple) and host[0].is_pinned() and host[1].is_pinned()
    n_other = eng.manager.num_free_blocks() * bs
    eng.prefill(99, B, to_device(synth.normal(rng, (n_other, hkv, D), "bf16"), "bf16"),
                to_device(synth.normal(rng, (n_other, hkv, D), "bf16"), "bf16"))
    assert set(eng.manager.block_table(99)) & set(old_table)
    eng.free(99)
    eng.manager.allocate_for_prefill(100, 5 * bs)
    eng.swap_in(2, 2, host)
    assert eng.manager.block_table(2) != old_table
    after = eng.attend(q, d_lens, 0.088, int(lens.max()))
    torch.cuda.synchronize()
    assert torch.equal(before.view(torch.int32), after.view(torch.int32))


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float8_e4m3fn])
def test_event_timed_steps_equal_plain_steps(dt, fused):
    """decode_step with timing events (three: split at the partial / merge
    boundary; two: around the whole step, a separate write launch included)
    gives bit for bit the outputs, cache and tables of plain decode steps,
    with the step's write inside the attention launch or in its own, and the
    events measure."""
    from paged_kv_cache_128_amd.engine import PagedKVEngine
    _banner(f"event-timed steps {dt} fused={fused}")
    rng = np.random.default_rng(91)
    B, hq, hkv, bs, D = 10, 28, 4, 16, 128
    lens = rng.integers(1, 200, B)
    N = int(np.ceil((lens + 4) / bs).sum()) + 8
    order = rng.permutation(N)
    width = int(np.ceil((lens.max() + 4) / bs))
    engs = [PagedKVEngine(N, hkv, bs, D, dt, B, width, order, fill_bits=0, partition_tokens=0, num_q_heads=hq)
            for _ in range(2)]
    k0 = to_device(synth.normal(rng, (int(lens.sum()), hkv, D), "bf16"), "bf16")
    v0 = to_device(synth.normal(rng, (int(lens.sum()), hkv, D), "bf16"), "bf16")
    for e in engs:
        e.prefill_many(list(range(B)), list(range(B)), [int(x) for x in lens], k0, v0)
    ids = np.arange(B, dtype=np.int64)
    for step in range(4):
        nk = to_device(synth.normal(rng, (B, hkv, D), "bf16"), "bf16")
        nv = to_device(synth.normal(rng, (B, hkv, D), "bf16"), "bf16")
        q = to_device(synth.normal(rng, (B, hq, D), "bf16"), "bf16")
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(3 - step % 2)]
        oa = engs[0].decode_step(ids, nk, nv, q, 0.088, events=evs, fused=fused)
        ob = engs[1].decode_step(ids, nk, nv, q, 0.088, fused=fused)
        torch.cuda.synchronize()
        assert all(a.elapsed_time(b) > 0 for a, b in zip(evs, evs[1:]))
        assert torch.equal(oa.view(torch.int32), ob.view(torch.int32)), step
        assert torch.equal(engs[0].pool.view(torch.uint8), engs[1].pool.view(torch.uint8)), step
        assert torch.equal(engs[0].tables, engs[1].tables) and torch.equal(engs[0].d_lens, engs[1].d_lens)


@pytest.mark.parametrize("q_dtype", ["bf16", "f16"])
def test_fused_fp8_step_codes_non_finite_new_rows_like_the_oracle(q_dtype):
    """The 8-bit decode step quantises the new rows inside the attention
    launch; rows holding +inf, -inf and NaN are stored exactly as the
    oracle's quantiser stores them (NaN codes with their signs, the scale
    from the finite elements).  Only the stored bytes are compared: the
    attention over such rows is NaN."""
    rng = np.random.default_rng(91)
    N, H, hq, bs, D, B = 64, 4, 28, 16, 128, 6
    lens = np.array([17, 1, 33, 64, 5, 48], dtype=np.int32)        # after the append
    codes, kc, vc, scales, ks, vs = pkv.new_fp8_pool(N, H, bs, D, "cuda", poison=True)
    width = 8
    tabs = np.full((B, width), -1, dtype=np.int32)
    perm = rng.permutation(N)
    at = 0
    for b in range(B):
        nb = -(-int(lens[b]) // bs)
        tabs[b, :nb] = perm[at:at + nb]
        at += nb
    slots = np.array([tabs[b, (lens[b] - 1) // bs] * bs + (lens[b] - 1) % bs for b in range(B)], dtype=np.int64)
    k = synth.normal(rng, (B, H, D), q_dtype)
    v = synth.normal(rng, (B, H, D), q_dtype)
    for t in (0, 3):
        _plant_non_finite(k, q_dtype, t)
        _plant_non_finite(v, q_dtype, t)
    q = synth.normal(rng, (B, hq, D), q_dtype)
    tables = torch.from_numpy(tabs).cuda()
    lens_out = torch.zeros(B, dtype=torch.int32, device="cuda")
    assert pkv.attention_path(B, hq, int(lens.max()), kc, 0) == "stream"
    pkv.decode_step_fp8(to_device(q, q_dtype), to_device(k, q_dtype), to_device(v, q_dtype), slots, lens, kc, vc,
                        ks, vs, tables, lens_out, 0.088, int(lens.max()))
    torch.cuda.synchronize()
    okc, ovc, oks, ovs = quant.new_fp8_pool(N, H, bs, D)
    quant.write_kv_fp8(_f32(k, q_dtype), _f32(v, q_dtype), slots, okc, ovc, oks, ovs, bs)
    for b in range(B):
        pb, off = divmod(int(slots[b]), bs)
        for got, want in ((kc, okc), (vc, ovc)):
            assert np.array_equal(_u8(got[pb, :, off]), want[pb, :, off]), b
        for got, want in ((ks, oks), (vs, ovs)):
            assert np.array_equal(_u8(got[pb, :, off]), want[pb, :, off]), b
    assert _u8(kc[int(slots[0]) // bs, 0, int(slots[0]) % bs])[[1, 4, 9]].tolist() == [0x7F, 0xFF, 0x7F]


def _spread_case(pattern, q_dtype, seed):
    """Sequences whose V rows sit at very different scales.  "outliers":
    every 37th token (token 0 included) has its V row times 2^24 and a key
    of -4 times the sum of its group's queries, so its weight is about
    e^-40 and the output is of order 1 (a reference exponent taken from
    the largest row scale alone would push every other weight below f16's
    range); "per-sequence": sequence b's rows all times 2^e_b, e_b from
    -40 to 40; "mixed": every row times 2^k, k uniform in [-12, 12].
    Returns what the test needs and each sequence's tolerance."""
    rng = np.random.default_rng(seed)
    hq, hkv, bs, D = 28, 4, 16, 128
    G = hq // hkv
    lens = np.array([1, 5, 300, 2000, 4096, 17], np.int64)
    B = len(lens)
    q = synth.normal(rng, (B, hq, D), q_dtype)
    qf = oracle.widen(q, q_dtype).astype(np.float32)
    exps = np.array([-40, -20, 0, 20, 40, -8])
    N = int(np.ceil(lens / bs).sum()) + 8
    m = oracle.BlockManager(N, bs, rng.permutation(N))
    okc, ovc, oks, ovs = quant.new_fp8_pool(N, hkv, bs, D)
    codes, kc, vc, scales, ks, vs = pkv.new_fp8_pool(N, hkv, bs, D, "cuda", poison=True)
    tol = np.full(B, 2e-3)
    for b, L in enumerate(lens):
        k = rng.standard_normal((L, hkv, D)).astype(np.float32)
        v = rng.standard_normal((L, hkv, D)).astype(np.float32)
        if pattern == "outliers":
            out_rows = np.arange(0, L, 37)
            v[out_rows] *= np.float32(2.0 ** 24)
            k[out_rows] = -4.0 * qf[b].reshape(hkv, G, D).sum(axis=1)
        elif pattern == "per-sequence":
            v *= np.float32(2.0 ** exps[b])
            tol[b] = 2e-3 * 2.0 ** exps[b]
        else:
            v *= (2.0 ** rng.integers(-12, 13, (L, 1, 1))).astype(np.float32)
            tol[b] = 2e-3 + 2.0 ** -18 * np.abs(v).max()
        slots = np.array(m.allocate_for_prefill(b, int(L)), np.int64)
        quant.write_kv_fp8(k, v, slots, okc, ovc, oks, ovs, bs)
        pkv.paged_kv_write_fp8(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                               torch.from_numpy(slots).cuda(), kc, vc, ks, vs)
    tabs = m.block_tables(list(range(B)), int(np.ceil(lens.max() / bs)), -1)
    return lens, tabs, q, (okc, ovc, oks, ovs), (kc, vc, ks, vs), tol


@pytest.mark.parametrize("pattern,q_dtype", [("outliers", "bf16"), ("outliers", "f16"),
                                             ("per-sequence", "bf16"), ("mixed", "bf16")])
def test_fp8_attention_far_apart_row_scales(pattern, q_dtype):
    """8-bit attention over rows whose V scales lie far apart, against the
    float64 oracle on the read-back values: a row with a huge scale and a
    negligible weight leaves the others' weights intact; sequences scaled
    as a whole by 2^-40 .. 2^40 keep the 2e-3 bound scaled with them; rows
    scaled by 2^-12 .. 2^12 stay within 2e-3 + 2^-18 of their largest
    value.  Long sequences span several ranges, so the merge is in the
    path."""
    _banner(f"fp8 attention, row scales far apart: {pattern}, q={q_dtype}")
    lens, tabs, q, o, g, tol = _spread_case(pattern, q_dtype, 4321)
    scale = float(np.float32(1.0 / np.sqrt(128)))
    ref = quant.decode_attention_fp8(q, q_dtype, *o, tabs, lens, scale)
    out = pkv.paged_decode_attention_fp8(to_device(q, q_dtype), *g, torch.from_numpy(tabs).cuda(),
                                         torch.from_numpy(lens.astype(np.int32)).cuda(), scale,
                                         max_context_len=int(lens.max())).double().cpu().numpy()
    assert np.all(np.isfinite(out))
    err = np.abs(out - ref).max(axis=(1, 2))
    _banner("per sequence: " + ", ".join(f"L={L} err {e:.2e} (tol {t:.1e})" for L, e, t in zip(lens, err, tol)))
    assert np.all(err <= tol), err / tol


@pytest.mark.parametrize("i", range(8))
def test_fp8_seeded_shape_sweep(i):
    """8 seeded shapes of 8-bit attention (bf16 or fp16 queries, H_kv 1-8,
    G 1-8, 2 to 40 sequences up to 2500 tokens, one of them a single token)
    against the float64 oracle on the read-back values."""
    rng = np.random.default_rng(9000 + i)
    q_dtype = ["bf16", "f16"][int(rng.integers(0, 2))]
    hkv = [1, 2, 4, 8][int(rng.integers(0, 4))]
    hq = hkv * int(rng.integers(1, 9))
    B = int(rng.integers(2, 41))
    max_len = int(rng.integers(1, 2501))
    _banner(f"fp8 sweep {i}: q={q_dtype} hq={hq} hkv={hkv} B={B} max_len={max_len}")
    lens, tabs, q, o, g = _fp8_case(q_dtype, hq, hkv, B, max_len, 9100 + i)
    scale = float(np.float32(1.0 / np.sqrt(128)))
    ref = quant.decode_attention_fp8(q, q_dtype, *o, tabs, lens, scale)
    out = pkv.paged_decode_attention_fp8(to_device(q, q_dtype), *g, torch.from_numpy(tabs).cuda(),
                                         torch.from_numpy(lens.astype(np.int32)).cuda(), scale,
                                         max_context_len=int(lens.max())).double().cpu().numpy()
    assert np.all(np.isfinite(out))
    err = float(np.abs(out - ref).max())
    _banner(f"  max abs err {err:.3e}")
    assert err <= 2e-3, err


@pytest.mark.parametrize("scale", [1e-3, 4.0, 64.0])
def test_fp8_extreme_score_ranges(scale):
    """8-bit attention with softmax scales far from 1/sqrt(D) (near-uniform
    weights, and score gaps beyond the rescale slack), against the oracle."""
    lens, tabs, q, o, g = _fp8_case("bf16", 28, 4, 12, 3000, 4343)
    s = float(np.float32(scale))
    ref = quant.decode_attention_fp8(q, "bf16", *o, tabs, lens, s)
    out = pkv.paged_decode_attention_fp8(to_device(q, "bf16"), *g, torch.from_numpy(tabs).cuda(),
                                         torch.from_numpy(lens.astype(np.int32)).cuda(), s,
                                         max_context_len=int(lens.max())).double().cpu().numpy()
    assert np.all(np.isfinite(out))
    err = float(np.abs(out - ref).max())
    _banner(f"fp8 extreme scores, scale {scale}: max abs err {err:.3e}")
    assert err <= 2e-3, err


def test_fp8_very_long_context():
    """One 65,536-token sequence over an 8-bit pool (H 28/4, bf16 queries):
    spread over every range of the launch, its pieces folded by the
    multi-wave merge; against the oracle on the read-back values."""
    rng = np.random.default_rng(8080)
    hq, hkv, bs, D, L = 28, 4, 16, 128, 65536
    N = L // bs + 4
    m = oracle.BlockManager(N, bs, rng.permutation(N))
    okc, ovc, oks, ovs = quant.new_fp8_pool(N, hkv, bs, D)
    codes, kc, vc, scales, ks, vs = pkv.new_fp8_pool(N, hkv, bs, D, "cuda", poison=True)
    slots = np.array(m.allocate_for_prefill(0, L), np.int64)
    k = synth.normal(rng, (L, hkv, D), "bf16")
    v = synth.normal(rng, (L, hkv, D), "bf16")
    quant.write_kv_fp8(_f32(k, "bf16"), _f32(v, "bf16"), slots, okc, ovc, oks, ovs, bs)
    pkv.paged_kv_write_fp8(to_device(k, "bf16"), to_device(v, "bf16"), torch.from_numpy(slots).cuda(),
                           kc, vc, ks, vs)
    tabs = m.block_tables([0], L // bs, -1)
    lens = np.array([L], np.int64)
    q = synth.normal(rng, (1, hq, D), "bf16")
    scale = float(np.float32(1.0 / np.sqrt(D)))
    ref = quant.decode_attention_fp8(q, "bf16", okc, ovc, oks, ovs, tabs, lens, scale)
    out = pkv.paged_decode_attention_fp8(to_device(q, "bf16"), kc, vc, ks, vs, torch.from_numpy(tabs).cuda(),
                                         torch.from_numpy(lens.astype(np.int32)).cuda(), scale,
                                         max_context_len=L).double().cpu().numpy()
    err = float(np.abs(out - ref).max())
    _banner(f"fp8 65536-token context: max abs err {err:.3e}")
    assert err <= 2e-3, err
