"""GPU parity of swap to host ([impl-detail] "异构内存支持"): the gather and
scatter kernels against the oracle's over the whole pool, and a round trip
through pinned host memory in the engine: after swap-out, reuse of the
released blocks by another sequence, and swap-in onto other blocks, the
attention output is bit for bit what it was before."""
import numpy as np
import pytest
import torch

import oracle
import synth
import paged_kv_cache_128_amd as pkv

from gpu_harness import bits_u, to_device, TORCH_DTYPE

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,H,bs,D,n", [("bf16", 4, 16, 128, 300), ("f32", 2, 32, 64, 5)])
def test_gather_scatter_bit_exact(dtype, H, bs, D, n):
    print(f"[gpu] gather/scatter {dtype} n={n}", flush=True)
    rng = np.random.default_rng(n)
    N = n + 20
    kn = synth.normal(rng, (N, H, bs, D), dtype)
    vn = synth.normal(rng, (N, H, bs, D), dtype)
    pool, kc, vc = pkv.new_pool(N, H, bs, D, TORCH_DTYPE[dtype], "cuda")
    kc.copy_(to_device(kn, dtype))
    vc.copy_(to_device(vn, dtype))
    ids = rng.permutation(N)[:n].astype(np.int32)
    bits = (lambda a: a) if dtype == "bf16" else (lambda a: a.view(np.uint32))
    staged = pkv.gather_blocks(ids, kc, vc)
    torch.cuda.synchronize()
    ref = oracle.gather_blocks(ids, kn, vn)
    assert np.array_equal(bits_u(staged), bits(ref))
    dst = rng.permutation(N)[:n].astype(np.int32)
    pkv.scatter_blocks(staged, dst, kc, vc)
    torch.cuda.synchronize()
    oracle.scatter_blocks(ref, dst, kn, vn)
    assert np.array_equal(bits_u(kc), bits(kn)) and np.array_equal(bits_u(vc), bits(vn))


def test_engine_swap_round_trip_is_bit_exact():
    from paged_kv_cache_128_amd.engine import PagedKVEngine
    print("[gpu] engine swap round trip", flush=True)
    rng = np.random.default_rng(71)
    B, hq, hkv, bs, D = 6, 28, 4, 16, 128
    lens = rng.integers(20, 400, B)
    N = int(np.ceil(lens / bs).sum()) + 40
    width = int(np.ceil(lens.max() / bs))
    eng = PagedKVEngine(N, hkv, bs, D, torch.bfloat16, B + 1, N, rng.permutation(N), num_q_heads=hq)
    k = to_device(synth.normal(rng, (int(lens.sum()), hkv, D), "bf16"), "bf16")
    v = to_device(synth.normal(rng, (int(lens.sum()), hkv, D), "bf16"), "bf16")
    eng.prefill_many(list(range(B)), list(range(B)), [int(x) for x in lens], k, v)
    q = to_device(synth.normal(rng, (B, hq, D), "bf16"), "bf16")
    d_lens = torch.from_numpy(lens.astype(np.int32)).cuda()
    before = eng.attend(q, d_lens, 0.088, int(lens.max())).clone()
    old_table = eng.manager.block_table(2)
    host = eng.swap_out(2)
    # another sequence takes every free block (the released ones sit at the
    # back of the free list) and overwrites them
    n_other = eng.manager.num_free_blocks() * bs
    eng.prefill(99, B, to_device(synth.normal(rng, (n_other, hkv, D), "bf16"), "bf16"),
                to_device(synth.normal(rng, (n_other, hkv, D), "bf16"), "bf16"))
    assert set(eng.manager.block_table(99)) & set(old_table)
    eng.free(99)
    eng.manager.allocate_for_prefill(100, 5 * bs)   # shifts the free list so swap-in lands elsewhere
    eng.swap_in(2, 2, host)
    assert eng.manager.block_table(2) != old_table
    after = eng.attend(q, d_lens, 0.088, int(lens.max()))
    torch.cuda.synchronize()
    assert torch.equal(before.view(torch.int32), after.view(torch.int32))


def test_swap_out_copy_overlaps_later_work():
    """swap_out's device-to-host copy runs on the engine's copy stream: work
    queued after it on the compute stream (fresh allocations the size of the
    staging array, filled with junk; a prompt written over the released
    blocks; an attention launch) neither waits for it nor disturbs what it
    copies."""
    from paged_kv_cache_128_amd.engine import PagedKVEngine
    print("[gpu] swap-out copy overlapping later work", flush=True)
    rng = np.random.default_rng(72)
    hq, hkv, bs, D = 28, 4, 16, 128
    lens = np.array([4096, 300, 700])
    B = len(lens)
    N = int(np.ceil(lens / bs).sum()) + 40
    eng = PagedKVEngine(N, hkv, bs, D, torch.bfloat16, B + 1, N, rng.permutation(N), num_q_heads=hq)
    k = to_device(synth.normal(rng, (int(lens.sum()), hkv, D), "bf16"), "bf16")
    v = to_device(synth.normal(rng, (int(lens.sum()), hkv, D), "bf16"), "bf16")
    eng.prefill_many(list(range(B)), list(range(B)), [int(x) for x in lens], k, v)
    q = to_device(synth.normal(rng, (B, hq, D), "bf16"), "bf16")
    d_lens = torch.from_numpy(lens.astype(np.int32)).cuda()
    before = eng.attend(q, d_lens, 0.088, int(lens.max())).clone()
    ids = np.array(eng.manager.block_table(0), dtype=np.int32)
    ref = pkv.gather_blocks(ids, eng.key_cache, eng.value_cache).clone()
    host = eng.swap_out(0)
    for _ in range(4):
        junk = torch.empty_like(ref)
        junk.view(torch.int16).fill_(-1)
    n_other = eng.manager.num_free_blocks() * bs
    eng.prefill(99, B, to_device(synth.normal(rng, (n_other, hkv, D), "bf16"), "bf16"),
                to_device(synth.normal(rng, (n_other, hkv, D), "bf16"), "bf16"))
    assert set(eng.manager.block_table(99)) & set(ids.tolist())
    d_lens2 = torch.tensor([0, 300, 700], dtype=torch.int32, device="cuda")
    eng.attend(q, d_lens2, 0.088, int(lens.max()))
    eng.wait_swap(0)
    assert torch.equal(host.view(torch.int16), ref.cpu().view(torch.int16))
    eng.free(99)
    eng.swap_in(0, 0, host)
    after = eng.attend(q, d_lens, 0.088, int(lens.max()))
    torch.cuda.synchronize()
    assert torch.equal(before.view(torch.int32), after.view(torch.int32))
