"""pkv_decode_step_noalloc (the decode step whose split-K partials live in
the library's own per-GPU device array) against pkv_decode_step with a
caller workspace: two calls in a row on one GPU, the second smaller (fewer
rows, fewer heads, another dtype), each compared bit for bit (output, pool,
tables, lengths) with the workspace entry point on an identical engine, and
with the float64 oracle within the workload's tolerance."""
import numpy as np
import pytest
import torch

import oracle
import synth
import paged_kv_cache_128_amd as pkv
from oracle.replay import decode_state

from gpu_harness import engine_for, to_device

pytestmark = pytest.mark.gpu


def _step(eng, wl, noalloc):
    cfg = wl.cfg
    B = len(wl.context_lens)
    out = torch.full((B, cfg.num_q_heads, cfg.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    eng.decode_step(np.arange(B, dtype=np.int64), to_device(wl.new_k, cfg.dtype), to_device(wl.new_v, cfg.dtype),
                    to_device(wl.q, cfg.dtype), cfg.scale, out=out, noalloc=noalloc)
    torch.cuda.synchronize()
    return out


def test_noalloc_step_equals_workspace_step_twice():
    pkv.load_library()
    for name in ("qwen2_7b_b64", "qwen2_1p5b_b32"):          # the second call is the smaller one
        cfg = synth.CONFIGS[name]
        wl = synth.decode_workload(cfg)
        B = len(wl.context_lens)
        need = pkv.workspace_size(B, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                                  int(wl.context_lens.max()), 0)
        assert 0 < need <= pkv.NOALLOC_SCRATCH_BYTES
        print(f"[gpu] no-alloc step, {name}: B={B}, workspace {need} bytes", flush=True)
        ref_eng = engine_for(wl, partition_tokens=0)
        want = _step(ref_eng, wl, noalloc=False)
        eng = engine_for(wl, partition_tokens=0)
        got = _step(eng, wl, noalloc=True)
        assert torch.equal(got.view(torch.int32), want.view(torch.int32)), name
        assert torch.equal(eng.pool.view(torch.int16), ref_eng.pool.view(torch.int16)), name
        assert torch.equal(eng.tables, ref_eng.tables) and torch.equal(eng.d_lens, ref_eng.d_lens), name
        st = decode_state(wl, width=eng.width)
        ref = oracle.decode_attention(wl.q, st.key_cache, st.value_cache, st.block_tables,
                                      st.context_lens, cfg.scale, cfg.dtype)
        err = float(np.abs(got.double().cpu().numpy() - ref).max())
        print(f"[gpu] no-alloc step, {name}: bit-equal to the workspace step, max abs err {err:.3e}", flush=True)
        assert err <= 2e-3
        del ref_eng, eng
        torch.cuda.empty_cache()


def test_noalloc_refuses_shapes_beyond_its_array():
    """A step whose workspace would exceed the array returns WORKSPACE and
    changes nothing (checked on the host side of the call)."""
    lay = pkv.CacheLayout(num_blocks=8, num_kv_heads=8, block_size=16, head_dim=64, dtype=pkv.PKV_F32,
                          reserved=0, block_stride=2 * 8 * 16 * 64, head_stride=16 * 64)
    # partition path (fp32): B * H_q * P * (D + 2) * 4 bytes with P = 2^20 / 512
    need = pkv.workspace_size(64, 64, 8, 64, 1 << 20, 0)
    assert need > pkv.NOALLOC_SCRATCH_BYTES
    slots = np.zeros(64, dtype=np.int64)
    lens = np.ones(64, dtype=np.int32)
    import ctypes
    st = pkv.load_library().pkv_decode_step_noalloc(
        None, pkv.PKV_F32, None, None, None, pkv._ptr(slots, ctypes.c_int64), pkv._ptr(lens, ctypes.c_int32), 64,
        None, None, ctypes.byref(lay), None, 1 << 16, None, 64, 1 << 20, 0.125, None)
    assert st == -7
