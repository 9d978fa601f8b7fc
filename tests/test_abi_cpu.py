"""The C-ABI library loads on a CPU-only host and exports every entry point
include/pkv.h declares; host-side argument checks of the GPU entry points
reject bad input before anything reaches the GPU.  CPU only."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_128_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "pkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = "\n".join(line for line in text.splitlines() if not line.lstrip().startswith("#"))
    names = re.findall(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*\([^;{()]*\)\s*;", text)
    return sorted(set(n for n in names if n not in ("if", "sizeof")))


def test_every_declared_symbol_is_exported():
    lib = pkv.load_library()
    names = _declared_functions()
    assert len(names) >= 20, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in pkv.h but not exported"
    # the binding wraps exactly the declared ABI
    assert set(pkv.SIGNATURES) == set(names)


def test_status_strings_and_version():
    lib = pkv.load_library()
    for code in range(-8, 1):
        assert lib.pkv_status_string(code)
    assert b"unknown" in lib.pkv_status_string(-99)
    assert pkv.version().startswith("pkv ")


def _layout(**kw):
    base = dict(num_blocks=64, num_kv_heads=4, block_size=16, head_dim=64, dtype=pkv.PKV_F32,
                reserved=0, block_stride=2 * 4 * 16 * 64, head_stride=16 * 64)
    base.update(kw)
    return pkv.CacheLayout(**base)


def test_pool_span_and_layout_validation():
    lib = pkv.load_library()
    lay = _layout()
    span = lib.pkv_pool_span_bytes(ctypes.byref(lay))
    assert span == ((64 - 1) * 2 * 4 * 16 * 64 + 3 * 16 * 64 + 16 * 64) * 4
    for bad in (dict(num_blocks=0), dict(head_stride=10), dict(block_stride=16 * 64),
                dict(dtype=7), dict(reserved=1)):
        assert lib.pkv_pool_span_bytes(ctypes.byref(_layout(**bad))) == 0


def test_attention_argument_checks_need_no_gpu():
    lib = pkv.load_library()
    lay = _layout()
    fake = ctypes.c_void_p(0x1000)
    def call(**kw):
        a = dict(out=fake, out_dtype=pkv.PKV_F32, q=fake, kc=fake, vc=fake, tables=fake, stride=4,
                 lens=fake, B=4, hq=4, max_len=64, scale=0.125, lay=lay, part=0, ws=None, wsb=0)
        a.update(kw)
        return lib.paged_decode_attention(a["out"], a["out_dtype"], a["q"], a["kc"], a["vc"],
                                          a["tables"], a["stride"], a["lens"], a["B"], a["hq"],
                                          a["max_len"], a["scale"], ctypes.byref(a["lay"]),
                                          a["part"], a["ws"], a["wsb"], None)
    assert call(hq=6) == -1                          # H_q % H_kv != 0
    assert call(max_len=65) == -1                    # beyond table width * bs
    assert call(out_dtype=pkv.PKV_BF16) == -1        # out dtype neither f32 nor cache dtype
    assert call(hq=4 * 9) == -5                      # group 9 > 8
    assert call(lay=_layout(head_dim=96, head_stride=16 * 96, block_stride=8 * 16 * 96)) == -5
    assert call(lay=_layout(block_size=8, head_stride=8 * 64, block_stride=8 * 8 * 64), max_len=32) == -5
    assert call(part=24) == -1                       # partition not a multiple of 16
    assert call(max_len=64, stride=4, part=16) == -7 # needs workspace, none given
    assert call(B=0) == 0                            # nothing to do
    assert call(scale=float("nan")) == -1


def test_workspace_size_formula():
    assert pkv.workspace_size(8, 32, 8, 128, 32768, 512) == 8 * 32 * 64 * 130 * 4
    assert pkv.workspace_size(4, 4, 4, 64, 512, 512) == 0
    assert pkv.workspace_size(4, 4, 4, 64, 513, 512) == 4 * 4 * 2 * 66 * 4


def test_write_argument_checks_need_no_gpu():
    lib = pkv.load_library()
    fake = ctypes.c_void_p(0x1000)
    lay = _layout()
    assert lib.paged_kv_write(fake, fake, fake, -1, fake, fake, ctypes.byref(lay), None) == -1
    assert lib.paged_kv_write(fake, fake, fake, 0, fake, fake, ctypes.byref(lay), None) == 0
    odd = _layout(dtype=pkv.PKV_BF16, head_dim=4, head_stride=16 * 8, block_stride=4 * 16 * 8)
    assert lib.paged_kv_write(fake, fake, fake, 3, fake, fake, ctypes.byref(odd), None) == -5
    assert lib.pkv_update_block_tables(fake, 4, 0, None, fake, fake, 3, 16, None) == -1
    assert lib.pkv_update_block_tables(fake, -1, 4, None, fake, fake, 3, 16, None) == -1


def test_table_row_copy_argument_checks_need_no_gpu():
    lib = pkv.load_library()
    fake = ctypes.c_void_p(0x1000)
    assert lib.pkv_copy_table_rows(fake, 8, 4, None, fake, 8, 4, None, -1, 8, None) == -1   # n < 0
    assert lib.pkv_copy_table_rows(fake, 4, 4, None, fake, 8, 4, None, 2, 8, None) == -1    # width > dst stride
    assert lib.pkv_copy_table_rows(fake, 8, 4, None, fake, 4, 4, None, 2, 8, None) == -1    # width > src stride
    assert lib.pkv_copy_table_rows(None, 8, 4, None, fake, 8, 4, None, 2, 8, None) == -1    # no table
    assert lib.pkv_copy_table_rows(fake, 8, 4, None, fake, 8, 4, None, 0, 8, None) == 0     # nothing to do


def test_manager_create_rejects_bad_arguments():
    with pytest.raises(ValueError):
        pkv.KVBlockManager(0, 16)
    with pytest.raises(ValueError):
        pkv.KVBlockManager(4, 16, [0, 1, 1, 2])
    with pytest.raises(ValueError):
        pkv.KVBlockManager(4, 0)


def test_block_copy_and_staging_dtype_checks_need_no_gpu():
    """The 16-bit block entry points refuse an 8-bit layout (its codes would
    move without their scales) and the 8-bit ones refuse a 16-bit layout or
    a missing scale array, before any launch; n == 0 is a no-op."""
    lib = pkv.load_library()
    fake = ctypes.c_void_p(0x1000)
    ids = (ctypes.c_int32 * 2)(0, 1)
    l16 = _layout(dtype=pkv.PKV_BF16, head_dim=128, head_stride=16 * 128, block_stride=2 * 4 * 16 * 128)
    l8 = _layout(dtype=pkv.PKV_FP8_E4M3, head_dim=128, head_stride=16 * 128, block_stride=2 * 4 * 16 * 128)
    assert lib.pkv_copy_blocks(ids, ids, 2, fake, fake, ctypes.byref(l8), None) == -5
    assert lib.pkv_gather_blocks(ids, 2, fake, fake, fake, ctypes.byref(l8), None) == -5
    assert lib.pkv_scatter_blocks(fake, ids, 2, fake, fake, ctypes.byref(l8), None) == -5
    assert lib.pkv_copy_blocks_fp8(ids, ids, 2, fake, fake, fake, fake, ctypes.byref(l16), None) == -5
    assert lib.pkv_gather_blocks_fp8(ids, 2, fake, fake, fake, fake, fake, fake, ctypes.byref(l16), None) == -5
    assert lib.pkv_scatter_blocks_fp8(fake, fake, ids, 2, fake, fake, fake, fake, ctypes.byref(l16), None) == -5
    assert lib.pkv_copy_blocks_fp8(ids, ids, 2, fake, fake, None, fake, ctypes.byref(l8), None) == -1
    assert lib.pkv_gather_blocks_fp8(ids, 2, fake, fake, fake, fake, fake, None, ctypes.byref(l8), None) == -1
    assert lib.pkv_scatter_blocks_fp8(fake, fake, ids, 2, fake, fake, fake, None, ctypes.byref(l8), None) == -1
    assert lib.pkv_copy_blocks_fp8(ids, ids, -1, fake, fake, fake, fake, ctypes.byref(l8), None) == -1
    assert lib.pkv_copy_blocks_fp8(ids, ids, 0, fake, fake, fake, fake, ctypes.byref(l8), None) == 0
    assert lib.pkv_gather_blocks_fp8(ids, 0, fake, fake, fake, fake, fake, fake, ctypes.byref(l8), None) == 0


def test_slot_mapping_check_matches_brute_force():
    """pkv_check_slot_mapping names the first entry whose in-range slot an
    earlier entry holds (a write race), ignores out-of-range slots (the
    writes skip them), and refuses bad arguments with first_repeat = -1."""
    import numpy as np
    lib = pkv.load_library()
    rng = np.random.default_rng(5)
    hits = 0
    for _ in range(300):
        n, N = int(rng.integers(0, 40)), int(rng.integers(1, 60))
        sl = np.ascontiguousarray(rng.integers(-3, N + 3, n), dtype=np.int64)
        want, seen = -1, set()
        for i, x in enumerate(sl.tolist()):
            if 0 <= x < N:
                if x in seen:
                    want = i
                    break
                seen.add(x)
        first = ctypes.c_int64(-7)
        st = lib.pkv_check_slot_mapping(sl.ctypes.data if n else None, n, N, ctypes.byref(first))
        assert (st, first.value) == ((0, -1) if want < 0 else (-1, want)), (sl, N)
        hits += want >= 0
    assert 50 < hits < 250
    first = ctypes.c_int64(-7)
    assert lib.pkv_check_slot_mapping(None, 3, 10, ctypes.byref(first)) == -1 and first.value == -1
    assert lib.pkv_check_slot_mapping(None, -1, 10, None) == -1
    assert lib.pkv_check_slot_mapping(None, 0, 10, None) == 0


def test_debug_slot_check_refuses_a_repeated_slot_before_any_launch(monkeypatch):
    """With the debug check on, the write entry points raise on a slot two
    rows would write, before anything is launched (CPU tensors here, so a
    launch could not even start)."""
    import numpy as np
    import torch
    pkv.check_slot_mapping(np.array([4, 1, -1, -1, 99]), 64)
    with pytest.raises(pkv.InvalidArgumentError, match="slot 1 written twice"):
        pkv.check_slot_mapping(np.array([4, 1, 7, 1]), 64)
    monkeypatch.setattr(pkv, "DEBUG_SLOTS", True)
    pool = torch.zeros(4, 2, 2, 16, 64)
    k = torch.zeros(3, 2, 64)
    with pytest.raises(pkv.InvalidArgumentError, match="entry 2"):
        pkv.decode_write(k, k, np.array([5, 9, 5]), np.array([6, 10, 6], dtype=np.int32), pool[:, 0], pool[:, 1])
    with pytest.raises(pkv.InvalidArgumentError, match="slot 17"):
        pkv.paged_kv_write(k, k, torch.tensor([17, 3, 17]), pool[:, 0], pool[:, 1])
