"""Python binding of libpkv: paged KV cache write, paged decode attention and
the host block manager, for MI355X (gfx950).

Argument marshalling only: every step runs in libpkv (HIP kernels and the C++
manager).  PyTorch supplies device memory and the current stream.  There is
no fallback: if the library is missing, importing the GPU entry points
raises.

Pool convention used by ``new_pool``: one tensor ``[N, 2, H_kv, bs, D]``
per layer, K in ``[:, 0]`` and V in ``[:, 1]`` (each block holds its K half
then its V half); the library also accepts separate ``[N, H_kv, bs, D]``
tensors, or any views with contiguous ``[bs, D]`` tiles.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libpkv.so")

PKV_F32, PKV_F16, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2, 3
SORT_ON_RELEASE = 1

STATUS = {0: "OK", -1: "INVALID", -2: "OOM", -3: "NOT_LIVE", -4: "ALREADY_PREFILLED",
          -5: "UNSUPPORTED", -6: "HIP", -7: "WORKSPACE", -8: "INVARIANT"}


class PkvError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        self.name = STATUS.get(status, str(status))
        msg = _lib_handle().pkv_status_string(status).decode() if _LIB is not None else self.name
        super().__init__(f"{what}: {self.name} ({msg})" if what else f"{self.name} ({msg})")


class InvalidArgumentError(PkvError, ValueError):
    pass


class OutOfBlocksError(PkvError):
    pass


class NotLiveError(PkvError, ValueError):
    pass


class AlreadyPrefilledError(PkvError, ValueError):
    pass


_ERRORS = {-1: InvalidArgumentError, -2: OutOfBlocksError, -3: NotLiveError,
           -4: AlreadyPrefilledError}


def _check(status: int, what: str) -> int:
    if status < 0:
        raise _ERRORS.get(status, PkvError)(status, what)
    return status


# With PKV_DEBUG_SLOTS=1 in the environment every write entry point first
# checks its slot mapping on the host (pkv_check_slot_mapping) and raises
# on a slot that two rows would write; device slot tensors are copied to
# the host for it (a synchronising copy: debug runs only).
DEBUG_SLOTS = os.environ.get("PKV_DEBUG_SLOTS", "") == "1"


def check_slot_mapping(slots, num_slots: int) -> None:
    """Raise InvalidArgumentError if an in-range slot appears twice in
    ``slots`` (host array, or a tensor copied to the host); slots outside
    [0, num_slots) are ignored, as the writes skip them."""
    if hasattr(slots, "detach"):
        slots = slots.detach().cpu().numpy()
    arr = np.ascontiguousarray(slots, dtype=np.int64).reshape(-1)
    first = ctypes.c_int64(-1)
    st = _lib_handle().pkv_check_slot_mapping(_ptr(arr, ctypes.c_int64), arr.size, int(num_slots),
                                               ctypes.byref(first))
    if st < 0 and first.value >= 0:
        raise InvalidArgumentError(st, f"slot {int(arr[first.value])} written twice "
                                       f"(entry {first.value} repeats an earlier one)")
    _check(st, "pkv_check_slot_mapping")


def _debug_slots(slots, lay) -> None:
    if DEBUG_SLOTS:
        check_slot_mapping(slots, int(lay.num_blocks) * int(lay.block_size))


class CacheLayout(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("block_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64)]


_LIB = None
_P = ctypes.c_void_p
_I32, _I64, _U32, _F32, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_float, ctypes.c_size_t
# typed host arrays travel as plain addresses (see _ptr)
_PI32 = _PI64 = _P

# name -> (restype, argtypes); the complete exported C ABI
SIGNATURES = {
    "pkv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pkv_version": (ctypes.c_char_p, []),
    "pkv_pool_span_bytes": (_SZ, [ctypes.POINTER(CacheLayout)]),
    "pkv_manager_create": (_P, [_I32, _I32, _PI32, _U32]),
    "pkv_manager_destroy": (None, [_P]),
    "pkv_can_allocate": (ctypes.c_int, [_P, _I32]),
    "pkv_num_free_blocks": (_I32, [_P]),
    "pkv_num_live_sequences": (_I32, [_P]),
    "pkv_allocate_for_prefill": (ctypes.c_int, [_P, _I64, _I32, _PI64]),
    "pkv_append_slot_for_decode": (ctypes.c_int, [_P, _I64, _PI64]),
    "pkv_append_slots_for_decode": (ctypes.c_int, [_P, _PI64, _I32, _PI64, _PI32, _PI32]),
    "pkv_free_sequence": (ctypes.c_int, [_P, _I64]),
    "pkv_share_prefix": (ctypes.c_int, [_P, _I64, _I64, _I32]),
    "pkv_append_tokens": (ctypes.c_int, [_P, _I64, _I32, _PI64]),
    "pkv_admit_batch": (ctypes.c_int, [_P, _PI64, _PI32, _I32, _I32, _PI64, _PI32]),
    "pkv_swap_out": (ctypes.c_int, [_P, _I64, _PI32, _I32, _PI32]),
    "pkv_swap_in": (ctypes.c_int, [_P, _I64, _PI32, _I32, _PI32]),
    "pkv_is_swapped": (ctypes.c_int, [_P, _I64]),
    "pkv_gather_blocks": (ctypes.c_int, [_PI32, _I32, _P, _P, _P, ctypes.POINTER(CacheLayout), _P]),
    "pkv_scatter_blocks": (ctypes.c_int, [_P, _PI32, _I32, _P, _P, ctypes.POINTER(CacheLayout), _P]),
    "paged_prefill_attention": (ctypes.c_int, [_P, _I32, _P, _P, _P, _I32, _I32, _P, _P,
                                               ctypes.POINTER(CacheLayout), _P, _I32, _I32, _I32, _F32, _P]),
    "paged_prefill_attention_fp8_workspace_size": (_SZ, [_I32, _I32, ctypes.POINTER(CacheLayout)]),
    "paged_prefill_attention_fp8": (ctypes.c_int, [_P, _I32, _P, _I32, _P, _P, _I32, _I32, _P, _P, _P, _P,
                                                   ctypes.POINTER(CacheLayout), _P, _I32, _I32, _I32, _F32, _P,
                                                   _SZ, _P]),
    "pkv_block_ref_count": (_I32, [_P, _I32]),
    "pkv_take_block_copies": (ctypes.c_int, [_P, _PI32, _PI32, _I32, _PI32]),
    "pkv_copy_blocks": (ctypes.c_int, [_PI32, _PI32, _I32, _P, _P, ctypes.POINTER(CacheLayout), _P]),
    "pkv_copy_blocks_fp8": (ctypes.c_int, [_PI32, _PI32, _I32, _P, _P, _P, _P, ctypes.POINTER(CacheLayout), _P]),
    "pkv_gather_blocks_fp8": (ctypes.c_int, [_PI32, _I32, _P, _P, _P, _P, _P, _P,
                                             ctypes.POINTER(CacheLayout), _P]),
    "pkv_scatter_blocks_fp8": (ctypes.c_int, [_P, _P, _PI32, _I32, _P, _P, _P, _P,
                                              ctypes.POINTER(CacheLayout), _P]),
    "paged_kv_write_fp8": (ctypes.c_int, [_P, _P, _I32, _P, _I32, _P, _P, _P, _P,
                                          ctypes.POINTER(CacheLayout), _P]),
    "pkv_decode_write_fp8": (ctypes.c_int, [_P, _P, _I32, _PI64, _PI32, _I32, _P, _P, _P, _P,
                                            ctypes.POINTER(CacheLayout), _P, _I32, _I32, _P, _P]),
    "pkv_decode_step_fp8": (ctypes.c_int, [_P, _I32, _P, _I32, _P, _P, _PI64, _PI32, _I32, _P, _P, _P, _P,
                                           ctypes.POINTER(CacheLayout), _P, _I32, _P, _I32, _I32, _F32, _I32,
                                           _P, _SZ, _P]),
    "paged_decode_attention_fp8": (ctypes.c_int, [_P, _I32, _P, _I32, _P, _P, _P, _P, _P, _I32, _P,
                                                  _I32, _I32, _I32, _F32, ctypes.POINTER(CacheLayout),
                                                  _I32, _P, _SZ, _P]),
    "pkv_context_len": (_I32, [_P, _I64]),
    "pkv_get_block_table": (ctypes.c_int, [_P, _I64, _PI32, _I32, _PI32]),
    "pkv_get_block_tables": (ctypes.c_int, [_P, _PI64, _I32, _I32, _I32, _PI32]),
    "pkv_get_context_lens": (ctypes.c_int, [_P, _PI64, _I32, _PI32]),
    "pkv_get_free_list": (ctypes.c_int, [_P, _PI32, _I32, _PI32]),
    "pkv_check_invariants": (ctypes.c_int, [_P]),
    "pkv_check_slot_mapping": (ctypes.c_int, [_PI64, ctypes.c_int64, ctypes.c_int64, _PI64]),
    "paged_kv_write": (ctypes.c_int, [_P, _P, _P, _I32, _P, _P, ctypes.POINTER(CacheLayout), _P]),
    "pkv_decode_write": (ctypes.c_int, [_P, _P, _PI64, _PI32, _I32, _P, _P, ctypes.POINTER(CacheLayout),
                                        _P, _I32, _I32, _P, _P]),
    "pkv_decode_step": (ctypes.c_int, [_P, _I32, _P, _P, _P, _PI64, _PI32, _I32, _P, _P,
                                       ctypes.POINTER(CacheLayout), _P, _I32, _P, _I32, _I32,
                                       ctypes.c_float, _P, _SZ, _P]),
    "pkv_decode_step_noalloc": (ctypes.c_int, [_P, _I32, _P, _P, _P, _PI64, _PI32, _I32, _P, _P,
                                               ctypes.POINTER(CacheLayout), _P, _I32, _P, _I32, _I32,
                                               ctypes.c_float, _P]),
    "pkv_decode_step_partial": (ctypes.c_int, [_P, _I32, _P, _P, _P, _PI64, _PI32, _I32, _P, _P,
                                               ctypes.POINTER(CacheLayout), _P, _I32, _P, _I32, _I32,
                                               ctypes.c_float, _P, _SZ, _P]),
    "pkv_decode_step_merge": (ctypes.c_int, [_P, _I32, _P, _P, _P, _PI64, _PI32, _I32, _P, _P,
                                             ctypes.POINTER(CacheLayout), _P, _I32, _P, _I32, _I32,
                                             ctypes.c_float, _P, _SZ, _P]),
    "paged_decode_attention_workspace_size": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "paged_decode_attention": (ctypes.c_int, [_P, _I32, _P, _P, _P, _P, _I32, _P, _I32, _I32, _I32,
                                              _F32, ctypes.POINTER(CacheLayout), _I32, _P, _SZ, _P]),
    "paged_decode_attention_partial": (ctypes.c_int, [_P, _I32, _P, _P, _P, _P, _I32, _P, _I32, _I32,
                                                      _I32, _F32, ctypes.POINTER(CacheLayout), _I32,
                                                      _P, _SZ, _P]),
    "paged_decode_attention_merge": (ctypes.c_int, [_P, _I32, _P, _P, _P, _P, _I32, _P, _I32, _I32,
                                                    _I32, _F32, ctypes.POINTER(CacheLayout), _I32,
                                                    _P, _SZ, _P]),
    "paged_decode_attention_path": (ctypes.c_int, [_I32, _I32, _I32, ctypes.POINTER(CacheLayout), _I32]),
    "pkv_update_block_tables": (ctypes.c_int, [_P, _I32, _I32, _P, _P, _P, _I32, _I32, _P]),
    "pkv_copy_table_rows": (ctypes.c_int, [_P, _I32, _I32, _P, _P, _I32, _I32, _P, _I32, _I32, _P]),
}


def _lib_handle():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libpkv is not built ({LIB_PATH} missing): run "
                               "`python -m paged_kv_cache_128_amd._build` first")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def load_library():
    """Load libpkv (raises when it is missing) and return the ctypes handle."""
    return _lib_handle()


def version() -> str:
    return _lib_handle().pkv_version().decode()


def _np_i64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int64)


def _ptr(a: np.ndarray, ty):
    """Address of a host array's first element for a C pointer argument of
    element type ``ty`` (the caller keeps ``a`` alive across the call).  The
    array interface is the cheapest route to it (about half the cost of
    ``ctypes.data_as`` per call, which the decode step pays several times)."""
    return a.__array_interface__["data"][0]


# --------------------------------------------------------------------------
# Host block manager
# --------------------------------------------------------------------------
class KVBlockManager:
    """Host block manager in libpkv (see ``pkv_manager_*`` in include/pkv.h)."""

    def __init__(self, num_blocks: int, block_size: int,
                 initial_free_order: Optional[Sequence[int]] = None,
                 sort_on_release: bool = False):
        lib = _lib_handle()
        order = None
        if initial_free_order is not None:
            order = np.ascontiguousarray(initial_free_order, dtype=np.int32)
            if order.shape != (num_blocks,):
                raise ValueError("initial_free_order must have num_blocks entries")
        h = lib.pkv_manager_create(int(num_blocks), int(block_size),
                                   None if order is None else _ptr(order, ctypes.c_int32),
                                   SORT_ON_RELEASE if sort_on_release else 0)
        if not h:
            raise ValueError("invalid block manager arguments")
        self._h = ctypes.c_void_p(h)
        self._lib = lib
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.pkv_manager_destroy(h)
            self._h = None

    # queries
    def can_allocate(self, num_tokens: int) -> bool:
        return bool(_check(self._lib.pkv_can_allocate(self._h, int(num_tokens)), "can_allocate"))

    def num_free_blocks(self) -> int:
        return int(self._lib.pkv_num_free_blocks(self._h))

    def num_live_sequences(self) -> int:
        return int(self._lib.pkv_num_live_sequences(self._h))

    def context_len(self, seq_id: int) -> int:
        return _check(self._lib.pkv_context_len(self._h, int(seq_id)), "context_len")

    def block_table(self, seq_id: int) -> list:
        cap = self.num_blocks
        out = np.empty(cap, dtype=np.int32)
        n = ctypes.c_int32(0)
        _check(self._lib.pkv_get_block_table(self._h, int(seq_id), _ptr(out, ctypes.c_int32), cap,
                                             ctypes.byref(n)), "block_table")
        return out[:n.value].tolist()

    def block_tables(self, seq_ids: Sequence[int], width: int, pad: int = -1,
                     out: Optional[np.ndarray] = None) -> np.ndarray:
        ids = _np_i64(seq_ids)
        if out is None:
            out = np.empty((len(ids), width), dtype=np.int32)
        _check(self._lib.pkv_get_block_tables(self._h, _ptr(ids, ctypes.c_int64), len(ids), int(width),
                                              int(pad), _ptr(out, ctypes.c_int32)), "block_tables")
        return out

    def context_lens(self, seq_ids: Sequence[int]) -> np.ndarray:
        ids = _np_i64(seq_ids)
        out = np.empty(len(ids), dtype=np.int32)
        _check(self._lib.pkv_get_context_lens(self._h, _ptr(ids, ctypes.c_int64), len(ids),
                                              _ptr(out, ctypes.c_int32)), "context_lens")
        return out

    def free_list(self) -> list:
        out = np.empty(self.num_blocks, dtype=np.int32)
        n = ctypes.c_int32(0)
        _check(self._lib.pkv_get_free_list(self._h, _ptr(out, ctypes.c_int32), self.num_blocks,
                                           ctypes.byref(n)), "free_list")
        return out[:n.value].tolist()

    def check_invariants(self) -> bool:
        return self._lib.pkv_check_invariants(self._h) == 0

    # operations
    def allocate_for_prefill(self, seq_id: int, num_tokens: int, want_slots: bool = True):
        slots = np.empty(max(int(num_tokens), 0), dtype=np.int64) if want_slots else None
        _check(self._lib.pkv_allocate_for_prefill(
            self._h, int(seq_id), int(num_tokens),
            None if slots is None else _ptr(slots, ctypes.c_int64)), "allocate_for_prefill")
        return slots

    def append_slot_for_decode(self, seq_id: int) -> int:
        s = ctypes.c_int64(0)
        _check(self._lib.pkv_append_slot_for_decode(self._h, int(seq_id), ctypes.byref(s)),
               "append_slot_for_decode")
        return s.value

    def append_slots_for_decode(self, seq_ids, slots_out: Optional[np.ndarray] = None,
                                lens_out: Optional[np.ndarray] = None,
                                new_block_out: Optional[np.ndarray] = None):
        """Batched all-or-nothing append.  Returns (slots int64, lens int32,
        new_block int32); the optional outputs (e.g. numpy views of pinned
        host tensors) are filled in place."""
        ids = seq_ids if (isinstance(seq_ids, np.ndarray) and seq_ids.dtype == np.int64
                          and seq_ids.flags.c_contiguous) else _np_i64(seq_ids)
        n = len(ids)
        slots = slots_out if slots_out is not None else np.empty(n, dtype=np.int64)
        lens = lens_out if lens_out is not None else np.empty(n, dtype=np.int32)
        newb = new_block_out if new_block_out is not None else np.empty(n, dtype=np.int32)
        _check(self._lib.pkv_append_slots_for_decode(
            self._h, _ptr(ids, ctypes.c_int64), n, _ptr(slots, ctypes.c_int64),
            _ptr(lens, ctypes.c_int32), _ptr(newb, ctypes.c_int32)), "append_slots_for_decode")
        return slots, lens, newb

    def _append_at(self, ids_addr: int, n: int, slots_addr: int, lens_addr: int, newb_addr: int) -> None:
        """append_slots_for_decode on host buffers given by address (the
        engine's persistent arrays, whose addresses it computes once)."""
        _check(self._lib.pkv_append_slots_for_decode(self._h, ids_addr, n, slots_addr, lens_addr, newb_addr),
               "append_slots_for_decode")

    def free_sequence(self, seq_id: int) -> None:
        _check(self._lib.pkv_free_sequence(self._h, int(seq_id)), "free_sequence")

    def append_tokens(self, seq_id: int, num_tokens: int) -> np.ndarray:
        """Slots of num_tokens new tokens of a live sequence, all or nothing
        (see pkv_append_tokens)."""
        slots = np.empty(max(int(num_tokens), 0), dtype=np.int64)
        _check(self._lib.pkv_append_tokens(self._h, int(seq_id), int(num_tokens),
                                           _ptr(slots, ctypes.c_int64)), "append_tokens")
        return slots

    def admit_batch(self, seq_ids, chunk_lens, extend_live: bool = False):
        """All-or-nothing admission of a batch of prefill chunks (see
        pkv_admit_batch): returns (slots int64 of every chunk concatenated,
        lens int32 after)."""
        ids = _np_i64(seq_ids)
        cl = np.ascontiguousarray(chunk_lens, dtype=np.int32)
        if cl.shape != ids.shape:
            raise ValueError("one chunk length per sequence")
        if np.any(cl < 0):
            raise InvalidArgumentError(-1, "admit_batch: chunk lengths must be >= 0")
        slots = np.empty(int(cl.sum()), dtype=np.int64)
        lens = np.empty(len(ids), dtype=np.int32)
        _check(self._lib.pkv_admit_batch(self._h, _ptr(ids, ctypes.c_int64), _ptr(cl, ctypes.c_int32), len(ids),
                                         1 if extend_live else 0, _ptr(slots, ctypes.c_int64),
                                         _ptr(lens, ctypes.c_int32)), "admit_batch")
        return slots, lens

    def swap_out(self, seq_id: int) -> np.ndarray:
        """Release a live sequence's blocks, keeping its length; returns the
        released ids in table order (see pkv_swap_out)."""
        ids = np.empty(self.num_blocks, dtype=np.int32)
        n = ctypes.c_int32(0)
        _check(self._lib.pkv_swap_out(self._h, int(seq_id), _ptr(ids, ctypes.c_int32), self.num_blocks,
                                      ctypes.byref(n)), "swap_out")
        return ids[:n.value].copy()

    def swap_in(self, seq_id: int) -> np.ndarray:
        """Fresh blocks for a swapped sequence; returns its new table."""
        ids = np.empty(self.num_blocks, dtype=np.int32)
        n = ctypes.c_int32(0)
        _check(self._lib.pkv_swap_in(self._h, int(seq_id), _ptr(ids, ctypes.c_int32), self.num_blocks,
                                     ctypes.byref(n)), "swap_in")
        return ids[:n.value].copy()

    def is_swapped(self, seq_id: int) -> bool:
        return bool(_check(self._lib.pkv_is_swapped(self._h, int(seq_id)), "is_swapped"))

    def share_prefix(self, donor_id: int, seq_id: int, num_tokens: int) -> None:
        """New sequence on the donor's first ceil(num_tokens / bs) blocks
        (see pkv_share_prefix)."""
        _check(self._lib.pkv_share_prefix(self._h, int(donor_id), int(seq_id), int(num_tokens)),
               "share_prefix")

    def ref_count(self, block: int) -> int:
        return _check(self._lib.pkv_block_ref_count(self._h, int(block)), "ref_count")

    def take_copies(self):
        """Drain the copy-on-write queue: (src int32, dst int32) numpy arrays."""
        cap = self.num_blocks
        src = np.empty(cap, dtype=np.int32)
        dst = np.empty(cap, dtype=np.int32)
        n = ctypes.c_int32(0)
        _check(self._lib.pkv_take_block_copies(self._h, _ptr(src, ctypes.c_int32),
                                               _ptr(dst, ctypes.c_int32), cap, ctypes.byref(n)),
               "take_copies")
        return src[:n.value].copy(), dst[:n.value].copy()


# --------------------------------------------------------------------------
# Device entry points (torch tensors in, torch tensors out)
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def dtype_code(dtype) -> int:
    torch = _torch()
    codes = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16,
             torch.float8_e4m3fn: PKV_FP8_E4M3}
    if dtype not in codes:
        raise ValueError(f"unsupported dtype {dtype}")
    return codes[dtype]


def _stream_handle(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def cache_layout(key_cache, value_cache=None) -> CacheLayout:
    """Layout of K/V cache tensors shaped [N, H_kv, bs, D] whose [bs, D]
    tiles are contiguous (any block and head strides)."""
    if key_cache.dim() != 4:
        raise ValueError("key_cache must be [num_blocks, H_kv, block_size, head_dim]")
    n, h, bs, d = key_cache.shape
    st = key_cache.stride()
    if st[3] != 1 or st[2] != d:
        raise ValueError("each [block_size, head_dim] tile must be contiguous")
    if value_cache is not None:
        if value_cache.shape != key_cache.shape or value_cache.stride() != st \
                or value_cache.dtype != key_cache.dtype:
            raise ValueError("value_cache must match key_cache in shape, strides and dtype")
    return CacheLayout(n, h, bs, d, dtype_code(key_cache.dtype), 0, st[0], st[1])


def new_fp8_pool(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
                 device="cuda", poison: bool = False):
    """8-bit KV pool: codes [N, 2, H_kv, bs, D] (torch.float8_e4m3fn) and scale
    bytes [N, 2, H_kv, bs] (uint8).  Returns (codes, key view, value view,
    scales, key-scale view, value-scale view).  ``poison`` fills codes with
    0x7F (NaN) and scales with 0xFF so reads of unwritten rows show."""
    torch = _torch()
    codes = torch.empty((num_blocks, 2, num_kv_heads, block_size, head_dim), dtype=torch.float8_e4m3fn,
                        device=device)
    scales = torch.empty((num_blocks, 2, num_kv_heads, block_size), dtype=torch.uint8, device=device)
    if poison:
        codes.view(torch.uint8).fill_(0x7F)
        scales.fill_(0xFF)
    return codes, codes[:, 0], codes[:, 1], scales, scales[:, 0], scales[:, 1]


def _check_scales(key_cache, key_scales, value_scales):
    torch = _torch()
    n, h, bs, d = key_cache.shape
    st = key_cache.stride()
    for t in (key_scales, value_scales):
        if t.dtype != torch.uint8 or tuple(t.shape) != (n, h, bs) or \
                tuple(t.stride()) != (st[0] // d, st[1] // d, 1):
            raise ValueError("scales must be uint8 [N, H_kv, bs] mirroring the code layout")


def paged_kv_write_fp8(key, value, slot_mapping, key_cache, value_cache, key_scales, value_scales,
                       stream=None) -> None:
    """paged_kv_write into 8-bit blocks: key/value [T, H_kv, D] (bf16, f16 or
    f32) quantised row by row (see paged_kv_write_fp8 in pkv.h)."""
    torch = _torch()
    lay = cache_layout(key_cache, value_cache)
    _check_scales(key_cache, key_scales, value_scales)
    T = key.shape[0]
    if key.shape != (T, lay.num_kv_heads, lay.head_dim) or value.shape != key.shape \
            or value.dtype != key.dtype or not (key.is_contiguous() and value.is_contiguous()):
        raise ValueError("key/value must be contiguous [num_tokens, H_kv, head_dim] of one dtype")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,) or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be contiguous int64 [num_tokens]")
    _debug_slots(slot_mapping, lay)
    st = _lib_handle().paged_kv_write_fp8(key.data_ptr(), value.data_ptr(), dtype_code(key.dtype),
                                          slot_mapping.data_ptr(), T, key_cache.data_ptr(),
                                          value_cache.data_ptr(), key_scales.data_ptr(),
                                          value_scales.data_ptr(), ctypes.byref(lay),
                                          _stream_handle(stream))
    _check(st, "paged_kv_write_fp8")


def decode_write_fp8(key, value, slots: np.ndarray, lens: np.ndarray, key_cache, value_cache,
                     key_scales, value_scales, block_tables=None, lens_out=None, stream=None) -> None:
    """pkv_decode_write into 8-bit blocks (host slots int64 and lens int32)."""
    torch = _torch()
    lay = cache_layout(key_cache, value_cache)
    _check_scales(key_cache, key_scales, value_scales)
    n = key.shape[0]
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    if key.shape != (n, lay.num_kv_heads, lay.head_dim) or value.shape != key.shape \
            or slots.shape != (n,) or lens.shape != (n,):
        raise ValueError("key/value [n, H_kv, D] with n slots and lens")
    tab_ptr, rows, stride = None, 0, 0
    if block_tables is not None:
        if block_tables.dtype != torch.int32 or block_tables.stride(1) != 1:
            raise ValueError("block_tables must be int32 with unit column stride")
        tab_ptr, rows, stride = block_tables.data_ptr(), block_tables.shape[0], block_tables.stride(0)
    _debug_slots(slots, lay)
    st = _lib_handle().pkv_decode_write_fp8(
        key.data_ptr(), value.data_ptr(), dtype_code(key.dtype), _ptr(slots, ctypes.c_int64),
        _ptr(lens, ctypes.c_int32), n, key_cache.data_ptr(), value_cache.data_ptr(),
        key_scales.data_ptr(), value_scales.data_ptr(), ctypes.byref(lay), tab_ptr, rows, stride,
        None if lens_out is None else lens_out.data_ptr(), _stream_handle(stream))
    _check(st, "pkv_decode_write_fp8")


def decode_step_fp8(q, key, value, slots: np.ndarray, lens: np.ndarray, key_cache, value_cache,
                    key_scales, value_scales, block_tables, lens_out, scale: float, max_context_len: int,
                    out=None, workspace=None, stream=None, phase: str = "both", events=None):
    """pkv_decode_step over 8-bit blocks: key/value [n, H_kv, D] and q
    [n, H_q, D] in one 16-bit type; slots int64 / lens int32 host arrays.
    ``phase`` and ``events`` as for decode_step."""
    torch = _torch()
    lay = cache_layout(key_cache, value_cache)
    _check_scales(key_cache, key_scales, value_scales)
    n, hq, d = q.shape
    if key.shape != (n, lay.num_kv_heads, lay.head_dim) or value.shape != key.shape \
            or key.dtype != q.dtype or value.dtype != q.dtype:
        raise ValueError("key/value must be [n, H_kv, head_dim] in q's dtype")
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    if out is None:
        out = torch.empty((n, hq, d), dtype=torch.float32, device=q.device)
    need = workspace_size(n, hq, lay.num_kv_heads, d, max_context_len, 0)
    if need > 0 and workspace is None:
        if phase != "both":
            raise ValueError("a split-phase call needs an explicit workspace shared by both phases")
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if phase != "merge":
        _debug_slots(slots, lay)
    head = (out.data_ptr(), dtype_code(out.dtype), q.data_ptr(), dtype_code(q.dtype), key.data_ptr(),
            value.data_ptr(), _ptr(slots, ctypes.c_int64), _ptr(lens, ctypes.c_int32), n, key_cache.data_ptr(),
            value_cache.data_ptr(), key_scales.data_ptr(), value_scales.data_ptr(), ctypes.byref(lay),
            block_tables.data_ptr(), block_tables.stride(0), lens_out.data_ptr(), hq, int(max_context_len),
            float(scale))
    tail = (None if workspace is None else workspace.data_ptr(),
            0 if workspace is None else workspace.numel() * workspace.element_size(), _stream_handle(stream))
    fn = _lib_handle().pkv_decode_step_fp8
    if events is not None and len(events) == 2:
        if phase != "both":
            raise ValueError("events time both phases of one call")
        _record(events[0], stream)
        _check(fn(*head, 3, *tail), "pkv_decode_step_fp8")
        _record(events[1], stream)
        return out
    if events is not None:
        if phase != "both":
            raise ValueError("events time both phases of one call")
        _record(events[0], stream)
        _check(fn(*head, 1, *tail), "pkv_decode_step_fp8")
        _record(events[1], stream)
        _check(fn(*head, 2, *tail), "pkv_decode_step_fp8")
        _record(events[2], stream)
        return out
    _check(fn(*head, {"partial": 1, "merge": 2, "both": 3}[phase], *tail), "pkv_decode_step_fp8")
    return out


def paged_decode_attention_fp8(q, key_cache, value_cache, key_scales, value_scales, block_tables,
                               context_lens, scale: float, out=None, out_dtype=None,
                               max_context_len: Optional[int] = None, workspace=None, stream=None,
                               phase: str = "both"):
    """Decode attention over 8-bit blocks (see paged_decode_attention_fp8 in
    pkv.h); q [B, H_q, 128] bf16 or f16."""
    torch = _torch()
    lay = cache_layout(key_cache, value_cache)
    _check_scales(key_cache, key_scales, value_scales)
    B, hq, d = q.shape
    if d != lay.head_dim or not q.is_contiguous():
        raise ValueError("q must be contiguous [B, H_q, head_dim]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B \
            or block_tables.stride(1) != 1:
        raise ValueError("block_tables must be int32 [B, W] with unit column stride")
    if context_lens.dtype != torch.int32 or context_lens.shape != (B,) or not context_lens.is_contiguous():
        raise ValueError("context_lens must be contiguous int32 [B]")
    if max_context_len is None:
        max_context_len = block_tables.shape[1] * lay.block_size
    if out is None:
        out = torch.empty((B, hq, d), dtype=torch.float32 if out_dtype is None else out_dtype,
                          device=q.device)
    need = workspace_size(B, hq, lay.num_kv_heads, d, max_context_len, 0)
    if need > 0 and workspace is None:
        if phase != "both":
            raise ValueError("a split-phase call needs an explicit workspace shared by both phases")
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    phases = {"partial": 1, "merge": 2, "both": 3}[phase]
    st = _lib_handle().paged_decode_attention_fp8(
        out.data_ptr(), dtype_code(out.dtype), q.data_ptr(), dtype_code(q.dtype), key_cache.data_ptr(),
        value_cache.data_ptr(), key_scales.data_ptr(), value_scales.data_ptr(), block_tables.data_ptr(),
        block_tables.stride(0), context_lens.data_ptr(), B, hq, int(max_context_len), float(scale),
        ctypes.byref(lay), phases, None if workspace is None else workspace.data_ptr(),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream_handle(stream))
    _check(st, "paged_decode_attention_fp8")
    return out


def paged_prefill_attention(q, q_start, key_cache, value_cache, block_tables, context_lens,
                            scale: float, max_q_len: int, max_context_len: Optional[int] = None,
                            out=None, out_dtype=None, stream=None):
    """Chunked-prefill causal attention (see paged_prefill_attention in
    pkv.h): q [T, H_q, D]; q_start int32 [B + 1] and context_lens int32 [B]
    device tensors; max_q_len (host) bounds the rows of one sequence."""
    torch = _torch()
    lay = cache_layout(key_cache, value_cache)
    T, hq, d = q.shape
    B = context_lens.shape[0]
    if d != lay.head_dim or q.dtype != key_cache.dtype or not q.is_contiguous():
        raise ValueError("q must be contiguous [T, H_q, head_dim] in the cache dtype")
    if q_start.dtype != torch.int32 or q_start.shape != (B + 1,) or not q_start.is_contiguous():
        raise ValueError("q_start must be contiguous int32 [B + 1]")
    if context_lens.dtype != torch.int32 or not context_lens.is_contiguous():
        raise ValueError("context_lens must be contiguous int32 [B]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] < B \
            or block_tables.stride(1) != 1:
        raise ValueError("block_tables must be int32 [>= B, W] with unit column stride")
    if max_context_len is None:
        max_context_len = block_tables.shape[1] * lay.block_size
    if out is None:
        out = torch.empty((T, hq, d), dtype=torch.float32 if out_dtype is None else out_dtype,
                          device=q.device)
    st = _lib_handle().paged_prefill_attention(
        out.data_ptr(), dtype_code(out.dtype), q.data_ptr(), q_start.data_ptr(), context_lens.data_ptr(),
        B, int(max_q_len), key_cache.data_ptr(), value_cache.data_ptr(), ctypes.byref(lay),
        block_tables.data_ptr(), block_tables.stride(0), hq, int(max_context_len), float(scale),
        _stream_handle(stream))
    _check(st, "paged_prefill_attention")
    return out


def prefill_fp8_workspace_size(num_seqs: int, max_context_len: int, key_cache, value_cache) -> int:
    """Bytes of the caller-owned staging paged_prefill_attention_fp8 needs."""
    lay = cache_layout(key_cache, value_cache)
    return int(_lib_handle().paged_prefill_attention_fp8_workspace_size(int(num_seqs), int(max_context_len),
                                                                        ctypes.byref(lay)))


def paged_prefill_attention_fp8(q, q_start, key_cache, value_cache, key_scales, value_scales, block_tables,
                                context_lens, scale: float, max_q_len: int, max_context_len: Optional[int] = None,
                                out=None, out_dtype=None, workspace=None, stream=None):
    """Chunked-prefill causal attention over 8-bit blocks (see
    paged_prefill_attention_fp8 in pkv.h): bf16 or fp16 q [T, H_q, D]; the other
    tensors as for paged_prefill_attention; ``workspace`` (uint8 device
    tensor, allocated here when None) holds the 16-bit staging."""
    torch = _torch()
    lay = cache_layout(key_cache, value_cache)
    _check_scales(key_cache, key_scales, value_scales)
    T, hq, d = q.shape
    B = context_lens.shape[0]
    if d != lay.head_dim or q.dtype not in (torch.bfloat16, torch.float16) or not q.is_contiguous():
        raise ValueError("q must be contiguous bf16 or fp16 [T, H_q, head_dim]")
    if q_start.dtype != torch.int32 or q_start.shape != (B + 1,) or not q_start.is_contiguous():
        raise ValueError("q_start must be contiguous int32 [B + 1]")
    if context_lens.dtype != torch.int32 or not context_lens.is_contiguous():
        raise ValueError("context_lens must be contiguous int32 [B]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] < B \
            or block_tables.stride(1) != 1:
        raise ValueError("block_tables must be int32 [>= B, W] with unit column stride")
    if max_context_len is None:
        max_context_len = block_tables.shape[1] * lay.block_size
    if out is None:
        out = torch.empty((T, hq, d), dtype=torch.float32 if out_dtype is None else out_dtype,
                          device=q.device)
    need = prefill_fp8_workspace_size(B, max_context_len, key_cache, value_cache)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = _lib_handle().paged_prefill_attention_fp8(
        out.data_ptr(), dtype_code(out.dtype), q.data_ptr(), dtype_code(q.dtype), q_start.data_ptr(),
        context_lens.data_ptr(), B, int(max_q_len), key_cache.data_ptr(), value_cache.data_ptr(),
        key_scales.data_ptr(), value_scales.data_ptr(), ctypes.byref(lay), block_tables.data_ptr(),
        block_tables.stride(0), hq, int(max_context_len), float(scale), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_handle(stream))
    _check(st, "paged_prefill_attention_fp8")
    return out


def new_pool(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int, dtype,
             device="cuda", fill_bits: Optional[int] = None):
    """Allocate one interleaved pool [N, 2, H_kv, bs, D] and return
    (pool, key_cache view, value_cache view)."""
    torch = _torch()
    pool = torch.empty((num_blocks, 2, num_kv_heads, block_size, head_dim), dtype=dtype, device=device)
    if fill_bits is not None:
        itype = torch.int16 if pool.element_size() == 2 else torch.int32
        bits = fill_bits - (1 << 16) if itype is torch.int16 and fill_bits >= 1 << 15 else fill_bits
        if itype is torch.int32 and bits >= 1 << 31:
            bits -= 1 << 32
        pool.view(itype).fill_(bits)
    return pool, pool[:, 0], pool[:, 1]


def paged_kv_write(key, value, slot_mapping, key_cache, value_cache, stream=None) -> None:
    """Scatter key/value [T, H_kv, D] into the pool at slot_mapping [T]
    (int64 device tensor)."""
    torch = _torch()
    lay = cache_layout(key_cache, value_cache)
    T = key.shape[0]
    if key.shape != (T, lay.num_kv_heads, lay.head_dim) or value.shape != key.shape:
        raise ValueError("key/value must be [num_tokens, H_kv, head_dim]")
    if not (key.is_contiguous() and value.is_contiguous() and slot_mapping.is_contiguous()):
        raise ValueError("key, value and slot_mapping must be contiguous")
    if key.dtype != key_cache.dtype or value.dtype != key_cache.dtype:
        raise ValueError("key/value dtype must equal the cache dtype")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be int64 [num_tokens]")
    _debug_slots(slot_mapping, lay)
    st = _lib_handle().paged_kv_write(key.data_ptr(), value.data_ptr(), slot_mapping.data_ptr(), T,
                                      key_cache.data_ptr(), value_cache.data_ptr(),
                                      ctypes.byref(lay), _stream_handle(stream))
    _check(st, "paged_kv_write")


def gather_blocks(ids, key_cache, value_cache, staging=None, stream=None):
    """Blocks ids (host int32) of both pools into a staging tensor
    [n, 2, H_kv, bs, D] (see pkv_gather_blocks); returns it."""
    torch = _torch()
    lay = cache_layout(key_cache, value_cache)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    shape = (len(ids), 2, lay.num_kv_heads, lay.block_size, lay.head_dim)
    if staging is None:
        staging = torch.empty(shape, dtype=key_cache.dtype, device=key_cache.device)
    if tuple(staging.shape) != shape or not staging.is_contiguous() or staging.dtype != key_cache.dtype:
        raise ValueError("staging must be contiguous [n, 2, H_kv, bs, D] in the cache dtype")
    st = _lib_handle().pkv_gather_blocks(_ptr(ids, ctypes.c_int32), len(ids), key_cache.data_ptr(),
                                         value_cache.data_ptr(), staging.data_ptr(), ctypes.byref(lay),
                                         _stream_handle(stream))
    _check(st, "gather_blocks")
    return staging


def scatter_blocks(staging, ids, key_cache, value_cache, stream=None) -> None:
    """Staging entry j back into block ids[j] of both pools (see pkv_scatter_blocks)."""
    lay = cache_layout(key_cache, value_cache)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    shape = (len(ids), 2, lay.num_kv_heads, lay.block_size, lay.head_dim)
    if tuple(staging.shape) != shape or not staging.is_contiguous() or staging.dtype != key_cache.dtype \
            or staging.device != key_cache.device:
        raise ValueError("staging must be a contiguous device tensor [n, 2, H_kv, bs, D] in the cache dtype")
    st = _lib_handle().pkv_scatter_blocks(staging.data_ptr(), _ptr(ids, ctypes.c_int32), len(ids),
                                          key_cache.data_ptr(), value_cache.data_ptr(), ctypes.byref(lay),
                                          _stream_handle(stream))
    _check(st, "scatter_blocks")


def copy_blocks(src, dst, key_cache, value_cache, stream=None) -> None:
    """Copy whole blocks src[i] -> dst[i] (host int32 arrays) in both pools
    (see pkv_copy_blocks)."""
    lay = cache_layout(key_cache, value_cache)
    src = np.ascontiguousarray(src, dtype=np.int32)
    dst = np.ascontiguousarray(dst, dtype=np.int32)
    if src.shape != dst.shape or src.ndim != 1:
        raise ValueError("src and dst must be 1-D arrays of one length")
    st = _lib_handle().pkv_copy_blocks(_ptr(src, ctypes.c_int32), _ptr(dst, ctypes.c_int32),
                                       len(src), key_cache.data_ptr(), value_cache.data_ptr(),
                                       ctypes.byref(lay), _stream_handle(stream))
    _check(st, "copy_blocks")


def copy_blocks_fp8(src, dst, key_cache, value_cache, key_scales, value_scales, stream=None) -> None:
    """copy_blocks for an 8-bit pool: codes and scale bytes (see
    pkv_copy_blocks_fp8)."""
    lay = cache_layout(key_cache, value_cache)
    _check_scales(key_cache, key_scales, value_scales)
    src = np.ascontiguousarray(src, dtype=np.int32)
    dst = np.ascontiguousarray(dst, dtype=np.int32)
    if src.shape != dst.shape or src.ndim != 1:
        raise ValueError("src and dst must be 1-D arrays of one length")
    st = _lib_handle().pkv_copy_blocks_fp8(_ptr(src, ctypes.c_int32), _ptr(dst, ctypes.c_int32), len(src),
                                           key_cache.data_ptr(), value_cache.data_ptr(), key_scales.data_ptr(),
                                           value_scales.data_ptr(), ctypes.byref(lay), _stream_handle(stream))
    _check(st, "copy_blocks_fp8")


def _fp8_staging_shapes(lay, n):
    return ((n, 2, lay.num_kv_heads, lay.block_size, lay.head_dim), (n, 2, lay.num_kv_heads, lay.block_size))


def gather_blocks_fp8(ids, key_cache, value_cache, key_scales, value_scales, stream=None):
    """gather_blocks for an 8-bit pool: returns (codes [n, 2, H_kv, bs, D],
    scale bytes [n, 2, H_kv, bs]) (see pkv_gather_blocks_fp8)."""
    torch = _torch()
    lay = cache_layout(key_cache, value_cache)
    _check_scales(key_cache, key_scales, value_scales)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    cshape, sshape = _fp8_staging_shapes(lay, len(ids))
    codes = torch.empty(cshape, dtype=key_cache.dtype, device=key_cache.device)
    scales = torch.empty(sshape, dtype=torch.uint8, device=key_cache.device)
    st = _lib_handle().pkv_gather_blocks_fp8(_ptr(ids, ctypes.c_int32), len(ids), key_cache.data_ptr(),
                                             value_cache.data_ptr(), key_scales.data_ptr(), value_scales.data_ptr(),
                                             codes.data_ptr(), scales.data_ptr(), ctypes.byref(lay),
                                             _stream_handle(stream))
    _check(st, "gather_blocks_fp8")
    return codes, scales


def scatter_blocks_fp8(codes, scales, ids, key_cache, value_cache, key_scales, value_scales, stream=None) -> None:
    """scatter_blocks for an 8-bit pool: staged codes and scale bytes (as
    gather_blocks_fp8 returns them) back into blocks ids (see
    pkv_scatter_blocks_fp8)."""
    torch = _torch()
    lay = cache_layout(key_cache, value_cache)
    _check_scales(key_cache, key_scales, value_scales)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    cshape, sshape = _fp8_staging_shapes(lay, len(ids))
    if tuple(codes.shape) != cshape or codes.dtype != key_cache.dtype or not codes.is_contiguous() \
            or codes.device != key_cache.device:
        raise ValueError("codes must be a contiguous device tensor [n, 2, H_kv, bs, D] in the cache dtype")
    if tuple(scales.shape) != sshape or scales.dtype != torch.uint8 or not scales.is_contiguous() \
            or scales.device != key_cache.device:
        raise ValueError("scales must be a contiguous device uint8 tensor [n, 2, H_kv, bs]")
    st = _lib_handle().pkv_scatter_blocks_fp8(codes.data_ptr(), scales.data_ptr(), _ptr(ids, ctypes.c_int32),
                                              len(ids), key_cache.data_ptr(), value_cache.data_ptr(),
                                              key_scales.data_ptr(), value_scales.data_ptr(), ctypes.byref(lay),
                                              _stream_handle(stream))
    _check(st, "scatter_blocks_fp8")


def decode_write(key, value, slots: np.ndarray, lens: np.ndarray, key_cache, value_cache,
                 block_tables=None, lens_out=None, stream=None) -> None:
    """One decode step's write with host metadata (see pkv_decode_write):
    key/value [n, H_kv, D] device; slots int64 [n] and lens int32 [n] host
    (numpy); optional device block table [rows, W] and lens_out int32 [n]."""
    lay = cache_layout(key_cache, value_cache)
    n = key.shape[0]
    if key.shape != (n, lay.num_kv_heads, lay.head_dim) or value.shape != key.shape:
        raise ValueError("key/value must be [num_rows, H_kv, head_dim]")
    if not (key.is_contiguous() and value.is_contiguous()):
        raise ValueError("key and value must be contiguous")
    if key.dtype != key_cache.dtype or value.dtype != key_cache.dtype:
        raise ValueError("key/value dtype must equal the cache dtype")
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    if slots.shape != (n,) or lens.shape != (n,):
        raise ValueError("slots and lens must have one entry per row")
    torch = _torch()
    if block_tables is not None and (block_tables.dtype != torch.int32 or block_tables.dim() != 2
                                     or block_tables.stride(1) != 1):
        raise ValueError("block_tables must be int32 [rows, W] with unit column stride")
    if lens_out is not None and (lens_out.dtype != torch.int32 or lens_out.numel() < n
                                 or not lens_out.is_contiguous()):
        raise ValueError("lens_out must be a contiguous int32 tensor of at least n entries")
    _debug_slots(slots, lay)
    st = _lib_handle().pkv_decode_write(
        key.data_ptr(), value.data_ptr(), _ptr(slots, ctypes.c_int64), _ptr(lens, ctypes.c_int32), n,
        key_cache.data_ptr(), value_cache.data_ptr(), ctypes.byref(lay),
        None if block_tables is None else block_tables.data_ptr(),
        0 if block_tables is None else block_tables.shape[0],
        0 if block_tables is None else block_tables.stride(0),
        None if lens_out is None else lens_out.data_ptr(), _stream_handle(stream))
    _check(st, "pkv_decode_write")


def decode_step(q, key, value, slots: np.ndarray, lens: np.ndarray, key_cache, value_cache,
                block_tables, lens_out, scale: float, max_context_len: int, out=None,
                out_dtype=None, workspace=None, stream=None, phase: str = "both", events=None):
    """One decode step after the host-side append (see pkv_decode_step): the
    write of key/value [n, H_kv, D] at `slots` (host int64) and the attention
    of q [n, H_q, D] over the updated cache, with lens (host int32, lengths
    after the append) published to lens_out (device int32 [n]) and opened
    blocks to block_tables.  ``phase`` "partial" runs only the first launch
    and "merge" (same arguments and workspace) only the second.  ``events``
    (with phase "both") are recorded on the stream: three torch.cuda.Event
    before the first launch, between the two and after the second, or two
    around the whole call (no event between the launches); the arguments
    are checked and marshalled once for both launches."""
    torch = _torch()
    lay = cache_layout(key_cache, value_cache)
    n, hq, d = q.shape
    if key.shape != (n, lay.num_kv_heads, lay.head_dim) or value.shape != key.shape:
        raise ValueError("key/value must be [num_rows, H_kv, head_dim]")
    if not (key.is_contiguous() and value.is_contiguous() and q.is_contiguous()):
        raise ValueError("q, key and value must be contiguous")
    if key.dtype != key_cache.dtype or value.dtype != key_cache.dtype or q.dtype != key_cache.dtype:
        raise ValueError("q/key/value dtype must equal the cache dtype")
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    if slots.shape != (n,) or lens.shape != (n,):
        raise ValueError("slots and lens must have one entry per row")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.stride(1) != 1 \
            or block_tables.shape[0] < n:
        raise ValueError("block_tables must be int32 [>= n, W] with unit column stride")
    if lens_out.dtype != torch.int32 or lens_out.numel() < n or not lens_out.is_contiguous():
        raise ValueError("lens_out must be a contiguous int32 tensor of at least n entries")
    if out is None:
        od = torch.float32 if out_dtype is None else out_dtype
        out = torch.empty((n, hq, d), dtype=od, device=q.device)
    need = workspace_size(n, hq, lay.num_kv_heads, d, max_context_len, 0)
    if need > 0 and workspace is None:
        if phase != "both":
            raise ValueError("a split-phase call needs an explicit workspace shared by both phases")
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if phase != "merge":
        _debug_slots(slots, lay)
    args = (out.data_ptr(), dtype_code(out.dtype), q.data_ptr(), key.data_ptr(), value.data_ptr(),
            _ptr(slots, ctypes.c_int64), _ptr(lens, ctypes.c_int32), n, key_cache.data_ptr(),
            value_cache.data_ptr(), ctypes.byref(lay), block_tables.data_ptr(), block_tables.stride(0),
            lens_out.data_ptr(), hq, int(max_context_len), float(scale),
            None if workspace is None else workspace.data_ptr(),
            0 if workspace is None else workspace.numel() * workspace.element_size(),
            _stream_handle(stream))
    lib = _lib_handle()
    if events is not None and len(events) == 2:
        if phase != "both":
            raise ValueError("events time both phases of one call")
        _record(events[0], stream)
        _check(lib.pkv_decode_step(*args), "pkv_decode_step")
        _record(events[1], stream)
        return out
    if events is not None:
        if phase != "both":
            raise ValueError("events time both phases of one call")
        _record(events[0], stream)
        _check(lib.pkv_decode_step_partial(*args), "pkv_decode_step_partial")
        _record(events[1], stream)
        _check(lib.pkv_decode_step_merge(*args), "pkv_decode_step_merge")
        _record(events[2], stream)
        return out
    fn = {"both": "pkv_decode_step", "partial": "pkv_decode_step_partial",
          "merge": "pkv_decode_step_merge"}[phase]
    _check(getattr(lib, fn)(*args), fn)
    return out


NOALLOC_SCRATCH_BYTES = 36 << 20     # PKV_NOALLOC_SCRATCH_BYTES


def decode_step_noalloc(q, key, value, slots: np.ndarray, lens: np.ndarray, key_cache, value_cache,
                        block_tables, lens_out, scale: float, max_context_len: int, out,
                        stream=None):
    """pkv_decode_step_noalloc: decode_step with the split-K partials in the
    library's own per-GPU device array instead of a workspace, so the C call
    allocates nothing (``out`` is the caller's).  Calls on one GPU must not
    overlap (they share that array)."""
    torch = _torch()
    lay = cache_layout(key_cache, value_cache)
    n, hq, d = q.shape
    if key.shape != (n, lay.num_kv_heads, lay.head_dim) or value.shape != key.shape:
        raise ValueError("key/value must be [num_rows, H_kv, head_dim]")
    if not (key.is_contiguous() and value.is_contiguous() and q.is_contiguous()):
        raise ValueError("q, key and value must be contiguous")
    if key.dtype != key_cache.dtype or value.dtype != key_cache.dtype or q.dtype != key_cache.dtype:
        raise ValueError("q/key/value dtype must equal the cache dtype")
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    if slots.shape != (n,) or lens.shape != (n,):
        raise ValueError("slots and lens must have one entry per row")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.stride(1) != 1 \
            or block_tables.shape[0] < n:
        raise ValueError("block_tables must be int32 [>= n, W] with unit column stride")
    if lens_out.dtype != torch.int32 or lens_out.numel() < n or not lens_out.is_contiguous():
        raise ValueError("lens_out must be a contiguous int32 tensor of at least n entries")
    if out.shape != (n, hq, d) or not out.is_contiguous():
        raise ValueError("out must be contiguous [n, H_q, head_dim]")
    _debug_slots(slots, lay)
    st = _lib_handle().pkv_decode_step_noalloc(
        out.data_ptr(), dtype_code(out.dtype), q.data_ptr(), key.data_ptr(), value.data_ptr(),
        _ptr(slots, ctypes.c_int64), _ptr(lens, ctypes.c_int32), n, key_cache.data_ptr(),
        value_cache.data_ptr(), ctypes.byref(lay), block_tables.data_ptr(), block_tables.stride(0),
        lens_out.data_ptr(), hq, int(max_context_len), float(scale), _stream_handle(stream))
    _check(st, "pkv_decode_step_noalloc")
    return out


def _record(event, stream):
    if stream is None:
        event.record()
    else:
        event.record(stream)


def workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                   max_context_len: int, partition_tokens: int = 0) -> int:
    return int(_lib_handle().paged_decode_attention_workspace_size(
        num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, partition_tokens))


def paged_decode_attention(q, key_cache, value_cache, block_tables, context_lens, scale: float,
                           out=None, out_dtype=None, partition_tokens: int = 0,
                           max_context_len: Optional[int] = None, workspace=None, stream=None,
                           phase: str = "both"):
    """Decode attention through block tables.  q [B, H_q, D]; block_tables
    int32 [B, W]; context_lens int32 [B].  Returns out [B, H_q, D] (float32
    unless ``out_dtype`` / ``out`` says otherwise).  ``phase`` = "partial" or
    "merge" runs one of the two launches (same arguments, same workspace)."""
    torch = _torch()
    lay = cache_layout(key_cache, value_cache)
    B, hq, d = q.shape
    if d != lay.head_dim or q.dtype != key_cache.dtype or not q.is_contiguous():
        raise ValueError("q must be contiguous [B, H_q, head_dim] in the cache dtype")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B \
            or block_tables.stride(1) != 1:
        raise ValueError("block_tables must be int32 [B, W] with unit column stride")
    if context_lens.dtype != torch.int32 or context_lens.shape != (B,) or not context_lens.is_contiguous():
        raise ValueError("context_lens must be contiguous int32 [B]")
    W = block_tables.shape[1]
    if max_context_len is None:
        max_context_len = W * lay.block_size
    if out is None:
        od = torch.float32 if out_dtype is None else out_dtype
        out = torch.empty((B, hq, d), dtype=od, device=q.device)
    if out.shape != (B, hq, d) or not out.is_contiguous():
        raise ValueError("out must be contiguous [B, H_q, head_dim]")
    need = workspace_size(B, hq, lay.num_kv_heads, d, max_context_len, partition_tokens)
    if need > 0 and workspace is None:
        if phase != "both":
            raise ValueError("a split-phase call needs an explicit workspace shared by both phases")
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    fn = {"both": "paged_decode_attention", "partial": "paged_decode_attention_partial",
          "merge": "paged_decode_attention_merge"}[phase]
    st = getattr(_lib_handle(), fn)(
        out.data_ptr(), dtype_code(out.dtype), q.data_ptr(), key_cache.data_ptr(),
        value_cache.data_ptr(), block_tables.data_ptr(), block_tables.stride(0),
        context_lens.data_ptr(), B, hq, int(max_context_len), float(scale), ctypes.byref(lay),
        int(partition_tokens), ws_ptr, ws_bytes, _stream_handle(stream))
    _check(st, "paged_decode_attention")
    return out


def attention_path(num_seqs: int, num_q_heads: int, max_context_len: int, key_cache,
                   partition_tokens: int = 0) -> str:
    """"stream" or "partition": the attention kernel the library picks."""
    lay = cache_layout(key_cache)
    st = _check(_lib_handle().paged_decode_attention_path(num_seqs, num_q_heads, max_context_len,
                                                          ctypes.byref(lay), partition_tokens),
                "paged_decode_attention_path")
    return {1: "stream", 2: "partition"}[st]


def update_block_tables(block_tables, lens, new_block, block_size: int, rows=None, stream=None) -> None:
    """Apply one batched append's new blocks to a device block table."""
    n = lens.shape[0]
    if block_tables.dtype != _torch().int32 or block_tables.dim() != 2 or block_tables.stride(1) != 1:
        raise ValueError("block_tables must be int32 [rows, W] with unit column stride")
    st = _lib_handle().pkv_update_block_tables(
        block_tables.data_ptr(), block_tables.shape[0], block_tables.stride(0),
        None if rows is None else rows.data_ptr(),
        lens.data_ptr(), new_block.data_ptr(), n, int(block_size), _stream_handle(stream))
    _check(st, "update_block_tables")


def copy_table_rows(dst, src, n: int, dst_rows=None, src_rows=None, width: Optional[int] = None,
                    stream=None) -> None:
    """Rows of int32 device tables (see pkv_copy_table_rows): row src_rows[i]
    (or i) of ``src`` to row dst_rows[i] (or i) of ``dst`` for i < n; the row
    lists are device int32 tensors or None."""
    torch = _torch()
    for t in (dst, src):
        if t.dtype != torch.int32 or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError("tables must be int32 [rows, W] with unit column stride")
    for r in (dst_rows, src_rows):
        if r is not None and (r.dtype != torch.int32 or r.numel() < n or not r.is_contiguous()):
            raise ValueError("row lists must be contiguous int32 tensors of at least n entries")
    w = min(dst.shape[1], src.shape[1]) if width is None else int(width)
    st = _lib_handle().pkv_copy_table_rows(
        dst.data_ptr(), dst.stride(0), dst.shape[0], None if dst_rows is None else dst_rows.data_ptr(),
        src.data_ptr(), src.stride(0), src.shape[0], None if src_rows is None else src_rows.data_ptr(),
        int(n), w, _stream_handle(stream))
    _check(st, "copy_table_rows")


__all__ = [
    "KVBlockManager", "CacheLayout", "PkvError", "InvalidArgumentError", "OutOfBlocksError",
    "NotLiveError", "AlreadyPrefilledError", "paged_kv_write", "paged_decode_attention",
    "workspace_size", "update_block_tables", "copy_table_rows", "attention_path", "decode_write", "decode_step", "new_pool",
    "decode_step_noalloc", "NOALLOC_SCRATCH_BYTES",
    "copy_blocks", "gather_blocks", "scatter_blocks", "copy_blocks_fp8", "gather_blocks_fp8",
    "scatter_blocks_fp8", "new_fp8_pool", "paged_kv_write_fp8", "decode_write_fp8",
    "paged_decode_attention_fp8", "PKV_FP8_E4M3", "paged_prefill_attention", "decode_step_fp8",
    "paged_prefill_attention_fp8", "prefill_fp8_workspace_size",
    "cache_layout", "load_library",
    "version", "dtype_code", "PKV_F32", "PKV_F16", "PKV_BF16", "SIGNATURES",
]
