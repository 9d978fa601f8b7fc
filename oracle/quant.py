"""FP8 KV blocks (oracle, test infrastructure only).

[impl-detail] "实践建议" notes that the KV cache inside a block can be
quantised on its own.  Reading taken here (the pages fix no format): every
token row of every KV head is quantised on its own when it is written, so a
block's rows never need re-quantising as the block fills:

* codes: OCP 8-bit floating point E4M3 (the "E4M3FN" variant: bias 7, no
  infinities, S.1111.111 is NaN, largest finite 448, smallest subnormal
  2^-9), encoded with round-to-nearest-even;
* scale: one power of two per row, stored as an OCP E8M0 byte (value
  2^(byte - 127)): the smallest 2^e with max|x| / 2^e <= 448, e clamped to
  [-126, 127]; an all-zero row takes e = 0;
* code = E4M3(x * 2^-e), and the row reads back as decode(code) * 2^e; a
  code of negative zero (0x80) is stored as 0x00, so stored codes never use
  0x80, which the other 8-bit E4M3 variant (no negative zero) reads as NaN;
* non-finite inputs (the pages say nothing of them; reading taken): the
  scale is chosen from the row's finite elements only, and an infinity or a
  NaN is stored as the NaN code with its sign (0x7F / 0xFF), so it reads
  back as NaN, as a non-finite value in a 16-bit cache would poison the
  attention that reads it.

Multiplying by 2^-e is exact in float32 (the inputs are float32-widened
16-bit or float32 values), so the only rounding is the E4M3 one.  Pins:
``tests/test_oracle_quant.py``.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

from .cache import copy_blocks, gather_blocks, scatter_blocks
from .slots import split_slot

E4M3_MAX = 448.0


def e4m3_decode(code: int) -> float:
    """Value of one E4M3 byte (NaN for S.1111.111)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * man * 2.0 ** -9          # subnormal: m/8 * 2^(1-7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def e4m3_encode(x: float) -> int:
    """Nearest E4M3 byte to the finite value x (|x| <= 448), ties to an even
    mantissa; the sign of zero is kept.  An infinity or a NaN gives the NaN
    code with its sign."""
    x = float(x)
    sign = 0x80 if np.signbit(x) else 0
    if not np.isfinite(x):
        return sign | 0x7F
    if abs(x) > E4M3_MAX:
        raise ValueError("E4M3 encode of an out-of-range value")
    a = abs(x)
    if a < 2.0 ** -6:
        return sign | int(np.rint(a * 2.0 ** 9))          # 0..8 (8 = smallest normal)
    E = int(np.floor(np.log2(a)))
    if 2.0 ** E > a:                                     # guard log2 rounding
        E -= 1
    elif 2.0 ** (E + 1) <= a:
        E += 1
    r = int(np.rint(a * 2.0 ** (3 - E)))                 # 8..16
    return sign | (((E + 7) << 3) + (r - 8))


def row_scale_exponent(row: np.ndarray) -> int:
    """e of the row's scale 2^e: smallest with max|x| <= 448 * 2^e, the
    maximum over the row's finite elements."""
    r = row.astype(np.float64)
    r = r[np.isfinite(r)]
    amax = float(np.max(np.abs(r))) if r.size else 0.0
    if amax == 0.0:
        return 0
    m, k = np.frexp(amax)                                 # amax = m * 2^k, m in [0.5, 1)
    M, E = 2.0 * m, int(k) - 1                            # amax = M * 2^E, M in [1, 2)
    e = E - 8 + (1 if M > 1.75 else 0)                    # 448 = 1.75 * 2^8
    return min(max(e, -126), 127)


def quantize_row(row: np.ndarray) -> Tuple[np.ndarray, int]:
    """(codes uint8 [D], scale byte) of one float32 row."""
    e = row_scale_exponent(row)
    scaled = row.astype(np.float32) * np.float32(2.0 ** -e)
    codes = np.array([e4m3_encode(v) for v in scaled], dtype=np.uint8)
    codes[codes == 0x80] = 0x00
    return codes, e + 127


def dequantize(codes: np.ndarray, scale_bytes: np.ndarray) -> np.ndarray:
    """float64 values of codes [..., D] with per-row scale bytes [...]."""
    table = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[codes] * np.exp2(scale_bytes.astype(np.float64) - 127.0)[..., None]


def quantize_rows(rows: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """quantize_row over the last axis of float32 ``rows`` [..., D], in
    numpy array form (same steps: the scale exponent from frexp of the row
    max, the exact power-of-two scaling, then E4M3 round to nearest even);
    returns (codes uint8 [..., D], scale bytes uint8 [...])."""
    x = rows.astype(np.float32)
    fin = np.isfinite(x)
    amax = np.where(fin, np.abs(x), 0.0).max(axis=-1).astype(np.float64)
    m, k = np.frexp(amax)
    e = (k - 1) - 8 + (2.0 * m > 1.75)
    e = np.where(amax == 0.0, 0, np.clip(e, -126, 127)).astype(np.int64)
    y = (x.astype(np.float64) * np.exp2(-e.astype(np.float64))[..., None])   # exact
    y = np.where(fin, y, 0.0)                            # non-finite elements: NaN code below
    a = np.abs(y)
    sign = np.where(np.signbit(y), 0x80, 0)
    sub = a < 2.0 ** -6
    E = np.floor(np.log2(np.where(sub, 1.0, a))).astype(np.int64)
    E = np.where(np.exp2(E.astype(np.float64)) > a, E - 1, E)                   # guard log2 rounding
    E = np.where(np.exp2(E.astype(np.float64) + 1) <= a, E + 1, E)
    r = np.rint(a * np.exp2((3 - E).astype(np.float64))).astype(np.int64)
    normal = ((E + 7) << 3) + (r - 8)
    code = np.where(sub, np.rint(a * 2.0 ** 9).astype(np.int64), normal)
    code = np.where(code == 0, 0, code | sign)
    code = np.where(fin, code, np.where(np.signbit(x), 0xFF, 0x7F))
    return code.astype(np.uint8), (e + 127).astype(np.uint8)


def new_fp8_pool(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int):
    """Codes [N, H_kv, bs, D] and scale bytes [N, H_kv, bs] for K and for V,
    filled with a poison pattern (code 0x7F is NaN; scale byte 0xFF)."""
    kc = np.full((num_blocks, num_kv_heads, block_size, head_dim), 0x7F, dtype=np.uint8)
    vc = kc.copy()
    ks = np.full((num_blocks, num_kv_heads, block_size), 0xFF, dtype=np.uint8)
    vs = ks.copy()
    return kc, vc, ks, vs


def write_kv_fp8(key: np.ndarray, value: np.ndarray, slot_mapping: Sequence[int],
                 key_cache: np.ndarray, value_cache: np.ndarray, key_scales: np.ndarray,
                 value_scales: np.ndarray, block_size: int) -> None:
    """Cache write ([MiniPaged-Qwen] §12) into FP8 blocks: token i's row of
    every head is quantised on its own and stored with its scale byte at
    (pb, h, off) = split(slot_mapping[i]).  key/value are float32 [T, H, D]
    (the widened inputs).  Slots outside the pool are skipped."""
    capacity = key_cache.shape[0] * block_size
    for i, slot in enumerate(slot_mapping):
        slot = int(slot)
        if slot < 0 or slot >= capacity:
            continue
        pb, off = split_slot(slot, block_size)
        key_cache[pb, :, off], key_scales[pb, :, off] = quantize_rows(key[i])
        value_cache[pb, :, off], value_scales[pb, :, off] = quantize_rows(value[i])


def copy_blocks_fp8(pairs: Sequence[Tuple[int, int]], key_cache: np.ndarray, value_cache: np.ndarray,
                    key_scales: np.ndarray, value_scales: np.ndarray) -> None:
    """Copy-on-write copies of 8-bit blocks ([impl-detail]
    "Copy-on-Write机制": the new block takes the shared block's k and v).
    A stored row is its codes together with its scale byte, so the whole-block
    copy of cache.copy_blocks is applied to the code arrays [N, H, bs, D] and
    to the scale arrays [N, H, bs] alike."""
    copy_blocks(pairs, key_cache, value_cache)
    copy_blocks(pairs, key_scales, value_scales)


def gather_blocks_fp8(ids: Sequence[int], key_cache: np.ndarray, value_cache: np.ndarray,
                      key_scales: np.ndarray, value_scales: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Swap-out staging of 8-bit blocks ([impl-detail] "异构内存支持"):
    (codes [n, 2, H, bs, D], scale bytes [n, 2, H, bs]) of blocks ``ids`` in
    order, K half then V half, as cache.gather_blocks stages them."""
    return gather_blocks(ids, key_cache, value_cache), gather_blocks(ids, key_scales, value_scales)


def scatter_blocks_fp8(codes: np.ndarray, scales: np.ndarray, ids: Sequence[int], key_cache: np.ndarray,
                       value_cache: np.ndarray, key_scales: np.ndarray, value_scales: np.ndarray) -> None:
    """Swap-in of 8-bit blocks: staged entry j (codes and scale bytes) back
    into block ids[j]."""
    scatter_blocks(codes, ids, key_cache, value_cache)
    scatter_blocks(scales, ids, key_scales, value_scales)


def decode_attention_fp8(q: np.ndarray, q_dtype: str, key_cache: np.ndarray,
                         value_cache: np.ndarray, key_scales: np.ndarray,
                         value_scales: np.ndarray, block_tables: np.ndarray,
                         context_lens: Sequence[int], scale: float) -> np.ndarray:
    """Paged decode attention over FP8 blocks: each sequence's rows are
    gathered in table order and truncated at L ([MiniPaged-Qwen] §13), read
    back as decode(code) * 2^e in float64, and fed to the same softmax
    attention as the 16-bit path.  q [B, H_q, D] in ``q_dtype`` storage."""
    from .attention import contiguous_attention, widen
    from .cache import gather_logical
    B, h_q, d = q.shape
    out = np.zeros((B, h_q, d), dtype=np.float64)
    bs = key_cache.shape[2]
    for b in range(B):
        L = int(context_lens[b])
        table = [int(x) for x in block_tables[b]]
        kc = gather_logical(key_cache, table, L)
        vc = gather_logical(value_cache, table, L)
        # scale bytes gathered the same way: [H, L]
        ks = gather_logical(key_scales[..., None], table, L)[..., 0]
        vs = gather_logical(value_scales[..., None], table, L)[..., 0]
        out[b] = contiguous_attention(widen(q[b], q_dtype), dequantize(kc, ks),
                                      dequantize(vc, vs), scale)
    return out


def prefill_attention_fp8(q: np.ndarray, q_dtype: str, q_start: Sequence[int], key_cache: np.ndarray,
                          value_cache: np.ndarray, key_scales: np.ndarray, value_scales: np.ndarray,
                          block_tables: np.ndarray, context_lens: Sequence[int], scale: float) -> np.ndarray:
    """Chunked-prefill attention over FP8 blocks: the causal multi-query
    attention of attention.prefill_attention ([impl-detail] "分块注意力"),
    with every cached row read back as decode(code) * 2^e in float64.
    q [T, H_q, D] in ``q_dtype`` storage.  Returns float64 [T, H_q, D]."""
    from .attention import prefill_attention, widen
    return prefill_attention(widen(q, q_dtype), q_start, dequantize(key_cache, key_scales),
                             dequantize(value_cache, value_scales), block_tables, context_lens, scale, "f64")
