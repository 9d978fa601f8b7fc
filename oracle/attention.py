"""Decode and chunked-prefill attention (oracle, test infrastructure only).

The quantity is [MiniPaged-Qwen] §1.1 / §13:
    O = softmax(scale * q K^T) V
for one new query per sequence against that sequence's L cached tokens, with
the GQA head map of §14 (kvh = qh // (H_q / H_kv)) and no causal mask (the
single decode query sits at the last position and sees all L tokens).

``decode_attention`` is the gather-then-contiguous form: rebuild each
sequence's logical K/V from the pool in table order, truncate at L, then do
ordinary softmax attention in float64 ([impl-detail] "分块注意力"
``paged_attention_forward``, corrected to truncate at L rather than reading
whole blocks, to apply the GQA map and to drop the causal mask).

``decode_attention_online`` walks the positions one at a time through the
block table with a running max / sum / accumulator, the "online softmax"
CPU reference [MiniPaged-Qwen] §17.3 names; it is the second route used to
check the first.

``prefill_attention`` is the multi-query form: a chunk of query rows at the
last positions of a sequence, each under the causal mask of [impl-detail]
"分块注意力".  Pins: ``tests/test_oracle_prefill.py``.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

from .cache import gather_logical
from .slots import kv_head_of


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values to float64.  bf16 is the upper half of
    an IEEE float32, so its 16-bit pattern shifted left by 16 is that float32."""
    if dtype == "bf16":
        a = np.asarray(a, dtype=np.uint16)
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype in ("f16", "f32", "f64"):
        return np.asarray(a).astype(np.float64)
    raise ValueError(dtype)


def contiguous_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one sequence on contiguous float64 inputs.

    q [H_q, D]; k, v [H_kv, L, D].  Returns [H_q, D]; zeros when L == 0
    (reading for an empty history: the pages leave it open).
    """
    h_q, d = q.shape
    h_kv, L, _ = k.shape
    out = np.zeros((h_q, d), dtype=np.float64)
    if L == 0:
        return out
    for qh in range(h_q):
        kvh = kv_head_of(qh, h_q, h_kv)
        s = float(scale) * (k[kvh] @ q[qh])
        p = np.exp(s - s.max())
        out[qh] = (p @ v[kvh]) / p.sum()
    return out


def decode_attention(q: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
                     block_tables: np.ndarray, context_lens: Sequence[int], scale: float,
                     dtype: str, seqs: Optional[Iterable[int]] = None) -> np.ndarray:
    """Paged decode attention, gather-then-contiguous, float64.

    q [B, H_q, D] stored dtype; caches [N, H_kv, bs, D]; block_tables [B, W];
    context_lens [B].  Returns float64 [B, H_q, D]; rows not listed in
    ``seqs`` (when given) are left as NaN.
    """
    B, h_q, d = q.shape
    out = np.full((B, h_q, d), np.nan, dtype=np.float64)
    rows = range(B) if seqs is None else seqs
    for b in rows:
        L = int(context_lens[b])
        table = [int(x) for x in block_tables[b]]
        kc = widen(gather_logical(key_cache, table, L), dtype)
        vc = widen(gather_logical(value_cache, table, L), dtype)
        out[b] = contiguous_attention(widen(q[b], dtype), kc, vc, scale)
    return out


def decode_attention_online(q_b: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
                            block_table: Sequence[int], L: int, scale: float,
                            dtype: str) -> np.ndarray:
    """One sequence, position by position, through the block table
    ([MiniPaged-Qwen] §13 addressing, §17.3 online softmax):
        pb = table[pos // bs], off = pos % bs,
        m' = max(m, s); acc = acc e^(m - m') + e^(s - m') v;
        l = l e^(m - m') + e^(s - m').
    Returns acc / l, float64 [H_q, D].  Meant for tiny inputs only."""
    h_q, d = q_b.shape
    h_kv = key_cache.shape[1]
    bs = key_cache.shape[2]
    q = widen(q_b, dtype)
    out = np.zeros((h_q, d), dtype=np.float64)
    if L == 0:
        return out
    for qh in range(h_q):
        kvh = kv_head_of(qh, h_q, h_kv)
        m = -np.inf
        l = 0.0
        acc = np.zeros(d, dtype=np.float64)
        for pos in range(L):
            pb = int(block_table[pos // bs])
            off = pos % bs
            k = widen(key_cache[pb, kvh, off], dtype)
            v = widen(value_cache[pb, kvh, off], dtype)
            s = float(scale) * float(k @ q[qh])
            m_new = max(m, s)
            a = np.exp(m - m_new)
            e = np.exp(s - m_new)
            acc = acc * a + e * v
            l = l * a + e
            m = m_new
        out[qh] = acc / l
    return out


def prefill_attention(q: np.ndarray, q_start: Sequence[int], key_cache: np.ndarray,
                      value_cache: np.ndarray, block_tables: np.ndarray,
                      context_lens: Sequence[int], scale: float, dtype: str) -> np.ndarray:
    """Chunked-prefill attention through block tables, float64.

    Sequence b holds L_b = context_lens[b] cached tokens (the chunk's own K/V
    already written, [MiniPaged-Qwen] §1.1 and §12); its n_b query rows are
    q[q_start[b] : q_start[b + 1]], the last n_b positions: row i sits at
    p = L_b - n_b + i and attends to positions 0 .. p with the causal mask of
    [impl-detail] "分块注意力" (``create_causal_mask``), the GQA map of
    [MiniPaged-Qwen] §14 and the gather of [MiniPaged-Qwen] §13.  A full
    prefill is n_b = L_b; decode is n_b = 1.  Rows with p < 0 get zeros.
    Returns float64 [T, H_q, D].
    """
    T, h_q, d = q.shape
    h_kv = key_cache.shape[1]
    out = np.zeros((T, h_q, d), dtype=np.float64)
    for b in range(len(context_lens)):
        L = int(context_lens[b])
        r0, r1 = int(q_start[b]), int(q_start[b + 1])
        n = r1 - r0
        if n == 0 or L == 0:
            continue
        table = [int(x) for x in block_tables[b]]
        k = widen(gather_logical(key_cache, table, L), dtype)      # [H_kv, L, D]
        v = widen(gather_logical(value_cache, table, L), dtype)
        qb = widen(q[r0:r1], dtype)                                 # [n, H_q, D]
        pos = L - n + np.arange(n)                                  # query positions
        mask = np.arange(L)[None, :] <= pos[:, None]                # [n, L] causal
        for qh in range(h_q):
            kvh = kv_head_of(qh, h_q, h_kv)
            s = float(scale) * (qb[:, qh, :] @ k[kvh].T)            # [n, L]
            s = np.where(mask, s, -np.inf)
            smax = s.max(axis=1, keepdims=True)
            live = np.isfinite(smax[:, 0])
            e = np.where(mask, np.exp(s - np.where(live[:, None], smax, 0.0)), 0.0)
            den = e.sum(axis=1, keepdims=True)
            o = (e @ v[kvh]) / np.where(den > 0, den, 1.0)
            out[r0:r1, qh, :] = np.where(live[:, None], o, 0.0)
    return out
