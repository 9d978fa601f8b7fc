"""Seeded synthetic inputs for the paged KV cache hot path.

This module is shared by the CPU oracle and by the GPU path (tests, bench,
smoke).  It only draws random numbers and lays out workload descriptions: it
contains none of the method's arithmetic (no slot computation, no block counts,
no attention).  Both sides replay the same event lists through their own block
manager and their own kernels.

Value distributions follow the workload descriptions: K/V/q ~ N(0, 1) drawn in
float32 and cast to the storage dtype with round-to-nearest-even.  Storage
arrays are numpy ``uint16`` bit patterns for bf16, ``float16`` for fp16 and
``float32`` for fp32.

Draw order for the single-step decode workloads:
  1. context lengths, 2. placement (free-list permutation or churn trace),
  3. history K/V per sequence in logical order (K then V per sequence),
  4. new-token K/V, 5. q.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Iterator, List, Optional, Tuple

import numpy as np

# Quiet-NaN bit patterns used to poison pool memory that no write touched.
POISON_BITS = {"bf16": 0x7FC5, "f16": 0x7E05, "f32": 0x7FC00005}

STORAGE_NP = {"bf16": np.uint16, "f16": np.float16, "f32": np.float32}
ELEM_BYTES = {"bf16": 2, "f16": 2, "f32": 4}


def to_storage(a32: np.ndarray, dtype: str) -> np.ndarray:
    """Cast float32 values to the storage dtype, round-to-nearest-even."""
    a32 = np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "f32":
        return a32
    if dtype == "f16":
        return a32.astype(np.float16)
    if dtype == "bf16":
        u = a32.view(np.uint32)
        bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        return ((u + bias) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(dtype)


def poison_array(shape, dtype: str) -> np.ndarray:
    bits = POISON_BITS[dtype]
    if dtype == "bf16":
        return np.full(shape, bits, dtype=np.uint16)
    if dtype == "f16":
        return np.full(shape, bits, dtype=np.uint16).view(np.float16)
    return np.full(shape, bits, dtype=np.uint32).view(np.float32)


def normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return to_storage(rng.standard_normal(shape, dtype=np.float32), dtype)


@dataclasses.dataclass(frozen=True)
class Config:
    index: int                 # 1-based; the seed is 1000 + index
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                 # "f32" | "f16" | "bf16"
    block_size: int
    num_blocks: int
    batch: int
    fixed_lens: Optional[Tuple[int, ...]] = None
    len_range: Optional[Tuple[int, int]] = None   # inclusive uniform range
    placement: str = "permutation"                # "permutation" | "churn" | "identity"
    churn_priors: int = 0
    partition_tokens: int = 0                      # 0: library default
    # serving trace
    steps: int = 0
    lognormal: Optional[Tuple[float, float]] = None
    clip: Optional[Tuple[int, int]] = None
    p_finish: float = 0.0

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(D), rounded to float32."""
        return float(np.float32(1.0) / np.sqrt(np.float32(self.head_dim)))


CONFIGS: Dict[str, Config] = {
    c.name: c
    for c in [
        Config(1, "tiny", 4, 4, 64, "f32", 16, 64, 4, fixed_lens=(40, 17, 1, 64)),
        Config(2, "qwen2_1p5b_b32", 12, 2, 128, "f16", 16, 8192, 32, len_range=(128, 2048)),
        Config(3, "qwen2_7b_b64", 28, 4, 128, "bf16", 16, 65536, 64, len_range=(512, 8192),
               placement="churn", churn_priors=500),
        Config(4, "long_splitk", 32, 8, 128, "bf16", 32, 9216, 8, fixed_lens=(32768,) * 8,
               partition_tokens=512),
        Config(5, "serving_trace", 32, 8, 128, "bf16", 16, 69632, 256, placement="identity",
               steps=200, lognormal=(6.0, 1.0), clip=(16, 4096), p_finish=0.01),
    ]
}
CONFIG_BY_INDEX = {c.index: c for c in CONFIGS.values()}


# ---------------------------------------------------------------------------
# Churn trace: a seeded stream of admit / grow / free events on prior
# sequences that scrambles the free list before the measured sequences are
# admitted.  The stream never depends on block-manager state; the number of
# live priors and the tokens each prior may gain are capped so that, for the
# 65,536-block pool of the batch-64 workload, no event can run out of blocks
# (100 live priors of at most 8192 + 512 tokens each).
# ---------------------------------------------------------------------------
CHURN_LIVE_CAP = 100
CHURN_GROW_CAP = 512
CHURN_ID_BASE = 1_000_000


def churn_events(rng: np.random.Generator, priors: int,
                 prompt_range=(16, 8192)) -> List[tuple]:
    """Events: ("prefill", id, n) | ("grow", ids, rounds) | ("free", id)."""
    events: List[tuple] = []
    live: List[int] = []
    grown: Dict[int, int] = {}
    next_id = CHURN_ID_BASE
    admitted = 0
    while admitted < priors:
        u = rng.random()
        if u < 0.4 or not live:
            if len(live) >= CHURN_LIVE_CAP:
                victim = live.pop(int(rng.integers(len(live))))
                events.append(("free", victim))
                continue
            n = int(rng.integers(prompt_range[0], prompt_range[1] + 1))
            events.append(("prefill", next_id, n))
            live.append(next_id)
            grown[next_id] = 0
            next_id += 1
            admitted += 1
        elif u < 0.8:
            k = min(8, len(live))
            pick = rng.choice(len(live), size=k, replace=False)
            rounds = int(rng.integers(1, 65))
            ids = [live[int(i)] for i in pick if grown[live[int(i)]] + rounds <= CHURN_GROW_CAP]
            if ids:
                for i in ids:
                    grown[i] += rounds
                events.append(("grow", tuple(ids), rounds))
        else:
            victim = live.pop(int(rng.integers(len(live))))
            events.append(("free", victim))
    order = rng.permutation(len(live))
    for i in order:
        events.append(("free", live[int(i)]))
    return events


@dataclasses.dataclass
class DecodeWorkload:
    """One measured decode step: history prefill, then append + write + attend."""
    cfg: Config
    context_lens: np.ndarray          # int32 [B], lengths after the measured append
    initial_free_order: Optional[np.ndarray]   # int32 [N] or None (identity)
    churn: List[tuple]
    hist_k: List[np.ndarray]          # per sequence [L_b - 1, H_kv, D] storage dtype
    hist_v: List[np.ndarray]
    new_k: np.ndarray                 # [B, H_kv, D]
    new_v: np.ndarray
    q: np.ndarray                     # [B, H_q, D]

    @property
    def seq_ids(self) -> List[int]:
        return list(range(len(self.context_lens)))


def decode_workload(cfg: Config, batch: Optional[int] = None) -> DecodeWorkload:
    """Seeded single-step decode workload for configs 1-4.

    ``batch`` (optional) keeps only the first ``batch`` sequences; all draws
    are still made for the full batch so that the kept sequences are
    identical to those of the full workload.
    """
    rng = np.random.default_rng(cfg.seed)
    B = cfg.batch
    if cfg.fixed_lens is not None:
        lens = np.array(cfg.fixed_lens, dtype=np.int32)
    else:
        lo, hi = cfg.len_range
        lens = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    order = None
    churn: List[tuple] = []
    if cfg.placement == "permutation":
        order = rng.permutation(cfg.num_blocks).astype(np.int32)
    elif cfg.placement == "churn":
        churn = churn_events(rng, cfg.churn_priors)
    keep = B if batch is None else int(batch)
    hk, hv = [], []
    shape_tail = (cfg.num_kv_heads, cfg.head_dim)
    for b in range(B):
        n = int(lens[b]) - 1
        k = normal(rng, (n,) + shape_tail, cfg.dtype)
        v = normal(rng, (n,) + shape_tail, cfg.dtype)
        if b < keep:
            hk.append(k)
            hv.append(v)
    new_k = normal(rng, (B,) + shape_tail, cfg.dtype)[:keep]
    new_v = normal(rng, (B,) + shape_tail, cfg.dtype)[:keep]
    q = normal(rng, (B, cfg.num_q_heads, cfg.head_dim), cfg.dtype)[:keep]
    return DecodeWorkload(cfg, lens[:keep].copy(), order, churn, hk, hv,
                          np.ascontiguousarray(new_k), np.ascontiguousarray(new_v),
                          np.ascontiguousarray(q))


def extra_step_tensors(cfg: Config, batch: int, count: int, seed_offset: int = 0):
    """Fresh new-token K/V and q for ``count`` further decode steps."""
    rng = np.random.default_rng(cfg.seed * 7919 + 17 + seed_offset)
    out = []
    for _ in range(count):
        k = normal(rng, (batch, cfg.num_kv_heads, cfg.head_dim), cfg.dtype)
        v = normal(rng, (batch, cfg.num_kv_heads, cfg.head_dim), cfg.dtype)
        q = normal(rng, (batch, cfg.num_q_heads, cfg.head_dim), cfg.dtype)
        out.append((k, v, q))
    return out


# ---------------------------------------------------------------------------
# Serving trace (config 5): 256 rows of live sequences, each step appends one
# token per row; after the step each row finishes with probability p and is
# refilled at once with a fresh prompt.
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class Refill:
    row: int
    old_id: int
    new_id: int
    prompt_len: int
    k: np.ndarray            # [prompt_len, H_kv, D]
    v: np.ndarray


@dataclasses.dataclass
class ServingStep:
    step: int
    new_k: np.ndarray        # [B, H_kv, D]
    new_v: np.ndarray
    q: np.ndarray            # [B, H_q, D]
    refills: List[Refill]    # applied after the step's attention


@dataclasses.dataclass
class ServingTrace:
    cfg: Config
    prompt_lens: np.ndarray  # int32 [B] for the initial rows (seq id = row)
    hist_k: List[np.ndarray]
    hist_v: List[np.ndarray]
    steps: Iterator[ServingStep]


def _prompt_len(rng, cfg: Config) -> int:
    mu, sd = cfg.lognormal
    lo, hi = cfg.clip
    return int(min(max(int(round(rng.lognormal(mu, sd))), lo), hi))


def serving_trace(cfg: Config, steps: Optional[int] = None, batch: Optional[int] = None) -> ServingTrace:
    rng = np.random.default_rng(cfg.seed)
    B = cfg.batch if batch is None else int(batch)
    n_steps = cfg.steps if steps is None else int(steps)
    tail = (cfg.num_kv_heads, cfg.head_dim)
    prompts = np.array([_prompt_len(rng, cfg) for _ in range(B)], dtype=np.int32)
    hk = []
    hv = []
    for b in range(B):
        hk.append(normal(rng, (int(prompts[b]),) + tail, cfg.dtype))
        hv.append(normal(rng, (int(prompts[b]),) + tail, cfg.dtype))

    def gen():
        row_ids = list(range(B))
        next_id = B
        for s in range(n_steps):
            k = normal(rng, (B,) + tail, cfg.dtype)
            v = normal(rng, (B,) + tail, cfg.dtype)
            q = normal(rng, (B, cfg.num_q_heads, cfg.head_dim), cfg.dtype)
            fin = np.nonzero(rng.random(B) < cfg.p_finish)[0]
            refills = []
            for r in fin:
                r = int(r)
                n = _prompt_len(rng, cfg)
                rk = normal(rng, (n,) + tail, cfg.dtype)
                rv = normal(rng, (n,) + tail, cfg.dtype)
                refills.append(Refill(r, row_ids[r], next_id, n, rk, rv))
                row_ids[r] = next_id
                next_id += 1
            yield ServingStep(s, k, v, q, refills)

    return ServingTrace(cfg, prompts, hk, hv, gen())


# ---------------------------------------------------------------------------
# Random manager op traces for host-logic parity tests.
# ---------------------------------------------------------------------------
def manager_op_trace(seed: int, n_ops: int, max_id: int = 40, max_prefill: int = 80):
    """Random ops, including ones that must fail (double free, unknown ids,
    prefill of a live id, OOM on a small pool, duplicate ids in a batch)."""
    rng = np.random.default_rng(seed)
    ops = []
    for _ in range(n_ops):
        u = rng.random()
        if u < 0.3:
            ops.append(("prefill", int(rng.integers(max_id)), int(rng.integers(0, max_prefill + 1))))
        elif u < 0.55:
            ops.append(("append", int(rng.integers(max_id))))
        elif u < 0.75:
            k = int(rng.integers(1, 9))
            ids = [int(x) for x in rng.integers(max_id, size=k)]
            ops.append(("append_batch", tuple(ids)))
        elif u < 0.95:
            ops.append(("free", int(rng.integers(max_id))))
        else:
            ops.append(("can_allocate", int(rng.integers(0, 4 * max_prefill))))
    return ops


def manager_share_trace(seed: int, n_ops: int, max_id: int = 24, max_prefill: int = 40):
    """Random ops with prefix sharing: prefills, shares of a (random-length)
    prefix of a donor, single and batched appends, frees and capacity
    queries, including ones that must fail (unknown donors, live targets,
    prefixes longer than the donor, OOM, duplicate ids)."""
    rng = np.random.default_rng(seed)
    ops = []
    for _ in range(n_ops):
        u = rng.random()
        if u < 0.2:
            ops.append(("prefill", int(rng.integers(max_id)), int(rng.integers(0, max_prefill + 1))))
        elif u < 0.4:
            ops.append(("share", int(rng.integers(max_id)), int(rng.integers(max_id)),
                        int(rng.integers(0, max_prefill + 8))))
        elif u < 0.6:
            ops.append(("append", int(rng.integers(max_id))))
        elif u < 0.8:
            k = int(rng.integers(1, 9))
            ids = [int(x) for x in rng.integers(max_id, size=k)]
            ops.append(("append_batch", tuple(ids)))
        elif u < 0.97:
            ops.append(("free", int(rng.integers(max_id))))
        else:
            ops.append(("can_allocate", int(rng.integers(0, 4 * max_prefill))))
    return ops


__all__ = [
    "manager_share_trace",
    "CONFIGS", "CONFIG_BY_INDEX", "Config", "DecodeWorkload", "decode_workload",
    "serving_trace", "ServingTrace", "ServingStep", "Refill", "churn_events",
    "manager_op_trace", "extra_step_tensors", "to_storage", "poison_array", "normal",
    "POISON_BITS", "STORAGE_NP", "ELEM_BYTES",
]
