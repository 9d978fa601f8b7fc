#!/usr/bin/env python3
"""Benchmark of the paged KV cache decode hot path on one MI355X.

One step = the whole hot path over one batch: host block-manager append for
every sequence, then the write of the new K/V rows (with the blocks the
append opened published into the device block table) and paged decode
attention over the updated cache.  With the stream attention path the write
runs inside the attention launch (pkv_decode_step), followed by the split-K
merge launch; ``--separate-write`` runs it as its own launch instead.
Default workload: the Qwen2-7B-shaped batch-64 decode (H_q 28, H_kv 4,
D 128, bf16, block_size 16, context lengths U[512, 8192], pool of 65,536
blocks fragmented by a seeded churn of 500 prior sequences).  Inputs are
seeded synthetic tensors (``synth``), resident in HBM before timing starts.

Prints ONE JSON line.  ``value`` is the KV bytes the steps' attention must
read (sum over sequences of L * H_kv * 2 * D * elem_bytes) divided by the
wall time of the timed steps.  ``roofline`` is for the step's first launch
(the dominant kernel): its algorithmic bytes (the KV bytes read, plus the
new rows written when the write runs inside it) over its mean duration from
HIP events recorded on the launch stream around it on every fifth timed
step.

``--config serving_trace`` runs the serving-trace workload instead (its
own JSON line: the trace's 200 decode steps with per-step finishes and
refills; see measure_serving).

    python bench.py [--steps K] [--warmup W] [--config NAME]
    python bench.py --calibrate-copy      # plain 1 GiB copy, for PMC scaling
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E peak, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix peak
CSRC = os.path.join(ROOT, "paged_kv_cache_128_amd", "csrc")
# the decode attention kernels are built from this file and the headers it includes
KERNEL_SOURCES = [os.path.join(CSRC, "pkv_kernels.hip"), os.path.join(CSRC, "pkv_internal.h"),
                  os.path.join(CSRC, "pkv_fp8_codec.h"), os.path.join(ROOT, "include", "pkv.h")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel_name: str, workload: str):
    """HBM bytes per launch from the committed PMC summary
    profiles/<kernel>_<workload>.md, if it was taken from the current kernel
    source."""
    path = os.path.join(ROOT, "profiles", f"{kernel_name}_{workload}.md")
    if not os.path.exists(path):
        return None, None
    text = open(path).read()
    sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    tb = re.search(r"traffic_bytes_per_launch:\s*([0-9.]+)", text)
    if not sha or not tb or sha.group(1) != kernel_source_sha():
        return None, None
    return float(tb.group(1)), sha.group(1)


def calibrate_copy():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_launch": n,
                      "bytes_written_per_launch": n, "launches": 5}), flush=True)


def cpu_baseline(cfg, wl, budget_s: float, reps: int = 3):
    """The CPU oracle, untuned, on the same workload: churned pool state and
    history prefill (untimed), then per sequence the measured append, write
    and float64 gather-then-contiguous attention (timed).  Sequences are
    taken in order until ``budget_s`` of timed work; the whole pass is
    repeated ``reps`` times on a fresh replay and the median pass reported."""
    import oracle
    from oracle.replay import replay_churn
    import synth
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        passes = [_cpu_pass(cfg, wl, budget_s, oracle, replay_churn, synth) for _ in range(reps)]
    passes.sort(key=lambda p: p[0] / p[2])
    nbytes, nseq, secs = passes[len(passes) // 2]
    log(f"cpu baseline: {nseq} sequences, {nbytes} KV bytes in {secs:.2f}s (median of {reps})")
    return {"value": nbytes / secs / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {nseq} of {len(wl.context_lens)} sequences of the same workload "
                      f"(append + write + float64 gather-then-contiguous attention), "
                      f"{nbytes} KV bytes in {secs:.2f} s on one host thread, median of {reps} passes",
            "decode_tokens_per_s": nseq / secs}


def _cpu_pass(cfg, wl, budget_s, oracle, replay_churn, synth):
    mgr = oracle.BlockManager(cfg.num_blocks, cfg.block_size, wl.initial_free_order)
    replay_churn(mgr, wl.churn)
    fill = synth.poison_array((), cfg.dtype)
    kc, vc = oracle.new_pool(cfg.num_blocks, cfg.num_kv_heads, cfg.block_size, cfg.head_dim, fill)
    elem = synth.ELEM_BYTES[cfg.dtype]
    done_bytes = 0
    done_seqs = 0
    elapsed = 0.0
    for b in range(len(wl.context_lens)):
        slots = mgr.allocate_for_prefill(b, int(wl.context_lens[b]) - 1)
        oracle.write_kv(wl.hist_k[b], wl.hist_v[b], slots, kc, vc, cfg.block_size)
        t0 = time.perf_counter()
        step = [mgr.append_slot_for_decode(b)]
        oracle.write_kv(wl.new_k[b:b + 1], wl.new_v[b:b + 1], step, kc, vc, cfg.block_size)
        L = mgr.context_len(b)
        table = np.array([mgr.block_table(b)], dtype=np.int32)
        oracle.decode_attention(wl.q[b:b + 1], kc, vc, table, [L], cfg.scale, cfg.dtype)
        elapsed += time.perf_counter() - t0
        done_bytes += L * cfg.num_kv_heads * 2 * cfg.head_dim * elem
        done_seqs += 1
        if elapsed >= budget_s:
            break
    return done_bytes, done_seqs, elapsed


def measure_block_copy(eng, pairs: int = 256, iters: int = 50):
    """Copy-on-write block copies (pkv_copy_blocks) on the workload's pool:
    ``pairs`` allocated blocks copied into free ones per launch, timed with
    HIP events around ``iters`` back-to-back launches.  Algorithmic bytes:
    every copied block is read once and written once."""
    import torch
    import paged_kv_cache_128_amd as pkv
    free = np.array(eng.manager.free_list()[:pairs], dtype=np.int32)
    tabs = eng.tables.cpu().numpy()
    used = tabs[tabs >= 0][:pairs].astype(np.int32)
    n = min(len(free), len(used))
    if n == 0:
        return None
    src, dst = used[:n], free[:n]
    block_bytes = 2 * eng.num_kv_heads * eng.block_size * eng.head_dim * eng.pool.element_size()
    for _ in range(5):
        pkv.copy_blocks(src, dst, eng.key_cache, eng.value_cache)
    torch.cuda.synchronize()
    # back-to-back launches between one event pair, as copies arrive in a
    # serving loop (an isolated launch would time mostly the launch itself)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        pkv.copy_blocks(src, dst, eng.key_cache, eng.value_cache)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / iters
    moved = 2 * n * block_bytes
    gbps = moved / (us * 1e-6) / 1e9
    log(f"block copy: {n} blocks of {block_bytes} B in {us:.2f} us per launch ({gbps:.0f} GB/s)")
    return {"kernel": "block_copy_kernel", "blocks_per_launch": n, "block_bytes": block_bytes,
            "algorithmic_bytes_per_launch": moved, "mean_launch_us": round(us, 3),
            "achieved_gbps": round(gbps, 2), "peak_gbps": HBM_PEAK_GBPS,
            "frac": round(gbps / HBM_PEAK_GBPS, 4)}


def measure_swap(eng, seqs: int = 8, iters: int = 5):
    """Swap to host on the workload's pool: the first ``seqs`` sequences'
    blocks gathered into a staging array (pkv_gather_blocks, HBM-bound) and
    copied to pinned host memory, timed separately with HIP events; the
    sequences are then swapped back in.  Reported: staging GB/s (read + write
    of the blocks), device-to-host GB/s, and an attention launch's time alone
    and with the copy in flight on a side stream (as the engine queues it)."""
    import torch
    import paged_kv_cache_128_amd as pkv
    seqs = min(seqs, len(eng.row_seq))
    ids = np.concatenate([np.array(eng.manager.block_table(s), dtype=np.int32) for s in range(seqs)])
    block_bytes = 2 * eng.num_kv_heads * eng.block_size * eng.head_dim * eng.pool.element_size()
    staged = pkv.gather_blocks(ids, eng.key_cache, eng.value_cache)
    host = torch.empty(staged.shape, dtype=staged.dtype, pin_memory=True)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    for _ in range(iters):
        pkv.gather_blocks(ids, eng.key_cache, eng.value_cache, staging=staged)
    ev[1].record()
    for _ in range(iters):
        host.copy_(staged, non_blocking=True)
    ev[2].record()
    torch.cuda.synchronize()
    g_us = ev[0].elapsed_time(ev[1]) * 1e3 / iters
    c_us = ev[1].elapsed_time(ev[2]) * 1e3 / iters
    nbytes = len(ids) * block_bytes
    # The engine's swap_out queues the copy on a side stream: an attention
    # launch over every row on the compute stream, alone and with that copy
    # in flight beside it (median of a few launches each).
    rows = len(eng.row_seq)
    qa = torch.randn((rows, eng._nq, eng.head_dim), device="cuda").to(eng.dtype)
    lens_d = eng.d_lens[:rows]
    maxl = int(lens_d.max())
    cs = torch.cuda.Stream()

    def attn_us(with_copy):
        ts = []
        for _ in range(iters):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            if with_copy:
                with torch.cuda.stream(cs):
                    host.copy_(staged, non_blocking=True)
            e0.record()
            eng.attend(qa, lens_d, 0.088, maxl)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(ts))
    alone, beside = attn_us(False), attn_us(True)
    log(f"swap: {len(ids)} blocks ({nbytes / 1e6:.1f} MB): gather {g_us:.1f} us, device-to-host {c_us:.1f} us; "
        f"attention {alone:.1f} us alone, {beside:.1f} us beside the copy")
    return {"kernel": "block_stage_kernel<gather>", "blocks": int(len(ids)), "bytes": int(nbytes),
            "gather_us": round(g_us, 2), "gather_gbps": round(2 * nbytes / (g_us * 1e-6) / 1e9, 1),
            "gather_frac_hbm": round(2 * nbytes / (g_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "device_to_host_us": round(c_us, 2),
            "device_to_host_gbps": round(nbytes / (c_us * 1e-6) / 1e9, 1),
            "attention_us_alone": round(alone, 2), "attention_us_beside_copy": round(beside, 2)}


def measure_prefill(cfg, seqs: int = 8, prompt: int = 2048, iters: int = 20, seed: int = 2024, kv8: bool = False):
    """Full-prompt prefill attention (paged_prefill_attention) with the
    workload's head shape: ``seqs`` prompts of ``prompt`` tokens admitted and
    written through the engine, then the attention launch timed with HIP
    events around ``iters`` back-to-back launches after 0.3 s of untimed
    ones.  Useful FLOPs: row i of a
    prompt sees i + 1 keys, 4 * D FLOPs per key and query head (Q.K and P.V).
    ``kv8``: the same over an 8-bit pool (paged_prefill_attention_fp8: the
    blocks' dequantisation into the 16-bit staging, then the prefill kernel,
    both inside each timed launch)."""
    import torch
    from paged_kv_cache_128_amd.engine import PagedKVEngine
    import paged_kv_cache_128_amd as pkv
    tdtype = {"bf16": torch.bfloat16, "f16": torch.float16}[cfg.dtype]
    bs, D, hq, hkv = cfg.block_size, cfg.head_dim, cfg.num_q_heads, cfg.num_kv_heads
    per = -(-prompt // bs)
    g = torch.Generator(device="cuda").manual_seed(seed)
    eng = PagedKVEngine(seqs * per + 8, hkv, bs, D, torch.float8_e4m3fn if kv8 else tdtype, seqs, per,
                        np.random.default_rng(seed).permutation(seqs * per + 8), num_q_heads=hq)
    T = seqs * prompt
    k = torch.randn((T, hkv, D), device="cuda", generator=g).to(tdtype)
    v = torch.randn((T, hkv, D), device="cuda", generator=g).to(tdtype)
    q = torch.randn((T, hq, D), device="cuda", generator=g).to(tdtype)
    scale = 1.0 / float(np.sqrt(D))
    out = eng.prefill_chunk(list(range(seqs)), list(range(seqs)), [prompt] * seqs, k, v, q, scale)
    qs = torch.arange(0, T + 1, prompt, dtype=torch.int32, device="cuda")
    lens = torch.full((seqs,), prompt, dtype=torch.int32, device="cuda")
    if kv8:
        ws = torch.empty(pkv.prefill_fp8_workspace_size(seqs, prompt, eng.key_cache, eng.value_cache),
                         dtype=torch.uint8, device="cuda")

        def launch():
            pkv.paged_prefill_attention_fp8(q, qs, eng.key_cache, eng.value_cache, eng.key_scales,
                                            eng.value_scales, eng.tables, lens, scale, max_q_len=prompt,
                                            max_context_len=prompt, out=out, workspace=ws)
    else:
        def launch():
            pkv.paged_prefill_attention(q, qs, eng.key_cache, eng.value_cache, eng.tables, lens, scale,
                                        max_q_len=prompt, max_context_len=prompt, out=out)
    # warm-up: under the matrix-core load the clocks take a few hundred
    # milliseconds to settle (back-to-back batches measured 490, 429 and
    # 415 us), so launches run for 0.3 s before the timed ones
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < 0.3:
        for _ in range(10):
            launch()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        launch()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / iters
    flops = seqs * (prompt * (prompt + 1) // 2) * hq * 4 * D
    tflops = flops / (us * 1e-6) / 1e12
    log(f"prefill{' over 8-bit KV' if kv8 else ''}: {seqs} x {prompt} tokens in {us:.1f} us per launch "
        f"({tflops:.0f} TFLOP/s)")
    kname = (f"dequant_blocks_kernel + prefill_kernel<{cfg.dtype}, D={D}>" if kv8
             else f"prefill_kernel<{cfg.dtype}, D={D}>")
    return {"kernel": kname, "workload": f"{seqs} prompts of {prompt} "
            f"tokens, H_q={hq} H_kv={hkv}, causal, full prefill" + (", 8-bit KV pool" if kv8 else ""),
            "mean_launch_us": round(us, 2),
            "useful_flops_per_launch": flops, "achieved_tflops": round(tflops, 1),
            "bound": "mfma", "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "prefill_tokens_per_s": round(seqs * prompt / (us * 1e-6), 1)}


def measure_serving(cfg, args):
    """The serving-trace workload (``--config serving_trace``): 256 rows
    prefilled with their prompts, then the trace's decode steps, each row
    finishing with its per-step probability and refilled at once with a
    fresh prompt.  Every step's inputs and every refill's prompt K/V are
    generated and placed in HBM before the timed loop.  Per step, HIP events
    bracket the decode step (host append, the fused write + attention launch,
    the merge) and the refills after it (releases, then the step's admissions
    as one prefill_many: allocation, one prompt write, one table update).
    Prints one JSON line: K/V GB/s and decode tokens/s over the decode-step
    time, and the refill time separately."""
    import torch
    import synth
    from paged_kv_cache_128_amd.engine import PagedKVEngine
    tdtype = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[cfg.dtype]
    elem = synth.ELEM_BYTES[cfg.dtype]

    def dev(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    t_gen = time.perf_counter()
    tr = synth.serving_trace(cfg)
    B, H, D = cfg.batch, cfg.num_kv_heads, cfg.head_dim
    width = -(-(cfg.clip[1] + cfg.steps) // cfg.block_size)
    eng = PagedKVEngine(cfg.num_blocks, H, cfg.block_size, D, tdtype, B, width, None, num_q_heads=cfg.num_q_heads)
    eng.prefill_many(list(range(B)), list(range(B)), [int(x) for x in tr.prompt_lens],
                     dev(np.concatenate(tr.hist_k)), dev(np.concatenate(tr.hist_v)))
    # each step's refills as one admission: their prompts concatenated
    steps = [(dev(st.new_k), dev(st.new_v), dev(st.q),
              ([r.row for r in st.refills], [r.new_id for r in st.refills], [r.k.shape[0] for r in st.refills],
               dev(np.concatenate([r.k for r in st.refills])) if st.refills else None,
               dev(np.concatenate([r.v for r in st.refills])) if st.refills else None))
             for st in tr.steps]
    log(f"serving trace: {len(steps)} steps generated and resident in {time.perf_counter() - t_gen:.1f}s")
    row_ids = np.arange(B, dtype=np.int64)
    out = torch.empty((B, cfg.num_q_heads, D), dtype=torch.float32, device="cuda")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in steps]
    kv_bytes = 0
    n_refill = refill_tokens = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for (k, v, q, refills), ev in zip(steps, evs):
        ev[0].record()
        eng.decode_step(row_ids, k, v, q, cfg.scale, out=out)
        kv_bytes += int(eng.lens[:B].astype(np.int64).sum()) * H * 2 * D * elem
        ev[1].record()
        rows, new_ids, plens, rk, rv = refills
        if rows:
            for row, new_id in zip(rows, new_ids):
                eng.free(int(row_ids[row]))
                row_ids[row] = new_id
            eng.prefill_many(new_ids, rows, plens, rk, rv)
            n_refill += len(rows)
            refill_tokens += int(sum(plens))
        ev[2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_s = sum(e[0].elapsed_time(e[1]) for e in evs) / 1e3
    ref_s = sum(e[1].elapsed_time(e[2]) for e in evs) / 1e3
    tokens = B * len(steps)
    log(f"serving trace: {1e6 * dec_s / len(steps):.1f} us per decode step, {kv_bytes / len(steps) / 1e6:.1f} MB "
        f"K/V per step, {n_refill} refills ({refill_tokens} prompt tokens) in {1e3 * ref_s:.2f} ms")
    print(json.dumps({
        "metric": "paged decode attention KV-read GB/s (% of HBM peak) + decode tokens/s",
        "value": round(kv_bytes / dec_s / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": len(steps), "warmup": 0,
        "ms_per_step": round(dec_s * 1e3 / len(steps), 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {B} rows, prompts clip(round(lognormal{tuple(cfg.lognormal)}), "
                               f"{cfg.clip[0]}, {cfg.clip[1]}), {len(steps)} decode steps, finish probability "
                               f"{cfg.p_finish} per row and step, refilled at once",
                   "batch": B},
        "pct_hbm_peak": round(100 * kv_bytes / dec_s / 1e9 / HBM_PEAK_GBPS, 1),
        "decode_tokens_per_s": round(tokens / dec_s, 1),
        "decode_tokens_per_s_with_refills": round(tokens / (dec_s + ref_s), 1),
        "wall_tokens_per_s": round(tokens / wall, 1),
        "refills": n_refill, "refill_prompt_tokens": refill_tokens, "refill_ms": round(ref_s * 1e3, 3),
        "kernel_source_sha256_16": kernel_source_sha(),
    }), flush=True)


def measure_fp8(cfg, wl, args, ring, base, total_steps, width, tokens_per_s_16):
    """The same workload with an 8-bit KV pool (E4M3 codes + one scale byte
    per row; the history quantised by the prefill write): decode steps of
    append, quantising step write and 8-bit attention + merge.  Reported
    beside the 16-bit headline: KV bytes actually read (codes and scale
    bytes) per second, decode tokens/s, and the 8-bit attention kernel's
    roofline from HIP events on every --event-every-th step."""
    import torch
    from paged_kv_cache_128_amd.engine import PagedKVEngine
    B = len(wl.context_lens)
    eng = PagedKVEngine(cfg.num_blocks, cfg.num_kv_heads, cfg.block_size, cfg.head_dim,
                        torch.float8_e4m3fn, B, width, wl.initial_free_order, partition_tokens=0,
                        num_q_heads=cfg.num_q_heads)
    for ev in wl.churn:
        if ev[0] == "prefill":
            eng.manager.allocate_for_prefill(ev[1], ev[2], want_slots=False)
        elif ev[0] == "grow":
            for _ in range(ev[2]):
                eng.manager.append_slots_for_decode(list(ev[1]))
        else:
            eng.manager.free_sequence(ev[1])
    def dev(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    hk, hv = dev(np.concatenate(wl.hist_k)), dev(np.concatenate(wl.hist_v))
    eng.prefill_many(list(range(B)), list(range(B)), [int(L) - 1 for L in wl.context_lens], hk, hv)
    del hk, hv
    ids = np.arange(B, dtype=np.int64)
    out = torch.empty((B, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
    row_bytes = cfg.num_kv_heads * 2 * (cfg.head_dim + 1)       # K and V codes + scale bytes per token

    def kv8(step):
        return int((base + step).sum()) * row_bytes

    for s_ in range(args.warmup):
        k, v, q = ring[s_ % len(ring)]
        eng.decode_step(ids, k, v, q, cfg.scale, out=out, fused=not args.separate_write)
    timed = [i for i in range(args.steps) if i % max(1, args.event_every) == 0]
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in timed}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        k, v, q = ring[(args.warmup + i) % len(ring)]
        eng.decode_step(ids, k, v, q, cfg.scale, out=out, events=evs.get(i), fused=not args.separate_write)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = np.array([evs[i][0].elapsed_time(evs[i][1]) for i in timed])
    merge_ms = np.array([evs[i][1].elapsed_time(evs[i][2]) for i in timed])
    step_bytes = np.array([kv8(args.warmup + i) for i in range(args.steps)], dtype=np.float64)
    fused = not args.separate_write
    # the fused launch also writes the B new rows (codes and scale bytes)
    alg = float(step_bytes[timed].mean()) + (B * row_bytes if fused else 0)
    achieved = alg / (float(kern_ms.mean()) / 1e3) / 1e9
    kname = "attn_stream8_step_kernel" if fused else "attn_stream8_kernel"
    tps = B * args.steps / wall
    log(f"fp8 KV: {wall * 1e6 / args.steps:.1f} us/step, attention kernel {kern_ms.mean() * 1e3:.1f} us, "
        f"merge {merge_ms.mean() * 1e3:.1f} us, KV {step_bytes.mean() / 1e6:.1f} MB/step")
    return {
        "kv_dtype": "fp8_e4m3 codes + e8m0 row scales",
        "value": round(float(step_bytes.sum()) / wall / 1e9, 2),
        "unit": "GB/s",
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "kv_bytes_per_step": round(float(step_bytes.mean())),
        "decode_tokens_per_s": round(tps, 1),
        "tokens_per_s_vs_16bit": round(tps / tokens_per_s_16, 3),
        "roofline": {
            "kernel": f"{kname}<{cfg.dtype} q, D={cfg.head_dim}, "
                      f"G={cfg.num_q_heads // cfg.num_kv_heads}>",
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": recorded_traffic(kname, cfg.name)[0],
            "mean_launch_us": round(float(kern_ms.mean()) * 1e3, 3),
            "algorithmic_bytes_per_launch": round(alg),
        },
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="qwen2_7b_b64")
    ap.add_argument("--partition-tokens", type=int, default=-1,
                    help="split-K partition length (-1: the workload's own, else library default)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-iters", type=int, default=20)
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--event-every", type=int, default=5,
                    help="record the kernel-timing events on every n-th timed step")
    ap.add_argument("--separate-write", action="store_true",
                    help="run the step's write as its own launch instead of inside the attention")
    ap.add_argument("--no-fp8", action="store_true", help="skip the 8-bit KV measurement")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill attention measurement")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return

    import torch
    import synth
    from paged_kv_cache_128_amd.engine import PagedKVEngine

    cfg = synth.CONFIGS[args.config]
    if cfg.steps:
        measure_serving(cfg, args)
        return
    tdtype = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[cfg.dtype]
    t_gen = time.perf_counter()
    wl = synth.decode_workload(cfg)
    B = len(wl.context_lens)
    log(f"workload {cfg.name}: B={B} sum(L)={int(wl.context_lens.sum())} "
        f"(generated in {time.perf_counter() - t_gen:.1f}s)")

    def dev(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    total_steps = args.warmup + args.steps
    width = int(-(-(int(wl.context_lens.max()) + total_steps) // cfg.block_size))
    part = cfg.partition_tokens if args.partition_tokens < 0 else args.partition_tokens
    eng = PagedKVEngine(cfg.num_blocks, cfg.num_kv_heads, cfg.block_size, cfg.head_dim, tdtype, B,
                        width, wl.initial_free_order, partition_tokens=part,
                        num_q_heads=cfg.num_q_heads)
    for ev in wl.churn:
        if ev[0] == "prefill":
            eng.manager.allocate_for_prefill(ev[1], ev[2], want_slots=False)
        elif ev[0] == "grow":
            for _ in range(ev[2]):
                eng.manager.append_slots_for_decode(list(ev[1]))
        else:
            eng.manager.free_sequence(ev[1])
    eng.prefill_many(list(range(B)), list(range(B)), [int(L) - 1 for L in wl.context_lens],
                     dev(np.concatenate(wl.hist_k)), dev(np.concatenate(wl.hist_v)))
    tabs = eng.tables.cpu().numpy()
    adj = sum(int(np.count_nonzero(np.diff(r[r >= 0]) == 1)) for r in tabs)
    pairs = sum(max(int((r >= 0).sum()) - 1, 0) for r in tabs)
    frag = adj / pairs if pairs else 0.0
    del tabs

    ring = [(dev(wl.new_k), dev(wl.new_v), dev(wl.q))]
    for k, v, q in synth.extra_step_tensors(cfg, B, 7):
        ring.append((dev(k), dev(v), dev(q)))
    ids = np.arange(B, dtype=np.int64)
    out = torch.empty((B, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
    elem = synth.ELEM_BYTES[cfg.dtype]
    base = wl.context_lens.astype(np.int64)          # lengths after the first decode step

    def kv_bytes(step):
        return int((base + step).sum()) * cfg.num_kv_heads * 2 * cfg.head_dim * elem

    torch.cuda.synchronize()
    for s in range(args.warmup):
        k, v, q = ring[s % len(ring)]
        eng.decode_step(ids, k, v, q, cfg.scale, out=out, fused=not args.separate_write)
    torch.cuda.synchronize()

    # Kernel timing: HIP events around the step's kernels on every
    # --event-every-th timed step (each recorded event costs a few us of GPU
    # time, so events on every step would slow the very steps being timed).
    timed = [i for i in range(args.steps) if i % max(1, args.event_every) == 0]
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in timed}
    if torch.distributed.is_available() and torch.distributed.is_initialized():
        torch.distributed.barrier()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        s = args.warmup + i
        k, v, q = ring[s % len(ring)]
        eng.decode_step(ids, k, v, q, cfg.scale, out=out, events=evs.get(i), fused=not args.separate_write)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    split_ms = np.array([evs[i][0].elapsed_time(evs[i][1]) for i in timed])
    merge_ms = np.array([evs[i][1].elapsed_time(evs[i][2]) for i in timed])
    step_bytes = np.array([kv_bytes(args.warmup + i) for i in range(args.steps)], dtype=np.float64)
    timed_bytes = step_bytes[timed]
    total_kv = float(step_bytes.sum())
    value = total_kv / wall / 1e9
    tokens_per_s = B * args.steps / wall
    split_avg_s = float(split_ms.mean()) / 1e3
    # the first launch of a step also writes the step's new K/V rows when fused
    new_row_bytes = B * cfg.num_kv_heads * 2 * cfg.head_dim * elem
    attn_gbps = float(timed_bytes.mean()) / (float((split_ms + merge_ms).mean()) / 1e3) / 1e9
    log(f"timed {args.steps} steps: {wall * 1e6 / args.steps:.1f} us/step, split kernel "
        f"{split_ms.mean() * 1e3:.1f} us, merge {merge_ms.mean() * 1e3:.1f} us, "
        f"KV {step_bytes.mean() / 1e6:.1f} MB/step")

    # attention only, with a 1 GiB read before each launch pair (cold caches;
    # a read leaves no dirty lines behind to be written back during the launch)
    flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    lens_dev = torch.from_numpy(eng.manager.context_lens(list(range(B)))).cuda()
    maxlen = int(lens_dev.max().item())
    cold_bytes = int(lens_dev.sum().item()) * cfg.num_kv_heads * 2 * cfg.head_dim * elem
    q = ring[0][2]
    cold = []
    for _ in range(args.cold_iters):
        flush.sum()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        eng.attend(q, lens_dev, cfg.scale, maxlen, out=out, events=e)
        torch.cuda.synchronize()
        cold.append((e[0].elapsed_time(e[1]), e[0].elapsed_time(e[2])))
    cold = np.array(cold)
    del flush
    block_copy = measure_block_copy(eng)
    swap = measure_swap(eng)
    fp8 = None
    if not args.no_fp8 and cfg.dtype in ("bf16", "f16") and cfg.head_dim == 128:
        fp8 = measure_fp8(cfg, wl, args, ring, base, total_steps, width, tokens_per_s)
    prefill = prefill8 = None
    if not args.no_prefill and cfg.dtype in ("bf16", "f16") and cfg.head_dim == 128:
        prefill = measure_prefill(cfg)
        if cfg.dtype == "bf16" and not args.no_fp8:
            prefill8 = measure_prefill(cfg, kv8=True)

    import paged_kv_cache_128_amd as pkv
    path = pkv.attention_path(B, cfg.num_q_heads, int(base.max()) + total_steps, eng.key_cache, part)
    # the engine's step: the write runs inside the stream launch (pkv_decode_step)
    # when the stream path applies and the batch has at most 256 rows
    fused = path == "stream" and B <= 256 and not args.separate_write
    kernel_name = ("attn_stream_step_kernel" if fused else
                   {"stream": "attn_stream_kernel", "partition": "attn_split_kernel"}[path])
    traffic, _ = recorded_traffic(kernel_name, cfg.name)
    alg_bytes = float(timed_bytes.mean()) + (new_row_bytes if fused else 0)
    achieved = alg_bytes / split_avg_s / 1e9
    result = {
        "metric": "paged decode attention KV-read GB/s (% of HBM peak) + decode tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: one decode step (append, write, attention) of B={B} sequences, "
                        f"H_q={cfg.num_q_heads} H_kv={cfg.num_kv_heads} D={cfg.head_dim} "
                        f"{cfg.dtype} block_size={cfg.block_size}, pool {cfg.num_blocks} blocks",
            "batch": B,
            "context_lens": f"U[{cfg.len_range[0]}, {cfg.len_range[1]}]" if cfg.len_range else
                            list(map(int, cfg.fixed_lens)),
            "sum_context_first_step": int(base.sum()),
            "partition_tokens": part if part else "library default",
            "placement": cfg.placement,
            "adjacent_logical_neighbours_fraction": round(frag, 4),
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "decode_tokens_per_s": round(tokens_per_s, 1),
        "attention_kv_gbps": round(attn_gbps, 2),
        "attention_cold_us": {"attention_kernel": round(float(np.median(cold[:, 0])) * 1e3, 2),
                              "attention_plus_merge": round(float(np.median(cold[:, 1])) * 1e3, 2),
                              "kv_bytes": cold_bytes,
                              "kv_gbps": round(cold_bytes / (float(np.median(cold[:, 1])) / 1e3) / 1e9, 2),
                              "note": "1 GiB device read before each launch pair"},
        "roofline": {
            "kernel": f"{kernel_name}<{cfg.dtype}, D={cfg.head_dim}, "
                      f"G={cfg.num_q_heads // cfg.num_kv_heads}>",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "mean_launch_us": round(split_avg_s * 1e6, 3),
            "algorithmic_bytes_per_launch": round(alg_bytes),
        },
        "kernel_source_sha256_16": kernel_source_sha(),
        "copy_on_write": block_copy,
        "swap_to_host": swap,
        "fp8_kv": fp8,
        "prefill": prefill,
        "prefill_fp8": prefill8,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, wl, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
