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
# the decode attention kernels are built from this file and the device headers
# it includes; the prefill kernels from pkv_prefill.hip (the C header's comments
# do not enter the hash)
KERNEL_SOURCES = [os.path.join(CSRC, "pkv_kernels.hip"), os.path.join(CSRC, "pkv_internal.h"),
                  os.path.join(CSRC, "pkv_fp8_codec.h")]
PREFILL_SOURCES = [os.path.join(CSRC, "pkv_prefill.hip"), os.path.join(CSRC, "pkv_internal.h")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha(sources=None) -> str:
    h = hashlib.sha256()
    for path in (KERNEL_SOURCES if sources is None else sources):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel_name: str, workload: str, sources=None):
    """HBM bytes per launch from the committed PMC summary
    profiles/<kernel>_<workload>.md, if it was taken from the current kernel
    source."""
    path = os.path.join(ROOT, "profiles", f"{kernel_name}_{workload}.md")
    if not os.path.exists(path):
        return None, None
    text = open(path).read()
    sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    tb = re.search(r"traffic_bytes_per_launch:\s*([0-9.]+)", text)
    if not sha or not tb or sha.group(1) != kernel_source_sha(sources):
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


def _cpu_info():
    """Cores the process may run on, the BLAS threads, and the CPU model."""
    from threadpoolctl import threadpool_info
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [p.get("num_threads") for p in threadpool_info() if p.get("user_api") == "blas"]
    return {"affinity_cores": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count(),
            "blas_threads": blas[0] if blas else None, "cpu_model": model}


def cpu_baseline(cfg, wl, budget_s: float, eng=None, gpu_first=None, reps: int = 3):
    """The CPU oracle, untuned, on the same workload with the process's whole
    affinity set (NumPy's BLAS threads as they come): churned pool state and
    history prefill (untimed), then per sequence the measured append, write
    and float64 gather-then-contiguous attention (timed).  Sequences are
    taken in order until ``budget_s`` of timed work; the whole pass is
    repeated ``reps`` times on a fresh replay and the median pass reported.
    With ``gpu_first`` (the GPU output of the workload's first decode step)
    and ``eng`` the sampled sequences are also compared with the GPU: the
    largest attention difference, and whether every cached row of theirs
    (positions below the first step's length, gathered through both
    sides' tables) is bit for bit the oracle's."""
    import oracle
    from oracle.replay import replay_churn
    import synth
    info = _cpu_info()
    passes = []
    for _ in range(reps):
        nbytes, nseq, secs, state = _cpu_pass(cfg, wl, budget_s, oracle, replay_churn, synth)
        passes.append((nbytes, nseq, secs))       # every pass computes the same state; the last is kept
    passes.sort(key=lambda p: p[0] / p[2])
    nbytes, nseq, secs = passes[len(passes) // 2]
    ref, mgr, kc, vc = state
    nseq = min(nseq, int(np.count_nonzero(~np.isnan(ref[:, 0, 0]))))
    log(f"cpu baseline: {nseq} sequences, {nbytes} KV bytes in {secs:.2f}s (median of {reps}), "
        f"{info['affinity_cores']} cores, BLAS threads {info['blas_threads']}, {info['cpu_model']}")
    res = {"value": nbytes / secs / 1e9, "unit": "GB/s", "cores": info["affinity_cores"], "kind": "oracle",
           "sample": f"first {nseq} of {len(wl.context_lens)} sequences of the same workload "
                     f"(append + write + float64 gather-then-contiguous attention), "
                     f"{nbytes} KV bytes in {secs:.2f} s, median of {reps} passes",
           "decode_tokens_per_s": nseq / secs, **info}
    if gpu_first is not None and eng is not None:
        import torch
        err = float(np.abs(gpu_first[:nseq] - ref[:nseq]).max())
        exact = True
        bs, D, H = cfg.block_size, cfg.head_dim, cfg.num_kv_heads
        for b in range(nseq):
            L = int(mgr.context_len(b))
            nb = -(-L // bs)
            tab = eng.tables[b, :nb].long()
            for half, oc in ((0, kc), (1, vc)):
                g = eng.pool[tab, half].contiguous().cpu()                      # [nb, H, bs, D]
                u = np.uint16 if g.element_size() == 2 else np.uint32
                g = (g.view(torch.int16) if g.element_size() == 2 else g.view(torch.int32)).numpy().view(u)
                g = g.transpose(1, 0, 2, 3).reshape(H, nb * bs, D)[:, :L]
                o = np.ascontiguousarray(oracle.gather_logical(oc, mgr.block_table(b), L)).view(u)
                exact &= bool(np.array_equal(g, o))
        res["parity_sample"] = {"sequences": nseq, "max_abs_err": err, "tolerance": 1e-5 if cfg.dtype == "f32" else 2e-3,
                                "cached_rows_bit_exact": exact}
        log(f"cpu baseline parity: {nseq} sequences, max abs err {err:.3e}, cached rows bit-exact {exact}")
    return res


def _cpu_pass(cfg, wl, budget_s, oracle, replay_churn, synth):
    mgr = oracle.BlockManager(cfg.num_blocks, cfg.block_size, wl.initial_free_order)
    replay_churn(mgr, wl.churn)
    fill = synth.poison_array((), cfg.dtype)
    kc, vc = oracle.new_pool(cfg.num_blocks, cfg.num_kv_heads, cfg.block_size, cfg.head_dim, fill)
    elem = synth.ELEM_BYTES[cfg.dtype]
    B = len(wl.context_lens)
    ref = np.full((B, cfg.num_q_heads, cfg.head_dim), np.nan)
    done_bytes = 0
    done_seqs = 0
    elapsed = 0.0
    for b in range(B):
        slots = mgr.allocate_for_prefill(b, int(wl.context_lens[b]) - 1)
        oracle.write_kv(wl.hist_k[b], wl.hist_v[b], slots, kc, vc, cfg.block_size)
        t0 = time.perf_counter()
        step = [mgr.append_slot_for_decode(b)]
        oracle.write_kv(wl.new_k[b:b + 1], wl.new_v[b:b + 1], step, kc, vc, cfg.block_size)
        L = mgr.context_len(b)
        table = np.array([mgr.block_table(b)], dtype=np.int32)
        ref[b] = oracle.decode_attention(wl.q[b:b + 1], kc, vc, table, [L], cfg.scale, cfg.dtype)[0]
        elapsed += time.perf_counter() - t0
        done_bytes += L * cfg.num_kv_heads * 2 * cfg.head_dim * elem
        done_seqs += 1
        if elapsed >= budget_s:
            break
    return done_bytes, done_seqs, elapsed, (ref, mgr, kc, vc)


def _device_sleep(cycles: int = 200_000):
    """Keep the device busy for a moment (torch's spin kernel), so that a
    launch queued right after an event is already waiting when the event
    completes; without it the timing also holds the host's launch time."""
    import torch
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(cycles)


def measure_block_copy(eng, pairs: int = 256, iters: int = 50):
    """Copy-on-write block copies (pkv_copy_blocks) on the workload's pool:
    ``pairs`` allocated blocks copied into free ones per launch, each launch
    timed between two HIP events (median of ``iters``).  Algorithmic bytes:
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
    # each launch between two events queued behind a short device-side sleep,
    # so that the launch is queued before the first event completes (back to
    # back, the host's marshalling of the 256 pairs would set the pace)
    times = []
    for _ in range(iters):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        _device_sleep()
        e0.record()
        pkv.copy_blocks(src, dst, eng.key_cache, eng.value_cache)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    us = float(np.median(times))
    moved = 2 * n * block_bytes
    gbps = moved / (us * 1e-6) / 1e9
    log(f"block copy: {n} blocks of {block_bytes} B in {us:.2f} us per launch ({gbps:.0f} GB/s)")
    return {"kernel": "block_copy_kernel", "blocks_per_launch": n, "block_bytes": block_bytes,
            "algorithmic_bytes_per_launch": moved, "mean_launch_us": round(us, 3),
            "achieved_gbps": round(gbps, 2), "peak_gbps": HBM_PEAK_GBPS,
            "frac": round(gbps / HBM_PEAK_GBPS, 4)}


def measure_write(eng, k, v, iters: int = 50):
    """The step's write on its own: the last timed step's rows written again
    at its slots (the same values, so the cache is unchanged), by
    pkv_decode_write (host slots and lengths in the kernel arguments, table
    and lengths published) and by paged_kv_write (a device slot mapping).
    Each launch is timed alone between two HIP events queued behind a short
    device-side sleep, so that the launch is already queued when the first
    event completes (timed from an idle device, or back to back, the host's
    argument marshalling would set the pace instead); the median of
    ``iters``.  Algorithmic bytes: the new
    K and V rows read once and written once."""
    import torch
    import paged_kv_cache_128_amd as pkv
    n = k.shape[0]
    slots, lens = eng.slots[:n].copy(), eng.lens[:n].copy()
    d_slots = torch.from_numpy(slots).to("cuda")
    moved = 2 * 2 * k.numel() * k.element_size()
    res = {"rows": n, "algorithmic_bytes_per_launch": moved}
    for name, launch in (
            ("decode_write_kernel (pkv_decode_write)",
             lambda: pkv.decode_write(k, v, slots, lens, eng.key_cache, eng.value_cache,
                                      block_tables=eng.tables, lens_out=eng.d_lens)),
            ("kv_write_kernel (paged_kv_write)",
             lambda: pkv.paged_kv_write(k, v, d_slots, eng.key_cache, eng.value_cache))):
        for _ in range(5):
            launch()
        torch.cuda.synchronize()
        times = []
        for _ in range(iters):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            _device_sleep()
            e0.record()
            launch()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3)
        us = float(np.median(times))
        res[name] = round(us, 3)
        log(f"write: {name} {n} rows in {us:.2f} us per launch (median of {iters}, one launch per event pair)")
    res["note"] = ("launch-bound (a few hundred KB at most); the decode step's default path writes the rows "
                   "inside the attention launch instead")
    return res


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
            "matrix_flops_issued_per_launch": flops * 3 // 2,
            "note": "useful FLOPs: row i sees i + 1 keys; the matrix cores also run P.V's remainder pass "
                    "(1.5x the useful products)",
            "traffic": None if kv8 else recorded_traffic("prefill_kernel", f"{cfg.name}_{seqs}x{prompt}",
                                                          PREFILL_SOURCES)[0],
            "kernel_source_sha256_16": kernel_source_sha(PREFILL_SOURCES),
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
    time, and the refill time separately.  Unless --no-cpu-baseline, the
    output of every tenth step and the last is copied aside after that
    step's refills (outside both event pairs, inside the wall clock), and
    the oracle replays the trace afterwards (serving_cpu_baseline)."""
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
    # the pool starts as the oracle's does (every element the poison value), so the two compare whole
    eng = PagedKVEngine(cfg.num_blocks, H, cfg.block_size, D, tdtype, B, width, None, num_q_heads=cfg.num_q_heads,
                        fill_bits=synth.POISON_BITS[cfg.dtype])
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
    sampled = set(range(0, len(steps), 10)) | {len(steps) - 1}     # steps the oracle compares
    step_slots, kept = [], {}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, ((k, v, q, refills), ev) in enumerate(zip(steps, evs)):
        ev[0].record()
        eng.decode_step(row_ids, k, v, q, cfg.scale, out=out)
        kv_bytes += int(eng.lens[:B].astype(np.int64).sum()) * H * 2 * D * elem
        ev[1].record()
        step_slots.append(eng.slots[:B].copy())
        rows, new_ids, plens, rk, rv = refills
        if rows:
            for row, new_id in zip(rows, new_ids):
                eng.free(int(row_ids[row]))
                row_ids[row] = new_id
            eng.prefill_many(new_ids, rows, plens, rk, rv)
            n_refill += len(rows)
            refill_tokens += int(sum(plens))
        ev[2].record()
        if i in sampled and not args.no_cpu_baseline:
            kept[i] = out.clone()          # outside both event pairs; the refills do not touch out
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
        "cpu_baseline": None if args.no_cpu_baseline else serving_cpu_baseline(cfg, eng, step_slots, kept, width),
    }), flush=True)


def serving_cpu_baseline(cfg, eng, step_slots, kept, width):
    """The CPU oracle on the serving trace, untuned, with the process's whole
    affinity set: the trace regenerated from its seed and replayed on the
    oracle (oracle.replay.serving_replay: the manager's appends, writes and
    refills on every step), with the float64 attention on the steps the GPU
    run kept (every tenth and the last).  Reported as KV GB/s and decode
    tokens/s over those attentions (the replay's own time beside them).
    Compared with the GPU run: the slots of every step, the attention of
    every row at the sampled steps, and at the end the free list and the
    whole pool bit for bit."""
    import torch
    import oracle
    import synth
    from oracle.replay import serving_replay
    info = _cpu_info()
    tr = synth.serving_trace(cfg)
    B, H, D, elem = cfg.batch, cfg.num_kv_heads, cfg.head_dim, synth.ELEM_BYTES[cfg.dtype]
    t0 = time.perf_counter()
    t_attn = 0.0
    kv = 0
    err = 0.0
    slots_equal = True
    mgr = kc = vc = None
    for st, mgr, kc, vc, rows, slots in serving_replay(tr):
        slots_equal &= bool(np.array_equal(np.asarray(slots, np.int64), step_slots[st.step]))
        if st.step in kept:
            t1 = time.perf_counter()
            lens = mgr.context_lens(list(rows))
            ref = oracle.decode_attention(st.q, kc, vc, mgr.block_tables(list(rows), width, -1), lens,
                                          cfg.scale, cfg.dtype)
            t_attn += time.perf_counter() - t1
            kv += int(np.asarray(lens, np.int64).sum()) * H * 2 * D * elem
            err = max(err, float(np.abs(kept[st.step].double().cpu().numpy() - ref).max()))
    t_replay = time.perf_counter() - t0 - t_attn
    free_equal = eng.manager.free_list() == mgr.free
    pool_exact = True
    for half, oc in ((0, kc), (1, vc)):
        g = eng.pool[:, half].contiguous().cpu()
        u = np.uint16 if g.element_size() == 2 else np.uint32
        g = (g.view(torch.int16) if g.element_size() == 2 else g.view(torch.int32)).numpy().view(u)
        pool_exact &= bool(np.array_equal(g, oc.view(u)))
        del g
    n = len(kept)
    log(f"cpu baseline (serving): attention on {n} steps, {kv} KV bytes in {t_attn:.1f}s; replay (appends, "
        f"writes, refills) {t_replay:.1f}s; max abs err {err:.3e}, slots equal {slots_equal}, free list equal "
        f"{free_equal}, pool bit-exact {pool_exact}")
    return {"value": kv / t_attn / 1e9, "unit": "GB/s", "cores": info["affinity_cores"], "kind": "oracle",
            "sample": f"the serving trace replayed on the oracle over all {len(step_slots)} steps (appends, writes "
                      f"and refills: {t_replay:.1f} s, not in value), float64 attention of all {B} rows on the {n} "
                      f"steps the GPU run kept, every tenth and the last ({t_attn:.1f} s): value and tokens/s "
                      f"over those attentions",
            "decode_tokens_per_s": B * n / t_attn, "replay_s": t_replay, **info,
            "parity": {"steps_compared": n, "rows_per_step": B, "max_abs_err": err, "tolerance": 2e-3,
                       "slots_equal_every_step": slots_equal, "free_list_equal": free_equal,
                       "pool_bit_exact_at_end": pool_exact}}


def measure_fp8(cfg, wl, args, ring, base, width, tokens_per_s_16):
    """The same workload with an 8-bit KV pool (E4M3 codes + one scale byte
    per row; the history quantised by the prefill write), under the
    headline's protocol: decode steps of append, quantising step write and
    8-bit attention + merge, each timed step preceded by a 1 GiB device read
    (median with p10/p90 of two-event steps), the kernel's own time from the
    three-event steps.  Reported beside the 16-bit headline: KV bytes
    actually read (codes and scale bytes) per second, decode tokens/s, and
    the 8-bit step kernel's roofline."""
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
    fused = not args.separate_write

    def kv8(step):
        return int((base + step).sum()) * row_bytes

    for s_ in range(args.warmup):
        k, v, q = ring[s_ % len(ring)]
        eng.decode_step(ids, k, v, q, cfg.scale, out=out, fused=fused)
    flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    fl = _timed_steps(eng, ring, ids, out, cfg, args.warmup, args.steps, fused, flush)
    del flush
    step_bytes = np.array([kv8(args.warmup + i) for i in range(args.steps)], dtype=np.float64)
    t_med, t10, t90 = (float(np.percentile(fl["step_us"], x)) for x in (50, 10, 90))
    fl_bytes = float(step_bytes[fl["two_idx"]].mean())
    # the fused launch also writes the B new rows (codes and scale bytes)
    alg = float(step_bytes[fl["three_idx"]].mean()) + (B * row_bytes if fused else 0)
    kern_us = float(fl["kern_us"].mean())
    achieved = alg / (kern_us * 1e-6) / 1e9
    kname = "attn_stream8_step_kernel" if fused else "attn_stream8_kernel"
    tps = B / (t_med * 1e-6)
    log(f"fp8 KV flushed: {t_med:.1f} us median step (p10 {t10:.1f}, p90 {t90:.1f}), step kernel {kern_us:.1f} us, "
        f"merge {fl['merge_us'].mean():.1f} us, KV {fl_bytes / 1e6:.1f} MB/step")
    return {
        "kv_dtype": "fp8_e4m3 codes + e8m0 row scales",
        "value": round(fl_bytes / (t_med * 1e-6) / 1e9, 2),
        "unit": "GB/s",
        "ms_per_step": round(t_med / 1e3, 4),
        "step_us_p10": round(t10, 2), "step_us_p90": round(t90, 2),
        "kv_bytes_per_step": round(fl_bytes),
        "decode_tokens_per_s": round(tps, 1),
        "tokens_per_s_vs_16bit": round(tps / tokens_per_s_16, 3),
        "roofline": {
            "kernel": f"{kname}<{cfg.dtype} q, D={cfg.head_dim}, "
                      f"G={cfg.num_q_heads // cfg.num_kv_heads}>",
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": recorded_traffic(kname, cfg.name)[0],
            "mean_launch_us": round(kern_us, 3),
            "launches_timed": len(fl["kern_us"]),
            "algorithmic_bytes_per_launch": round(alg),
            "note": "launch time from events around the kernel in the flushed steps",
        },
    }


def _timed_steps(eng, ring, ids, out, cfg, s0, n, fused, flush, event_every=5):
    """n decode steps of the engine's rows, step s0 + i taking ring tensors
    (s0 + i) mod len(ring).  With ``flush`` (a device tensor) a read of it
    precedes every step outside its events; even steps then carry two events
    (around the whole step) and odd steps three (before the first launch,
    between the two launches, after the second).  Without, the steps run
    back to back and every ``event_every``-th carries three events.  Returns
    the wall time and the event times in microseconds; ``two_idx`` names the
    steps whose whole span was timed (the two-event steps, or with none the
    three-event ones)."""
    import torch
    evs = {}
    for i in range(n):
        if flush is not None:
            # a single step carries three events (its whole span is then e0 -> e2)
            evs[i] = [torch.cuda.Event(enable_timing=True) for _ in range(2 if i % 2 == 0 and n > 1 else 3)]
        elif i % max(1, event_every) == 0:
            evs[i] = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    if torch.distributed.is_available() and torch.distributed.is_initialized():
        torch.distributed.barrier()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        if flush is not None:
            flush.sum()
        k, v, q = ring[(s0 + i) % len(ring)]
        eng.decode_step(ids, k, v, q, cfg.scale, out=out, events=evs.get(i), fused=fused)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    two = sorted(i for i in evs if len(evs[i]) == 2)
    three = sorted(i for i in evs if len(evs[i]) == 3)
    whole = [(i, evs[i][0].elapsed_time(evs[i][1])) for i in two] or \
            [(i, evs[i][0].elapsed_time(evs[i][2])) for i in three]
    return {"wall_s": wall, "two_idx": [i for i, _ in whole], "three_idx": three,
            "step_us": np.array([ms * 1e3 for _, ms in whole]),
            "kern_us": np.array([evs[i][0].elapsed_time(evs[i][1]) * 1e3 for i in three]),
            "merge_us": np.array([evs[i][1].elapsed_time(evs[i][2]) * 1e3 for i in three])}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warm-steps", type=int, default=100,
                    help="back-to-back steps without a flush after the timed (flushed) ones")
    ap.add_argument("--config", default="qwen2_7b_b64")
    ap.add_argument("--partition-tokens", type=int, default=-1,
                    help="split-K partition length (-1: the workload's own, else library default)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    total_steps = args.warmup + args.steps + args.warm_steps
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
    # unused slots in the sequences' last blocks, and the free list, after the history prefill
    tail_waste = int(sum(int((r >= 0).sum()) for r in tabs) * cfg.block_size - (wl.context_lens - 1).sum())
    free_blocks = eng.manager.num_free_blocks()
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
    fused = not args.separate_write
    first_out = None
    for s in range(args.warmup):
        k, v, q = ring[s % len(ring)]
        eng.decode_step(ids, k, v, q, cfg.scale, out=out, fused=fused)
        if s == 0:
            first_out = out.clone()          # the workload's own first step, for the parity sample
    torch.cuda.synchronize()

    # Headline: flushed steps.  Before each timed step a 1 GiB device read
    # (outside its events) evicts the 256 MB Infinity Cache and the L2s; a
    # read leaves no dirty lines to be written back during the step.  Even
    # steps carry two events around the whole step (the headline times),
    # odd steps three (before the step kernel, between it and the merge,
    # after the merge) for the kernel's own duration.
    flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    fl = _timed_steps(eng, ring, ids, out, cfg, args.warmup, args.steps, fused, flush)
    s_warm = args.warmup + args.steps
    # Warm steps: back to back, no flush (kernel events on every 5th step).
    wm = _timed_steps(eng, ring, ids, out, cfg, s_warm, args.warm_steps, fused, None, args.event_every)
    del flush
    step_bytes = np.array([kv_bytes(args.warmup + i) for i in range(args.steps)], dtype=np.float64)
    fl_bytes = float(step_bytes[fl["two_idx"]].mean())
    t_med, t10, t90 = (float(np.percentile(fl["step_us"], x)) for x in (50, 10, 90))
    value = fl_bytes / (t_med * 1e-6) / 1e9
    warm_bytes = np.array([kv_bytes(s_warm + i) for i in range(args.warm_steps)], dtype=np.float64)
    warm_value = float(warm_bytes.sum()) / wm["wall_s"] / 1e9 if args.warm_steps else None
    log(f"flushed {args.steps} steps: {t_med:.1f} us median (p10 {t10:.1f}, p90 {t90:.1f}), step kernel "
        f"{fl['kern_us'].mean():.1f} us, merge {fl['merge_us'].mean():.1f} us (three-event steps); "
        f"KV {fl_bytes / 1e6:.1f} MB/step -> {value:.0f} GB/s")
    if args.warm_steps:
        log(f"warm {args.warm_steps} steps: {wm['wall_s'] * 1e6 / args.warm_steps:.1f} us/step wall, step kernel "
            f"{wm['kern_us'].mean():.1f} us, merge {wm['merge_us'].mean():.1f} us")
    k_last, v_last, _ = ring[(total_steps - 1) % len(ring)]
    write = measure_write(eng, k_last, v_last)
    block_copy = measure_block_copy(eng)
    swap = measure_swap(eng)
    fp8 = None
    if not args.no_fp8 and cfg.dtype in ("bf16", "f16") and cfg.head_dim == 128:
        fp8 = measure_fp8(cfg, wl, args, ring, base, width, B / (t_med * 1e-6))
    prefill = prefill8 = None
    if not args.no_prefill and cfg.dtype in ("bf16", "f16") and cfg.head_dim == 128:
        prefill = measure_prefill(cfg)
        if cfg.dtype == "bf16" and not args.no_fp8:
            prefill8 = measure_prefill(cfg, kv8=True)

    import paged_kv_cache_128_amd as pkv
    path = pkv.attention_path(B, cfg.num_q_heads, int(base.max()) + total_steps, eng.key_cache, part)
    # the engine's step: the write runs inside the stream launch (pkv_decode_step)
    # when the stream path applies and the batch has at most 256 rows
    fused_launch = path == "stream" and B <= 256 and fused
    kernel_name = ("attn_stream_step_kernel" if fused_launch else
                   {"stream": "attn_stream_kernel", "partition": "attn_split_kernel"}[path])
    traffic, _ = recorded_traffic(kernel_name, cfg.name)
    # the first launch of a step also writes the step's new K/V rows when fused
    new_row_bytes = B * cfg.num_kv_heads * 2 * cfg.head_dim * elem
    kern_bytes = float(step_bytes[fl["three_idx"]].mean()) + (new_row_bytes if fused_launch else 0)
    kern_us = float(fl["kern_us"].mean())
    achieved = kern_bytes / (kern_us * 1e-6) / 1e9
    result = {
        "metric": "paged decode attention KV-read GB/s (% of HBM peak) + decode tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_med / 1e3, 4),
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
            "seed": cfg.seed,
            "context_lens": f"U[{cfg.len_range[0]}, {cfg.len_range[1]}]" if cfg.len_range else
                            list(map(int, cfg.fixed_lens)),
            "sum_context_first_step": int(base.sum()),
            "partition_tokens": part if part else "library default",
            "attention_path": path,
            "placement": cfg.placement,
            "adjacent_logical_neighbours_fraction": round(frag, 4),
            "internal_fragmentation_tokens": tail_waste,
            "free_blocks_after_prefill": free_blocks,
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "decode_tokens_per_s": round(B / (t_med * 1e-6), 1),
        "flushed": {
            "what": "each timed step preceded, outside its events, by a 1 GiB device read; step = write and "
                    "attention (one launch when fused) + merge, timed with two events around it",
            "step_us_median": round(t_med, 2), "step_us_p10": round(t10, 2), "step_us_p90": round(t90, 2),
            "kv_bytes_per_step": round(fl_bytes),
            "gbps_at_p10_p90": [round(fl_bytes / (t10 * 1e-6) / 1e9, 1), round(fl_bytes / (t90 * 1e-6) / 1e9, 1)],
            "step_kernel_us_mean": round(kern_us, 2),
            "merge_us_mean": round(float(fl["merge_us"].mean()), 2),
            "steps_timed": len(fl["step_us"]),
        },
        "warm": None if not args.warm_steps else {
            "what": "back-to-back steps without a flush, host append included (wall clock)",
            "steps": args.warm_steps,
            "ms_per_step": round(wm["wall_s"] * 1e3 / args.warm_steps, 4),
            "value": round(warm_value, 2), "unit": "GB/s",
            "pct_hbm_peak": round(100.0 * warm_value / HBM_PEAK_GBPS, 2),
            "decode_tokens_per_s": round(B * args.warm_steps / wm["wall_s"], 1),
            "step_kernel_us_mean": round(float(wm["kern_us"].mean()), 2),
            "merge_us_mean": round(float(wm["merge_us"].mean()), 2),
        },
        "roofline": {
            "kernel": f"{kernel_name}<{cfg.dtype}, D={cfg.head_dim}, "
                      f"G={cfg.num_q_heads // cfg.num_kv_heads}>",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "mean_launch_us": round(kern_us, 3),
            "launches_timed": len(fl["kern_us"]),
            "algorithmic_bytes_per_launch": round(kern_bytes),
            "note": "launch time from events around the kernel in the flushed steps",
        },
        "kernel_source_sha256_16": kernel_source_sha(),
        "write": write,
        "copy_on_write": block_copy,
        "swap_to_host": swap,
        "fp8_kv": fp8,
        "prefill": prefill,
        "prefill_fp8": prefill8,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, wl, args.cpu_seconds, eng, first_out.double().cpu().numpy())
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
