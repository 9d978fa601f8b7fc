"""The C++ block manager (host code) under AddressSanitizer and
UndefinedBehaviorSanitizer: tests/native/manager_replay.cpp and manager.cpp
built with g++, then seeded traces of every manager operation (prefill,
single and batched appends, frees, capacity queries, prefix shares, prefill
chunks, swaps, batch admissions, copy-queue drains), failing ones included,
replayed through the C ABI with the invariants checked after every op
([mini-vLLM BM] "正确性不变量"; [MiniPaged-Qwen] §15).  CPU only."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GXX = shutil.which("g++")


@pytest.fixture(scope="module")
def replay_bin(tmp_path_factory):
    if GXX is None:
        pytest.skip("g++ not found")
    out = str(tmp_path_factory.mktemp("asan") / "manager_replay")
    cmd = [GXX, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "paged_kv_cache_128_amd", "csrc"),
           os.path.join(ROOT, "tests", "native", "manager_replay.cpp"),
           os.path.join(ROOT, "paged_kv_cache_128_amd", "csrc", "manager.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip(f"sanitizer build unavailable: {r.stderr[-400:]}")
    return out


def _line(op):
    kind = op[0]
    if kind == "prefill":
        return f"P {op[1]} {op[2]}"
    if kind == "append":
        return f"A {op[1]}"
    if kind == "append_batch":
        return "B %d %s" % (len(op[1]), " ".join(map(str, op[1])))
    if kind == "free":
        return f"F {op[1]}"
    if kind == "share":
        return f"S {op[1]} {op[2]} {op[3]}"
    return f"C {op[1]}"


def _mixed_trace(seed, n_ops, max_id=20, max_len=60):
    """Every operation kind, with ids and lengths that make some of them fail."""
    rng = np.random.default_rng(seed)
    lines = []
    for _ in range(n_ops):
        u = rng.random()
        sid = int(rng.integers(-1, max_id))
        if u < 0.12:
            lines.append(f"P {sid} {int(rng.integers(-1, max_len))}")
        elif u < 0.25:
            lines.append(f"A {sid}")
        elif u < 0.33:
            k = int(rng.integers(0, 7))
            lines.append("B %d %s" % (k, " ".join(str(int(x)) for x in rng.integers(0, max_id, k))))
        elif u < 0.41:
            lines.append(f"S {int(rng.integers(max_id))} {sid} {int(rng.integers(0, max_len))}")
        elif u < 0.49:
            lines.append(f"T {sid} {int(rng.integers(-1, max_len // 2))}")
        elif u < 0.55:
            lines.append(f"O {sid}")
        elif u < 0.61:
            lines.append(f"I {sid}")
        elif u < 0.71:
            k = int(rng.integers(0, 5))
            pairs = " ".join(f"{int(rng.integers(-1, max_id))} {int(rng.integers(-1, max_len))}" for _ in range(k))
            lines.append(f"M {int(rng.integers(2))} {k} {pairs}")
        elif u < 0.75:
            lines.append("Q")
        elif u < 0.97:
            lines.append(f"F {sid}")
        else:
            lines.append(f"C {int(rng.integers(-1, 4 * max_len))}")
    return lines


def _replay(binary, header, lines):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([binary], input=header + "\n" + "\n".join(lines) + "\n", capture_output=True,
                       text=True, env=env, timeout=120)
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-2000:]
    assert r.returncode == 0, (r.returncode, r.stderr[-2000:])
    return r.stdout


@pytest.mark.parametrize("seed,n_blocks,bs", [(41, 48, 4), (42, 9, 1), (43, 20, 16)])
def test_op_traces_under_sanitizers(replay_bin, seed, n_blocks, bs):
    lines = [_line(op) for op in synth.manager_op_trace(seed, 4000, max_id=30, max_prefill=50)]
    assert "ops" in _replay(replay_bin, f"{n_blocks} {bs} {seed % 2}", lines)


@pytest.mark.parametrize("seed,n_blocks,bs", [(51, 40, 4), (52, 16, 1), (53, 64, 16)])
def test_share_traces_under_sanitizers(replay_bin, seed, n_blocks, bs):
    lines = []
    for op in synth.manager_share_trace(seed, 4000):
        lines.append(_line(op))
        if op[0] in ("append", "append_batch"):
            lines.append("Q")
    assert "ops" in _replay(replay_bin, f"{n_blocks} {bs} 0", lines)


@pytest.mark.parametrize("seed,n_blocks,bs", [(61, 30, 4), (62, 12, 1), (63, 50, 16), (64, 7, 3)])
def test_mixed_traces_with_swaps_and_batches_under_sanitizers(replay_bin, seed, n_blocks, bs):
    assert "ops" in _replay(replay_bin, f"{n_blocks} {bs} {seed % 2}", _mixed_trace(seed, 6000))
