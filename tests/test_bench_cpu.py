"""Host-side behaviour of bench.py that needs no GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    """The library has no multi-GPU path: --gpus above 1 exits with status
    2 and says so, before touching a device."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_kernel_source_hash_covers_the_decode_sources():
    """The hash that ties a profile's traffic figure to the kernels changes
    with each decode source file and with nothing else."""
    sys.path.insert(0, ROOT)
    import bench
    base = bench.kernel_source_sha()
    assert len(base) == 16 and int(base, 16) >= 0
    assert bench.kernel_source_sha(bench.KERNEL_SOURCES) == base
    assert bench.kernel_source_sha(bench.PREFILL_SOURCES) != base
