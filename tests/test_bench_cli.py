"""bench.py's command line on the CPU: it measures one GPU only, so any other
--gpus value is refused with exit status 2 and a message, before the library
or the GPU is touched."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "single GPU" in r.stderr and f"--gpus {n}" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_reports_all_cores_and_one_thread():
    """The host baseline runs the oracle on every host core and on one thread
    (tiny workload, host tensors only) and reports both."""
    sys.path.insert(0, ROOT)
    import bench
    from paged_kv_cache_186_amd import workloads as W
    w = W.tiny(0, poison=False)
    lens = w.context_lens_np()
    host = {"k": w.k_pool, "v": w.v_pool, "q": w.q, "tables": w.block_tables_np(), "lens": lens,
            "scale": w.scale, "bs": w.block_size, "fmt": None}
    b = bench.decode_bytes(lens, w.num_heads, w.head_dim, 4, w.block_size)
    r = bench.cpu_baseline(host, b, 0.5)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s"
    assert r["cores"] == len(os.sched_getaffinity(0)) and r["value"] > 0
    assert r["cores_1"]["cores"] == 1 and r["cores_1"]["value"] > 0
