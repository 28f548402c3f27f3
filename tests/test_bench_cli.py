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
