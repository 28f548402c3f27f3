"""Build libpagedattn.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_186_amd.build          # or __graft_entry__.build()

Objects go to paged_kv_cache_186_amd/_build/, the shared library next to this
file.  Every call recompiles every source.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_NAME = "libpagedattn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

ARCH = "gfx950"
SOURCES = ["pa_decode.hip", "pa_decode_balanced.hip", "pa_decode_balanced_gqa2.hip",
           "pa_decode_balanced_gqa4.hip", "pa_decode_mfma.hip", "pa_mla_heads.hip", "pa_prefill.hip", "pa_prefill_tiles.hip", "pa_cache_ops.hip",
           "pa_api.cpp"]

# Packed-FP32 VALU forms are disabled: plain fp32 code only.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm install required to build libpagedattn)")


def _compile(src: str, build_dir: str, defines) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *[f"-D{d}" for d in defines], "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = False, out_path: str = LIB_PATH, defines=()) -> str:
    """Compile every source and link ``out_path``.  ``defines`` (NAME=VALUE
    strings) override the launch-shape constants of the kernels, for tuning."""
    build_dir = BUILD_DIR if out_path == LIB_PATH else out_path + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, defines), SOURCES))
    tmp = out_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link of {LIB_NAME} failed:\n{res.stderr}")
    os.replace(tmp, out_path)
    if verbose:
        print(f"built {out_path}")
    return out_path


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
