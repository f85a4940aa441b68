"""Build libua.so (the UA kernels and their C ABI) for gfx950 with hipcc.

Usage: ``python -m kv_cache_pruning_amd.build`` (or ``build()`` from Python).
The shared library is written next to this file; objects go to ``_build/``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libua.so")
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = os.environ.get("UA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["api.hip", "workspace.hip", "decode.hip", "compact.hip", "prefill.hip", "qknorm.hip", "backward.hip"]

FLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    f"--offload-arch={ARCH}",
    # Keep hipcc from forming packed fp32 (v_pk_*_f32) instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; install ROCm or set HIPCC")


def _compile(src: str, hipcc: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = [hipcc, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every HIP source and link libua.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc, list(extra_flags)), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
