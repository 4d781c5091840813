"""Build libpagedkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_235_amd._build

Every source is compiled on each call (one hipcc per file, in parallel) and
linked into ``paged_kv_cache_235_amd/libpagedkv.so``; the measurement kernels
of ``include/pkv_probe.h`` go into ``libpkvprobe.so`` beside it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libpagedkv.so")
PROBE_LIB_PATH = os.path.join(PKG, "libpkvprobe.so")
ARCH = "gfx950"

SOURCES = ["pkv_api.cpp", "block_allocator.cpp", "kv_write.hip", "decode.hip", "prefill.hip",
           "block_ops.hip"]
PROBE_SOURCES = ["peak_probe.hip"]

# -packed-fp32-ops: keep the compiler from forming packed fp32 instructions.
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpagedkv)")


# per-file flags.  decode.hip: its MFMA accumulators (INT8 P.V) in ordinary
# VGPRs rather than accumulation registers, which keeps the INT8 decode kernel
# at three waves per SIMD (164 registers at 4 heads per item instead of 200);
# and no atomic optimizer: its one atomic with a result (a work-counter claim
# by a single lane) would become a wave scan that reads the result at once,
# which makes the wave wait there for every load it has in flight.
FILE_FLAGS = {"decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs: list, path: str) -> None:
    tmp = path + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, path)


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    jobs = jobs or min(len(srcs), os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB_PATH)
    _link(objs[len(SOURCES):], PROBE_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {PROBE_LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
