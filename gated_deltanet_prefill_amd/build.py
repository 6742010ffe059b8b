"""Build ``libgdn.so`` (HIP kernels for gfx950 + the C ABI) in-tree.

    python -m gated_deltanet_prefill_amd.build

Every source is compiled with hipcc for gfx950 only, in parallel, then
linked into ``gated_deltanet_prefill_amd/libgdn.so``.  Packed-f32 VALU
instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgdn.so")
ROOT = os.path.dirname(HERE)

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]
SOURCES = ["gdn_api.cpp", "gdn_step.hip", "gdn_chunk_f32.hip",
           "gdn_chunk_bf16.hip", "gdn_chunk_f16.hip", "gdn_chunk_wy2_bf16.hip",
           "gdn_chunk_wy2_f16.hip", "gdn_chunk_vg_f32.hip",
           "gdn_chunk_vg_bf16.hip", "gdn_chunk_vg_f16.hip"]
# per-source flags: the pipelined kernel's four-slice form runs about 6%
# faster with the backend's instruction-level-parallelism scheduler, which
# slows the other kernels
EXTRA = {"gdn_chunk_wy2_bf16.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
         "gdn_chunk_wy2_f16.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build_library(jobs: int | None = None) -> str:
    """Compile all sources and link libgdn.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(int(sys.argv[1]) if len(sys.argv) > 1 else None))
