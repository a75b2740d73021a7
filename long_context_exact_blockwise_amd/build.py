"""Build libringattn.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Every source is compiled with hipcc for gfx950 only; packed-FP32 instructions
are disabled for all device code (-Xclang -target-feature -Xclang
-packed-fp32-ops).  Objects go to _build/ next to this file; the shared
library is written next to this file, where the binding loads it.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libringattn.so")
BUILD = os.path.join(HERE, "_build")
SOURCES = ["ringattn_api.hip", "attn_bf16.hip", "attn_bwd.hip", "attn_f32.hip", "ffn_bf16.hip", "probe.hip", "state.hip"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libringattn.so)")


FLAGS = [
    "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Per-source flags: the forward kernel and the feedforward GEMM are scheduled
# with LLVM's iterative ILP strategy (measured 1.2% and 1.9% faster; the
# backward kernels measured 10% slower with it and keep the default).
_ILP = ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]
SOURCE_FLAGS = {"attn_bf16.hip": _ILP, "ffn_bf16.hip": _ILP}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + FLAGS + SOURCE_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "-shared", "--offload-arch=gfx950", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
