"""Build libcsa2.so (HIP kernels for gfx950 + the C-ABI host code) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libcsa2.so")
ARCH = os.environ.get("CSA2_OFFLOAD_ARCH", "gfx950")

SOURCES = ["pack.hip", "score.hip", "topk.hip", "attend.hip", "index_gemm.hip", "pool.hip", "csa2_api.cpp"]

# -packed-fp32-ops: keep the compiler from forming packed fp32 instructions.
# -amdgpu-mfma-vgpr-form: MFMA accumulators in ordinary VGPRs, so the softmax
#   arithmetic on them needs no accumulator-register copies.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form",
          "-Wno-unused-command-line-argument"]


# Per-file flags.  index_gemm.hip software-pipelines its MFMAs ahead of an
# epilogue with branches; machine sinking would move them back below it.
EXTRA = {"index_gemm.hip": ["-mllvm", "-disable-machine-sink"]}


def _hipcc() -> str:
    for cand in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.isabs(cand) and os.path.exists(cand):
            return cand
    return "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libcsa2.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
