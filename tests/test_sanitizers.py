"""Host AddressSanitizer + UndefinedBehaviorSanitizer pass over the CPU oracle and the C-ABI
validation code (CPU only; no device is touched).

The oracle is rebuilt with clang and the host side of csa2_api.cpp with hipcc, both with ASan and
UBSan (host code only: each -fsanitize= follows -Xarch_host, the kernels are the product's own
objects).  A child Python, with the sanitizer runtime preloaded, then runs the oracle pins and the
ABI validation tests against those builds; any report stops it with a failure.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = "/opt/rocm/llvm"
HIPCC = "/opt/rocm/bin/hipcc"
BUILD = os.path.join(ROOT, "compressed_kv_cache_03_amd", "_build")
KERNEL_OBJS = ["pack", "score", "topk", "attend", "index_gemm", "pool"]
TESTS = ["test_abi.py", "test_oracle_codec.py", "test_oracle_score.py", "test_oracle_topk.py",
         "test_oracle_attend.py", "test_oracle_modes.py", "test_oracle_pool.py", "test_oracle_multirow.py"]

CHILD = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle, compressed_kv_cache_03_amd as csa2
oracle._LIB = {oracle_lib!r}
csa2.LIB_PATH = {csa2_lib!r}
import pytest
rc = pytest.main(["-q", "-s", "-x", "-p", "no:cacheprovider", "-m", "not gpu"] + {tests_list!r})
loaded = open("/proc/self/maps").read()
assert {oracle_lib!r} in loaded and {csa2_lib!r} in loaded, "sanitized builds not loaded"
sys.exit(rc)
"""


def _runtime():
    libs = glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))
    return libs[0] if libs else None


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"


def test_oracle_and_abi_validation_under_asan_ubsan(tmp_path):
    rt = _runtime()
    objs = [os.path.join(BUILD, o + ".o") for o in KERNEL_OBJS]
    if rt is None or not os.path.exists(HIPCC) or not all(os.path.exists(o) for o in objs):
        pytest.skip("needs the ROCm clang sanitizer runtime, hipcc and a built library (_build/*.o)")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           "-shared-libasan"]
    oracle_lib = str(tmp_path / "liboracle_san.so")
    _run([os.path.join(LLVM, "bin", "clang"), "-O1", "-g", *san, "-fPIC", "-shared", "-fopenmp",
          "-ffp-contract=off", "-std=gnu11", os.path.join(ROOT, "oracle", "csa2_oracle.c"), "-o", oracle_lib,
          "-lm"])
    host_san = []
    for f in san:
        host_san += ["-Xarch_host", f]
    api_obj = str(tmp_path / "csa2_api_san.o")
    _run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature",
          "-Xclang", "-packed-fp32-ops", *host_san, "-x", "hip", "-c",
          os.path.join(ROOT, "compressed_kv_cache_03_amd", "csrc", "csa2_api.cpp"), "-o", api_obj])
    csa2_lib = str(tmp_path / "libcsa2_san.so")
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", api_obj, *objs, "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-shared-libasan", "-o", csa2_lib])
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               LD_LIBRARY_PATH=os.path.join(LLVM, "lib") + ":" + env.get("LD_LIBRARY_PATH", ""))
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), oracle_lib=oracle_lib, csa2_lib=csa2_lib,
                        tests_list=[os.path.join(ROOT, "tests", t) for t in TESTS])
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=900)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
