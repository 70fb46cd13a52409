"""Build libfdllm.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

Usage: python -m kv_cache_attention_flash_amd.build [--jobs N] [--asan]
(--asan also builds libfdllm_asan.so, the host code under AddressSanitizer)
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libfdllm.so")
OBJ_DIR = os.path.join(HERE, "_build")
SOURCES = ["flash_cache.hip", "attention.hip", "select.hip", "loop.hip", "lm_head.hip", "fused.hip", "abi.cpp"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Wall", "-Wno-unused-function",
    # packed fp32 instructions stay off (compiler-generated only; never by hand)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(jobs: int = 4, verbose: bool = True) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


ASAN_OUT = os.path.join(HERE, "libfdllm_asan.so")
# Host code only: the device code is built as usual.
ASAN_HOST_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()


def asan_runtime() -> str | None:
    """The compiler's shared AddressSanitizer runtime (to preload), if present."""
    import glob
    llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "lib", "llvm")
    hits = sorted(glob.glob(os.path.join(llvm, "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def build_asan(verbose: bool = True) -> str:
    """libfdllm_asan.so: the C ABI's host code (argument validation, planning,
    dispatch) instrumented with AddressSanitizer, linked with the kernel
    objects of the last build().  Load it with the runtime preloaded
    (LD_PRELOAD=asan_runtime()) and FDL_LIB pointing at it."""
    obj = os.path.join(OBJ_DIR, "abi_asan.cpp.o")
    cmd = [hipcc(), *FLAGS, *ASAN_HOST_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, "abi.cpp"),
           "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on abi.cpp (host ASan):\n{res.stdout}\n{res.stderr}")
    objs = [os.path.join(OBJ_DIR, s + ".o") for s in SOURCES if s != "abi.cpp"] + [obj]
    tmp = ASAN_OUT + ".tmp"
    res = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, ASAN_OUT)
    if verbose:
        print(f"built {ASAN_OUT}")
    return ASAN_OUT


if __name__ == "__main__":
    j = 4
    if "--jobs" in sys.argv:
        j = int(sys.argv[sys.argv.index("--jobs") + 1])
    build(j)
    if "--asan" in sys.argv:
        build_asan()
