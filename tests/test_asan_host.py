"""The C ABI's host code (argument validation, workspace sizing, planning,
dispatch) under AddressSanitizer: the host-validation tests of
tests/test_abi_cpu.py run in a subprocess against libfdllm_asan.so with the
compiler's shared ASan runtime preloaded.  Skipped when that library has not
been built (`python -m kv_cache_attention_flash_amd.build --asan`, which
__graft_entry__.build() also runs)."""

import os
import subprocess
import sys

import pytest

from kv_cache_attention_flash_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_validation_under_asan():
    if not os.path.exists(B.ASAN_OUT):
        pytest.skip("libfdllm_asan.so not built")
    rt = B.asan_runtime()
    if rt is None:
        pytest.skip("no shared AddressSanitizer runtime next to the compiler")
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               FDL_LIB=B.ASAN_OUT)
    # the runtime is live in the child and the sanitised library is the one loaded
    probe = ("import ctypes; ctypes.CDLL(None).__asan_init; "
             "from kv_cache_attention_flash_amd import _lib; "
             "assert _lib.load()._name.endswith('libfdllm_asan.so')")
    subprocess.run([sys.executable, "-c", probe], env=env, check=True, timeout=300, cwd=ROOT)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"),
                        "-q", "-p", "no:cacheprovider"], env=env, capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
