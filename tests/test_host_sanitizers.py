"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The host-only sources (error state, packers, quantiser, KV page pool, step
validation and orchestration) are rebuilt with clang's -fsanitize=address,undefined
and the CPU tests that drive them through the C ABI run again against that
build, with the sanitizer runtime preloaded into the Python process. Any
out-of-bounds access, use after free or undefined behaviour aborts the run.
CPU only: no device code is sanitized and no GPU is touched.
"""
import os
import subprocess
import sys

import pytest

from w4a16_paged_kv_amd import build as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_TESTS = ["tests/test_abi.py", "tests/test_pack.py", "tests/test_kvpool.py", "tests/test_validate.py",
              "tests/test_quantize.py"]


def test_host_code_under_address_and_undefined_sanitizers():
    rt = b.asan_runtime()
    if rt is None:
        pytest.skip("clang's sanitizer runtime is not installed")
    lib = b.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=rt, W4A16_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", *HOST_TESTS, "-q", "-s", "-m", "not gpu",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in r.stdout and "Sanitizer" not in out, out[-4000:]
    print(r.stdout.strip().splitlines()[-1])
