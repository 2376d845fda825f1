"""Builds libw4a16.so for gfx950 in-tree with hipcc (one object per source,
compiled in parallel, then linked).

    python -m w4a16_paged_kv_amd.build             # the library
    python -m w4a16_paged_kv_amd.build sanitized   # + host code under ASan/UBSan

The sanitized variant (_build/asan/libw4a16.so) compiles the host-only C++
sources (error state, packers, quantiser, KV pool, validation, the step
orchestration) with clang's address and undefined-behaviour sanitizers and
links them with the ordinary HIP objects; the CPU tests run against it with
the sanitizer runtime preloaded (tests/test_host_sanitizers.py).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libw4a16.so")
SOURCES = ["host.cpp", "model.cpp", "gemv.hip", "attention.hip", "sample.hip", "prefill.hip", "w4a8.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
          "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
# packed fp32 vector instructions stay disabled in device code
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    path = os.path.join(CSRC, src)
    lang = ["-x", "hip"] + DEVICE if src.endswith(".hip") else ["-D__HIP_PLATFORM_AMD__"]
    cmd = [HIPCC] + lang + COMMON + ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


# ---------------------------------------------------------------- sanitized
CLANG = os.environ.get("W4_CLANGXX", "/opt/rocm/llvm/bin/clang++")
ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libw4a16.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def asan_runtime():
    """Path of clang's shared address-sanitizer runtime, or None."""
    import glob
    rt = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(CLANG)), "lib", "clang", "*", "lib",
                                       "linux", "libclang_rt.asan-x86_64.so")))
    return rt[-1] if rt and os.path.exists(CLANG) else None


def build_sanitized(verbose: bool = False) -> str:
    """Host sources with sanitizers (plain C++, no device code), HIP objects as
    for the library (compiled if missing)."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    objs = []
    for src in SOURCES:
        if src.endswith(".hip"):
            obj = os.path.join(BUILD, src + ".o")
            objs.append(obj if os.path.exists(obj) else _compile(src))
            continue
        obj = os.path.join(ASAN_DIR, src + ".o")
        cmd = [CLANG, "-x", "c++", "-std=c++17", "-O1", "-g", "-fPIC", "-D__HIP_PLATFORM_AMD__",
               "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC] + SAN_FLAGS + \
              ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
        objs.append(obj)
    cmd = [CLANG, "-shared", "-shared-libsan", "-o", ASAN_LIB] + SAN_FLAGS + objs + \
          ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    if verbose:
        print("built", ASAN_LIB)
    return ASAN_LIB


if __name__ == "__main__":
    build(verbose=True)
    if sys.argv[1:] == ["sanitized"]:
        build_sanitized(verbose=True)
