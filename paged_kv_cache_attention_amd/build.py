"""Builds libpkv.so (and the seeded-input fill library) for gfx950 with hipcc.

Run ``python paged_kv_cache_attention_amd/build.py`` (by path: importing the
package would load the library being rebuilt); both libraries are written
in-tree next to their sources.

The device sources (kernels.hip, prefill.hip, scratch.hip) and the host
runtime (runtime.cpp) compile to separate objects under ``_build/``, in
parallel, and link into libpkv.so.  The same kernel objects also link with a copy of the runtime
built with AddressSanitizer and UndefinedBehaviorSanitizer on the host side
only (``libpkv_san.so``), for the CPU tests of the allocator and the token
transaction; device code is never built with a sanitizer.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.environ.get("HIPCC", os.path.join(ROCM, "bin", "hipcc"))
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
ARCH = "gfx950"
BUILD_DIR = os.path.join(HERE, "_build")

# Packed FP32 instructions are disabled for all device code.
DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wall", "-Wno-unused-result"]
INCLUDES = ["-I", os.path.join(ROOT, "include")]
# Host-only sanitizer build of the runtime: plain clang++ on a C++ source
# (no device code on this line).
SAN_FLAGS = ["-std=c++17", "-O1", "-g", "-fPIC", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include")]

LIBPKV = os.path.join(HERE, "libpkv.so")
LIBPKV_SAN = os.path.join(HERE, "libpkv_san.so")
LIBSYNTH = os.path.join(ROOT, "synth", "libsynth.so")
KERNEL_SOURCES = ("kernels.hip", "prefill.hip", "scratch.hip")


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def _obj(name: str, suffix: str = "") -> str:
    return os.path.join(BUILD_DIR, os.path.splitext(name)[0] + suffix + ".o")


def _compile_device(name: str) -> str:
    out = _obj(name)
    _run([HIPCC, *DEVICE_FLAGS, *INCLUDES, "-c", os.path.join(HERE, "csrc", name), "-o", out])
    return out


def _compile_runtime() -> str:
    out = _obj("runtime.cpp")
    _run([HIPCC, *DEVICE_FLAGS, *INCLUDES, "-c", os.path.join(HERE, "csrc", "runtime.cpp"),
          "-o", out])
    return out


def _compile_runtime_sanitized() -> str:
    out = _obj("runtime.cpp", "_san")
    _run([CLANGXX, *SAN_FLAGS, *INCLUDES, "-c", os.path.join(HERE, "csrc", "runtime.cpp"),
          "-o", out])
    return out


def _link(objs, target: str) -> str:
    tmp = target + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, target)
    return target


def build_libpkv(sanitized: bool = True) -> str:
    """Compiles the sources in parallel and links libpkv.so (and, with
    sanitized=True, libpkv_san.so from the same device objects)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        kern = [ex.submit(_compile_device, n) for n in KERNEL_SOURCES]
        rt = ex.submit(_compile_runtime)
        san = ex.submit(_compile_runtime_sanitized) if sanitized else None
        kobjs = [f.result() for f in kern]
        _link([*kobjs, rt.result()], LIBPKV)
        if san is not None:
            _link([*kobjs, san.result()], LIBPKV_SAN)
    return LIBPKV


def asan_runtime() -> str:
    """The shared AddressSanitizer runtime (it carries the UndefinedBehavior
    handlers too) that a process loading libpkv_san.so must preload."""
    return subprocess.run([CLANGXX, "-print-file-name=libclang_rt.asan-x86_64.so"], check=True,
                          capture_output=True, text=True).stdout.strip()


def build_libsynth() -> str:
    tmp = LIBSYNTH + ".tmp"
    _run([HIPCC, *DEVICE_FLAGS, "-shared", os.path.join(ROOT, "synth", "csrc", "fill.hip"),
          "-o", tmp])
    os.replace(tmp, LIBSYNTH)
    return LIBSYNTH


def build_all() -> None:
    with concurrent.futures.ThreadPoolExecutor(max_workers=2) as ex:
        a = ex.submit(build_libpkv)
        b = ex.submit(build_libsynth)
        a.result()
        b.result()


if __name__ == "__main__":
    build_all()
    sys.exit(0)
