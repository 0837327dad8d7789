"""Builds libpkv.so (and the seeded-input fill library) for gfx950 with hipcc.

Run ``python paged_kv_cache_attention_amd/build.py`` (by path: importing the
package would load the library being rebuilt); both libraries are written
in-tree next to their sources.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed FP32 instructions are disabled for all device code.
COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-result"]

LIBPKV = os.path.join(HERE, "libpkv.so")
LIBSYNTH = os.path.join(ROOT, "synth", "libsynth.so")


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build_libpkv() -> str:
    srcs = [os.path.join(HERE, "csrc", f) for f in ("kernels.hip", "prefill.hip", "runtime.cpp")]
    tmp = LIBPKV + ".tmp"
    _run([HIPCC, *COMMON, "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp])
    os.replace(tmp, LIBPKV)
    return LIBPKV


def build_libsynth() -> str:
    tmp = LIBSYNTH + ".tmp"
    _run([HIPCC, *COMMON, os.path.join(ROOT, "synth", "csrc", "fill.hip"), "-o", tmp])
    os.replace(tmp, LIBSYNTH)
    return LIBSYNTH


def build_all() -> None:
    build_libpkv()
    build_libsynth()


if __name__ == "__main__":
    build_all()
    sys.exit(0)
