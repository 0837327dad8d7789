"""Device fill of seeded inputs: the same values as ``synth.normals``, written
by a small HIP kernel (``synth/csrc/fill.hip``) so large pools never cross PCIe.

Element ``i`` of the filled buffer equals ``synth.normals(key, start + i, ...)``
bit for bit: the kernel evaluates the same SplitMix64 output and reads the
same table bytes (uploaded from ``synth.table_for``).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import table_for

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None
_tables: dict = {}


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} missing; run `python paged_kv_cache_attention_amd/build.py`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.synth_fill.restype = ctypes.c_int
        lib.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                   ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                   ctypes.c_void_p]
        _lib = lib
    return _lib


def torch_dtype(dtype: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def device_table(dtype: str, device) -> torch.Tensor:
    key = (dtype, str(device))
    if key not in _tables:
        tab = table_for(dtype)
        host = torch.from_numpy(tab.view(np.int32 if dtype == "f32" else np.int16).copy())
        _tables[key] = host.to(device)
    return _tables[key]


def fill_normal(dst: torch.Tensor, key: int, dtype: str, start: int = 0, stream=None) -> None:
    """Fill a contiguous device tensor with N(0,1) values of stream ``key``."""
    if not dst.is_contiguous():
        raise ValueError("fill_normal needs a contiguous tensor")
    elem = 4 if dtype == "f32" else 2
    if dst.element_size() != elem:
        raise ValueError(f"tensor element size {dst.element_size()} does not match {dtype}")
    lib = _load()
    tab = device_table(dtype, dst.device)
    s = stream.cuda_stream if stream is not None else torch.cuda.current_stream(dst.device).cuda_stream
    err = lib.synth_fill(dst.data_ptr(), dst.numel(), start, key & ((1 << 64) - 1), tab.data_ptr(),
                         elem, s)
    if err != 0:
        raise RuntimeError(f"synth_fill failed with hipError {err}")


def to_device(host: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Copy host generator output (float32, or uint16 bfloat16 bits) to the device."""
    if dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(host, dtype=np.float32))
    else:
        t = torch.from_numpy(np.ascontiguousarray(host).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def to_host_bits(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Device tensor back to generator form (float32 or uint16 bits), bit for bit."""
    c = t.detach().contiguous().cpu()
    if dtype == "f32":
        return c.view(torch.int32).numpy().view(np.float32)
    return c.view(torch.int16).numpy().view(np.uint16)
