"""Seeded synthetic inputs, shared by the CPU oracle tests and the device path.

This package holds none of the attention arithmetic. It only draws numbers:

* a counter-based form of SplitMix64 (Steele, Lea and Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014; constants as in Vigna's public
  reference implementation).  Output ``i`` of a stream whose state starts at
  ``key`` is ``mix64(key + (i + 1) * GOLDEN)``, so any element of any stream can
  be computed directly from its index;
* N(0,1) deviates by the inverse-transform method on a 2**16-level table:
  entry ``i`` is the standard normal quantile at ``(i + 0.5) / 2**16``, rounded
  to float32 (and from there to bfloat16, round-to-nearest-even).  The top 16
  bits of the counter output select the entry.  The same table bytes are used
  on the host (numpy) and by the device fill kernel in ``synth/csrc``, so both
  produce bit-identical values;
* integer length distributions and Fisher-Yates shuffles for page tables.

The workload recipes built from these live in ``synth.workloads``.
"""
from __future__ import annotations

import functools

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB

TABLE_BITS = 16
TABLE_SIZE = 1 << TABLE_BITS

# Stream tags: each kind of drawn quantity gets its own stream.
TAG_LENGTHS = 1
TAG_SHUFFLE = 2
TAG_Q = 3
TAG_K = 4
TAG_V = 5
TAG_KPOOL = 6
TAG_VPOOL = 7
TAG_ABORT = 8
TAG_MISC = 9


def mix64_int(z: int) -> int:
    """SplitMix64 output function on one Python integer."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * _M1) & MASK64
    z = ((z ^ (z >> 27)) * _M2) & MASK64
    return z ^ (z >> 31)


def splitmix64_outputs(state: int, count: int) -> list[int]:
    """The first ``count`` outputs of a sequential SplitMix64 generator."""
    out = []
    for _ in range(count):
        state = (state + GOLDEN) & MASK64
        out.append(mix64_int(state))
    return out


def _mix64_array(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> np.uint64(30))
    z = z * np.uint64(_M1)
    z = z ^ (z >> np.uint64(27))
    z = z * np.uint64(_M2)
    return z ^ (z >> np.uint64(31))


def counter_bits(key: int, idx: np.ndarray) -> np.ndarray:
    """Output ``idx`` (0-based, uint64 array) of the stream starting at ``key``."""
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key & MASK64) + (idx + np.uint64(1)) * np.uint64(GOLDEN)
        return _mix64_array(z)


def stream_key(seed: int, *tags: int) -> int:
    """Derive an independent stream key from a seed and a tuple of tags."""
    s = seed & MASK64
    for t in tags:
        s = mix64_int((s + ((t + 1) & MASK64) * GOLDEN) & MASK64)
    return s


@functools.lru_cache(maxsize=None)
def normal_table_f32() -> np.ndarray:
    """2**16 standard-normal quantiles at midpoints, rounded to float32."""
    from scipy.special import ndtri

    u = (np.arange(TABLE_SIZE, dtype=np.float64) + 0.5) / TABLE_SIZE
    tab = ndtri(u).astype(np.float32)
    tab.setflags(write=False)
    return tab


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits.

    Inputs must be finite (the table is).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


@functools.lru_cache(maxsize=None)
def normal_table_bf16() -> np.ndarray:
    tab = f32_to_bf16_bits(normal_table_f32())
    tab.setflags(write=False)
    return tab


def table_for(dtype: str) -> np.ndarray:
    if dtype == "f32":
        return normal_table_f32()
    if dtype == "bf16":
        return normal_table_bf16()
    raise ValueError(f"unknown dtype {dtype!r}")


def normals_at(key: int, idx: np.ndarray, dtype: str) -> np.ndarray:
    """N(0,1) values at flat stream indices ``idx``.

    Returns float32 values for ``dtype='f32'`` and uint16 bfloat16 bit
    patterns for ``dtype='bf16'``.
    """
    bits = counter_bits(key, idx)
    return table_for(dtype)[(bits >> np.uint64(64 - TABLE_BITS)).astype(np.int64)]


def normals(key: int, start: int, count: int, dtype: str) -> np.ndarray:
    """N(0,1) values at flat stream indices ``start .. start+count-1``."""
    idx = np.arange(start, start + count, dtype=np.uint64)
    return normals_at(key, idx, dtype)


def uniform_below(key: int, idx: np.ndarray, bound: int) -> np.ndarray:
    """Integers uniform in ``[0, bound)`` by the multiply-shift method on 32 bits."""
    hi = counter_bits(key, idx) >> np.uint64(32)
    return ((hi * np.uint64(bound)) >> np.uint64(32)).astype(np.int64)


def uniform_ints(key: int, count: int, lo: int, hi: int) -> np.ndarray:
    """``count`` integers uniform in the inclusive range ``[lo, hi]``."""
    idx = np.arange(count, dtype=np.uint64)
    return lo + uniform_below(key, idx, hi - lo + 1)


def uniform_unit(key: int, idx: np.ndarray) -> np.ndarray:
    """Doubles uniform in ``[0, 1)`` from the top 53 bits."""
    return (counter_bits(key, idx) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def shuffle(key: int, n: int) -> np.ndarray:
    """A Fisher-Yates permutation of ``0 .. n-1`` (int32)."""
    perm = np.arange(n, dtype=np.int32)
    if n <= 1:
        return perm
    js = np.arange(n - 1, 0, -1, dtype=np.int64)
    hi = (counter_bits(key, np.arange(n - 1, dtype=np.uint64)) >> np.uint64(32))
    draws = ((hi * (js + 1).astype(np.uint64)) >> np.uint64(32)).astype(np.int64)
    for i, j in zip(js.tolist(), draws.tolist()):
        perm[i], perm[j] = perm[j], perm[i]
    return perm
