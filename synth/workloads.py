"""Workload recipes: the five synthetic configurations of the decode path.

Every quantity is drawn from ``synth`` streams keyed by the workload seed, so a
workload is reproducible from its name alone.  Lengths are *attended* lengths
``t``: the number of K/V rows the newest query reads, the newest row included.

Pool contents are a pure function of the flat element index inside each
layer's ``[physical_page, head, page_offset, head_width]`` block, drawn from the
K-pool / V-pool stream of that layer.  Rows appended during a step come from
the per-(layer, step) K/V streams and overwrite the pool slot of position
``t - 1``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import (TAG_ABORT, TAG_K, TAG_KPOOL, TAG_LENGTHS, TAG_Q, TAG_SHUFFLE,
               TAG_V, TAG_VPOOL, normals, shuffle, stream_key, uniform_ints,
               uniform_unit, counter_bits)

ELT_BYTES = {"f32": 4, "bf16": 2}


@dataclass
class Workload:
    name: str
    seed: int
    n: int
    layers: int
    heads: int
    head_width: int
    page_size: int
    num_pages: int
    dtype: str
    lengths: np.ndarray          # int64 [n], attended length incl. the newest row
    appends: bool                # the step writes row t-1 before attending
    page_tables: np.ndarray = field(default=None)  # int32 [n, pt_stride], -1 = unused
    abort_rate: float = 0.0
    description: str = ""
    kv_heads: int = 0            # K/V heads per layer; 0 = one per query head
    chunks: np.ndarray = field(default=None)  # prefill: new rows per request (ending at t)

    # ---- geometry -------------------------------------------------------
    @property
    def hkv(self) -> int:
        return self.kv_heads or self.heads

    @property
    def elt(self) -> int:
        return ELT_BYTES[self.dtype]

    @property
    def pt_stride(self) -> int:
        return int(self.page_tables.shape[1])

    @property
    def layer_elems(self) -> int:
        """Elements of one layer's K (or V) pool: P*H_kv*S*D."""
        return self.num_pages * self.hkv * self.page_size * self.head_width

    @property
    def row_elems(self) -> int:
        return self.n * self.heads * self.head_width

    @property
    def kv_row_elems(self) -> int:
        return self.n * self.hkv * self.head_width

    # ---- streams --------------------------------------------------------
    def kpool_key(self, layer: int) -> int:
        return stream_key(self.seed, TAG_KPOOL, layer)

    def vpool_key(self, layer: int) -> int:
        return stream_key(self.seed, TAG_VPOOL, layer)

    def q_key(self, layer: int, step: int = 0) -> int:
        return stream_key(self.seed, TAG_Q, layer, step)

    def k_key(self, layer: int, step: int = 0) -> int:
        return stream_key(self.seed, TAG_K, layer, step)

    def v_key(self, layer: int, step: int = 0) -> int:
        return stream_key(self.seed, TAG_V, layer, step)

    def q(self, layer: int, step: int = 0) -> np.ndarray:
        """Query rows ``[n, H, D]`` (float32 or bfloat16 bits)."""
        return normals(self.q_key(layer, step), 0, self.row_elems, self.dtype).reshape(
            self.n, self.heads, self.head_width)

    def k_new(self, layer: int, step: int = 0) -> np.ndarray:
        """New key rows ``[n, H_kv, D]``."""
        return normals(self.k_key(layer, step), 0, self.kv_row_elems, self.dtype).reshape(
            self.n, self.hkv, self.head_width)

    def v_new(self, layer: int, step: int = 0) -> np.ndarray:
        return normals(self.v_key(layer, step), 0, self.kv_row_elems, self.dtype).reshape(
            self.n, self.hkv, self.head_width)

    def chunk_rows(self, layer: int, step: int = 0):
        """Prefill rows of every request's chunk, packed request after request:
        q [T, H, D], k and v [T, H_kv, D] with T = sum of chunks."""
        total = int(np.sum(self.chunks))
        out = []
        for tag, heads in ((TAG_Q, self.heads), (TAG_K, self.hkv), (TAG_V, self.hkv)):
            key = stream_key(self.seed, tag, layer, 1000 + step)
            out.append(normals(key, 0, total * heads * self.head_width, self.dtype).reshape(
                total, heads, self.head_width))
        return tuple(out)

    @property
    def starts(self) -> np.ndarray:
        """Prefill: position of each chunk's first row (the retained prefix)."""
        return self.lengths - self.chunks

    def prefill_flops(self) -> int:
        """Score and value products of one prefill layer: 4 d_h per (new row,
        query head, attended row)."""
        c, st = self.chunks.astype(np.int64), self.starts.astype(np.int64)
        rows = int(np.sum(c * st + c * (c + 1) // 2))
        return rows * self.heads * 4 * self.head_width

    def pool_page(self, which: str, layer: int, page: int) -> np.ndarray:
        """Generator content of one physical page ``[H_kv, S, D]`` of one layer."""
        per_page = self.hkv * self.page_size * self.head_width
        key = self.kpool_key(layer) if which == "k" else self.vpool_key(layer)
        vals = normals(key, page * per_page, per_page, self.dtype)
        return vals.reshape(self.hkv, self.page_size, self.head_width)

    # ---- accounting -----------------------------------------------------
    def kv_bytes_per_layer(self) -> int:
        """Algorithmic K/V bytes one layer's attention must read:
        sum_r t_r*H_kv*2*D*elt (a K/V head shared by a group is read once)."""
        return int(self.lengths.sum()) * self.hkv * 2 * self.head_width * self.elt

    def kv_bytes(self) -> int:
        return self.kv_bytes_per_layer() * self.layers

    def abort_layer(self, step: int) -> np.ndarray:
        """Per request: the layer at which this step is aborted, or -1."""
        if self.abort_rate <= 0:
            return np.full(self.n, -1, dtype=np.int64)
        key = stream_key(self.seed, TAG_ABORT, step)
        idx = np.arange(self.n, dtype=np.uint64)
        hit = uniform_unit(key, 2 * idx) < self.abort_rate
        layer = ((counter_bits(key, 2 * idx + np.uint64(1)) >> np.uint64(32))
                 * np.uint64(self.layers) >> np.uint64(32)).astype(np.int64)
        return np.where(hit, layer, -1)


def pages_needed(lengths: np.ndarray, page_size: int) -> np.ndarray:
    return (np.asarray(lengths, dtype=np.int64) + page_size - 1) // page_size


def assign_page_tables(seed: int, lengths: np.ndarray, page_size: int, num_pages: int,
                       stride: int | None = None) -> np.ndarray:
    """Request r takes the next ceil(t_r/S) IDs of a seeded shuffle of [0, P)."""
    need = pages_needed(lengths, page_size)
    total = int(need.sum())
    if total > num_pages:
        raise ValueError(f"workload needs {total} pages, pool has {num_pages}")
    perm = shuffle(stream_key(seed, TAG_SHUFFLE), num_pages)
    stride = int(need.max()) if stride is None else stride
    pt = np.full((len(lengths), stride), -1, dtype=np.int32)
    off = 0
    for r, c in enumerate(need.tolist()):
        pt[r, :c] = perm[off:off + c]
        off += c
    return pt


def _finish(w: Workload, stride: int | None = None) -> Workload:
    w.page_tables = assign_page_tables(w.seed, w.lengths, w.page_size, w.num_pages, stride)
    return w


def tiny_geometry() -> dict:
    """Tiny fixture: 1 request, 2 layers, 2 heads, head width 2, 16-token pages,
    8 physical pages, float32, decoded token at a time to lengths 1..4."""
    return dict(name="tiny", seed=1, n=1, layers=2, heads=2, head_width=2,
                page_size=16, num_pages=8, dtype="f32", max_len=4)


def tiny_rows(seed: int, layer: int, position: int, heads: int, head_width: int):
    """q, k, v rows ``[H, D]`` float32 for one (layer, position) of the tiny fixture."""
    n = heads * head_width
    out = []
    for tag in (TAG_Q, TAG_K, TAG_V):
        out.append(normals(stream_key(seed, tag, layer, position), 0, n, "f32").reshape(
            heads, head_width))
    return tuple(out)


def batch32_fp32() -> Workload:
    """32 requests, 12 layers, H=12, D=64, 16-token pages, lengths U[1,1024],
    4096-page pool with shuffled page tables, float32, one decode step of all
    layers (append, then attend)."""
    seed = 2
    lengths = uniform_ints(stream_key(seed, TAG_LENGTHS), 32, 1, 1024)
    w = Workload("batch32_fp32_l12", seed, 32, 12, 12, 64, 16, 4096, "f32", lengths,
                 appends=True, description=batch32_fp32.__doc__)
    return _finish(w, stride=1024 // 16 + 8)


def batch256_bf16() -> Workload:
    """256 requests, one layer, H=32, D=128, 16-token pages, lengths U[512,4096],
    bf16 K/V and q, float32 accumulate, decode attention over existing rows."""
    seed = 3
    lengths = uniform_ints(stream_key(seed, TAG_LENGTHS), 256, 512, 4096)
    P = int(pages_needed(lengths, 16).sum()) + 256
    w = Workload("batch256_bf16", seed, 256, 1, 32, 128, 16, P, "bf16", lengths,
                 appends=False, description=batch256_bf16.__doc__)
    return _finish(w)


def skewed64_bf16() -> Workload:
    """64 requests, one layer, H=32, D=128, 16-token pages, lengths log-uniform
    in [16, 32768], bf16 K/V and q: long and short contexts in one batch."""
    seed = 4
    u = uniform_unit(stream_key(seed, TAG_LENGTHS), np.arange(64, dtype=np.uint64))
    lengths = np.minimum(32768, np.floor(16.0 * np.power(2048.0, u))).astype(np.int64)
    P = int(pages_needed(lengths, 16).sum()) + 64
    w = Workload("skewed64_bf16", seed, 64, 1, 32, 128, 16, P, "bf16", lengths,
                 appends=False, description=skewed64_bf16.__doc__)
    return _finish(w)


def fullstep128_bf16(extra_steps: int = 64) -> Workload:
    """Full decode step: 32 layers, 128 requests, H=32, D=128, 16-token pages,
    retained prefix U[1536,2560] before the step, bf16; each layer appends then
    attends; commit per request, with 1% of (request, step) aborted at a seeded
    layer.  ``lengths`` are the attended lengths of the first step.  The page
    tables of this workload come from the library's allocator; the pool is sized
    for ``extra_steps`` further committed tokens per request."""
    seed = 5
    prefix = uniform_ints(stream_key(seed, TAG_LENGTHS), 128, 1536, 2560)
    lengths = prefix + 1
    P = int(pages_needed(prefix + 1 + extra_steps, 16).sum()) + 128
    w = Workload("fullstep128_bf16_l32", seed, 128, 32, 32, 128, 16, P, "bf16", lengths,
                 appends=True, abort_rate=0.01, description=fullstep128_bf16.__doc__)
    w.page_tables = np.zeros((128, 0), dtype=np.int32)
    return w


def batch256_gqa8_bf16() -> Workload:
    """The 256-request bf16 batch with grouped K/V heads: H=32 query heads
    sharing H_kv=8 K/V heads (groups of 4), D=128, 16-token pages, lengths
    U[512,4096] from the same stream as the multi-head batch."""
    seed = 3
    lengths = uniform_ints(stream_key(seed, TAG_LENGTHS), 256, 512, 4096)
    P = int(pages_needed(lengths, 16).sum()) + 256
    w = Workload("batch256_gqa8_bf16", seed, 256, 1, 32, 128, 16, P, "bf16", lengths,
                 appends=False, description=batch256_gqa8_bf16.__doc__, kv_heads=8)
    return _finish(w)


def batch256_mqa_bf16() -> Workload:
    """The 256-request bf16 batch with one K/V head under all H=32 query
    heads (multi-query attention), D=128, 16-token pages, lengths U[512,4096]
    from the same stream as the multi-head batch."""
    seed = 3
    lengths = uniform_ints(stream_key(seed, TAG_LENGTHS), 256, 512, 4096)
    P = int(pages_needed(lengths, 16).sum()) + 256
    w = Workload("batch256_mqa_bf16", seed, 256, 1, 32, 128, 16, P, "bf16", lengths,
                 appends=False, description=batch256_mqa_bf16.__doc__, kv_heads=1)
    return _finish(w)


def prefill32_bf16() -> Workload:
    """Batched prefill: 32 requests, one layer, H=32, D=128, 16-token pages,
    bf16; each request appends a chunk of U[256, 2048] new rows after a
    retained prefix of U[0, 2048] rows, every new row attending causally."""
    seed = 6
    prefix = uniform_ints(stream_key(seed, TAG_LENGTHS, 0), 32, 0, 2048)
    chunks = uniform_ints(stream_key(seed, TAG_LENGTHS, 1), 32, 256, 2048)
    lengths = prefix + chunks
    P = int(pages_needed(lengths, 16).sum()) + 32
    w = Workload("prefill32_bf16", seed, 32, 1, 32, 128, 16, P, "bf16", lengths,
                 appends=True, description=prefill32_bf16.__doc__, chunks=chunks)
    return _finish(w)


def prefill32_fp32() -> Workload:
    """Batched float32 prefill in the geometry of the 12-layer float32 step:
    32 requests, one layer, H=12, D=64, 16-token pages, fp32; chunks of
    U[256, 2048] new rows after retained prefixes of U[0, 2048] rows, drawn as
    for the bf16 prefill but from their own seed."""
    seed = 7
    prefix = uniform_ints(stream_key(seed, TAG_LENGTHS, 0), 32, 0, 2048)
    chunks = uniform_ints(stream_key(seed, TAG_LENGTHS, 1), 32, 256, 2048)
    lengths = prefix + chunks
    P = int(pages_needed(lengths, 16).sum()) + 32
    w = Workload("prefill32_fp32", seed, 32, 1, 12, 64, 16, P, "f32", lengths,
                 appends=True, description=prefill32_fp32.__doc__, chunks=chunks)
    return _finish(w)


WORKLOADS = {
    "batch32_fp32_l12": batch32_fp32,
    "batch256_bf16": batch256_bf16,
    "batch256_gqa8_bf16": batch256_gqa8_bf16,
    "batch256_mqa_bf16": batch256_mqa_bf16,
    "prefill32_bf16": prefill32_bf16,
    "prefill32_fp32": prefill32_fp32,
    "skewed64_bf16": skewed64_bf16,
    "fullstep128_bf16_l32": fullstep128_bf16,
}


def expected_pages(lengths: np.ndarray, page_size: int) -> int:
    return int(sum(math.ceil(int(t) / page_size) for t in lengths))
