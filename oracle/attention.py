"""Float64 decode attention, written from the pages (test infrastructure only).

Sources, by page and section:

* riftco-transformer "Incremental Serving", section "Request flow": each layer
  receives query, key and value of shape [1, H, 1, d_h] and returns a context of
  the same shape; the new K/V row becomes part of the cache.
* same page, section "Paged KV-cache layout": per layer, key pages and value
  pages are laid out [physical_page, head, page_offset, head_width]; a request
  owns a logical-to-physical page table; default page size 16; a contiguous
  strategy is one page as long as the maximum context.
* learn_llm ch.38 "cached generation", section "Prepare every block, then commit
  every cache together" (the incremental mixture): each score is the dot
  product of the query with a retained key times 1/sqrt(d_h); the retained rows
  plus the candidate row at position len are scored (len+1 rows); a stable
  softmax over them weights the value rows.
* same page, section "Count attention-score cells, not total runtime": a
  complete-prefix call rebuilds the whole causal score grid; the cached call
  forms only the newest query's row.

* mbrenndoerfer "Rollout Serving, Caching, and Batching", key-value cache
  section: grouped-query or multi-query attention keeps fewer K/V heads than
  query heads.  Reading where the page is silent: query head h of H reads K/V
  head h // (H / H_kv) (consecutive groups); H_kv = H is the pages' case.

Floating point: everything is float64.  bfloat16 inputs arrive as uint16 bit
patterns and widen exactly (bits << 16 is the float32 with the same value).
"""
from __future__ import annotations

import math

import numpy as np


def kv_to_f64(x: np.ndarray) -> np.ndarray:
    """Exact float64 value of float32 data, or of bfloat16 data given as uint16 bits."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported K/V dtype {x.dtype}")


def gather_prefix(pages, page_table, t: int, page_size: int, head: int) -> np.ndarray:
    """Logical rows 0..t-1 of one head, read through a page table.

    ``pages[p]`` is physical page ``p`` of one layer, shaped [head, page_offset,
    head_width].  Logical row ``j`` lives at page ``page_table[j // S]``, slot
    ``j % S`` (Paged KV-cache layout).  Returns the raw dtype, shape [t, D].
    """
    if t < 0:
        raise ValueError("negative length")
    chunks = []
    for logical in range((t + page_size - 1) // page_size):
        physical = int(page_table[logical])
        rows = min(page_size, t - logical * page_size)
        chunks.append(np.asarray(pages[physical])[head, :rows, :])
    if not chunks:
        return np.zeros((0, 0))
    return np.concatenate(chunks, axis=0)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """softmax(q K^T / sqrt(d_h)) V for one query row, in float64.

    q: [D]; K, V: [t, D] with t >= 1.  The softmax subtracts the maximum score
    before exponentiating (the stable form the incremental mixture uses).
    """
    q = kv_to_f64(q)
    K = kv_to_f64(K)
    V = kv_to_f64(V)
    if K.shape[0] < 1:
        raise ValueError("softmax over an empty prefix is undefined")
    d = q.shape[-1]
    scores = (K @ q) * (1.0 / math.sqrt(d))
    shifted = np.exp(scores - scores.max())
    probs = shifted / shifted.sum()
    return probs @ V


def kv_head_of(h: int, num_heads: int, num_kv_heads: int) -> int:
    """K/V head read by query head h: consecutive groups of H / H_kv."""
    if num_heads % num_kv_heads:
        raise ValueError("query heads must be a multiple of K/V heads")
    return h // (num_heads // num_kv_heads)


def paged_decode_attention(q, k_pages, v_pages, page_table, t: int, page_size: int,
                           num_kv_heads: int | None = None):
    """Context [H, D] of one request whose attended prefix has ``t`` rows.

    q: [H, D]; ``k_pages`` / ``v_pages`` index physical pages of one layer,
    each [H_kv, S, D] (H_kv defaults to H).
    """
    H = q.shape[0]
    Hkv = H if num_kv_heads is None else num_kv_heads
    out = np.empty((H, q.shape[1]), dtype=np.float64)
    for h in range(H):
        kvh = kv_head_of(h, H, Hkv)
        K = gather_prefix(k_pages, page_table, t, page_size, kvh)
        V = gather_prefix(v_pages, page_table, t, page_size, kvh)
        out[h] = attend(q[h], K, V)
    return out


def append_and_attend(q, k_new, v_new, k_pages, v_pages, page_table, length: int,
                      page_size: int):
    """One layer's append-then-attend for a request with ``length`` committed rows.

    The retained rows 0..length-1 come from the pages; the candidate row (k_new,
    v_new) sits at position ``length``; the query attends to all length+1 rows.
    q: [H, D]; k_new, v_new: [H_kv, D] (H_kv = H unless K/V heads are shared).
    Returns the context [H, D] in float64.
    """
    H = q.shape[0]
    Hkv = k_new.shape[0]
    out = np.empty((H, q.shape[1]), dtype=np.float64)
    for h in range(H):
        kvh = kv_head_of(h, H, Hkv)
        K = kv_to_f64(gather_prefix(k_pages, page_table, length, page_size, kvh)) if length else \
            np.zeros((0, q.shape[1]))
        V = kv_to_f64(gather_prefix(v_pages, page_table, length, page_size, kvh)) if length else \
            np.zeros((0, q.shape[1]))
        K = np.concatenate([K.reshape(-1, q.shape[1]), kv_to_f64(k_new[kvh])[None, :]], axis=0)
        V = np.concatenate([V.reshape(-1, q.shape[1]), kv_to_f64(v_new[kvh])[None, :]], axis=0)
        out[h] = attend(q[h], K, V)
    return out


def prefill_attention(q, k_new, v_new, k_pages, v_pages, page_table, start: int,
                      page_size: int):
    """A chunk of n new rows at positions start..start+n-1, each attending
    causally: row i sees the retained rows 0..start-1 (from the pages) and the
    chunk's rows 0..i.

    The pages process a prompt one token at a time and name a batched prefill
    that writes the same paged cache as future work ("Incremental Serving",
    Paged KV-cache layout); reading: a chunk computes exactly what n
    token-at-a-time steps would, i.e. row i is the newest-query result at
    attended length start+i+1.  q: [n, H, D]; k_new, v_new: [n, H_kv, D].
    Returns the contexts [n, H, D] in float64.
    """
    n, H, D = q.shape
    Hkv = k_new.shape[1]
    out = np.empty((n, H, D), dtype=np.float64)
    for h in range(H):
        kvh = kv_head_of(h, H, Hkv)
        Kp = kv_to_f64(gather_prefix(k_pages, page_table, start, page_size, kvh)).reshape(-1, D)
        Vp = kv_to_f64(gather_prefix(v_pages, page_table, start, page_size, kvh)).reshape(-1, D)
        K = np.concatenate([Kp, kv_to_f64(k_new[:, kvh, :])], axis=0)
        V = np.concatenate([Vp, kv_to_f64(v_new[:, kvh, :])], axis=0)
        for i in range(n):
            out[i, h] = attend(q[i, h], K[:start + i + 1], V[:start + i + 1])
    return out


def causal_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Full causal attention over t rows: row i attends to rows 0..i.

    Builds the whole t-by-t score grid (the complete-prefix computation) with
    future positions masked out, then a row-wise stable softmax.  Q, K, V: [t, D].
    """
    Q = kv_to_f64(Q)
    K = kv_to_f64(K)
    V = kv_to_f64(V)
    t, d = Q.shape
    grid = (Q @ K.T) / math.sqrt(d)
    future = np.triu(np.ones((t, t), dtype=bool), k=1)
    grid = np.where(future, -np.inf, grid)
    grid = grid - grid.max(axis=1, keepdims=True)
    w = np.exp(grid)
    return (w / w.sum(axis=1, keepdims=True)) @ V


def split_partials(q, K, V, bounds):
    """Per split [b0, b1): (m, l, acc) with m = max score, l = sum exp(s - m),
    acc = sum exp(s - m) v, natural-log domain, float64."""
    q = kv_to_f64(q)
    K = kv_to_f64(K)
    V = kv_to_f64(V)
    scale = 1.0 / math.sqrt(q.shape[-1])
    parts = []
    for b0, b1 in bounds:
        s = (K[b0:b1] @ q) * scale
        m = s.max()
        e = np.exp(s - m)
        parts.append((m, e.sum(), e @ V[b0:b1]))
    return parts


def merge_partials(parts):
    """Log-sum-exp merge: o = sum_s e^(m_s - M) acc_s / sum_s e^(m_s - M) l_s."""
    M = max(m for m, _, _ in parts)
    num = sum(np.exp(m - M) * acc for m, _, acc in parts)
    den = sum(np.exp(m - M) * l for m, l, _ in parts)
    return num / den
