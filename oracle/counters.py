"""Work and byte counts of the decode path (test infrastructure only).

* learn_llm ch.38, section "Count attention-score cells, not total runtime":
  at retained length t a cached step forms t scores per batch-layer-head lane;
  a complete-prefix call forms a t-by-t grid per lane.
* same page, the model-wide work counters: every token forward appends one row
  to each layer cache and projects three rows (Q, K, V) per layer.
* mbrenndoerfer "Rollout Serving, Caching, and Batching", section on the
  key-value cache: the cache of one session takes 2 * L * H * d_h * S * 2 bytes
  (key and value, two bytes per scalar).
"""
from __future__ import annotations


def cached_score_cells(lanes: int, retained_lengths) -> int:
    """Score values formed by cached newest-query rows: lanes * sum(t)."""
    return lanes * sum(int(t) for t in retained_lengths)


def complete_prefix_score_cells(lanes: int, lengths) -> int:
    """Score values formed by complete-prefix grids: lanes * sum(t^2)."""
    return lanes * sum(int(t) * int(t) for t in lengths)


def qkv_projection_rows(layers: int, token_rows: int) -> int:
    """Q, K and V rows projected: three per layer per token row."""
    return 3 * layers * token_rows


def kv_cache_bytes(layers: int, heads: int, head_width: int, positions: int,
                   scalar_bytes: int = 2) -> int:
    """Bytes of one session's K and V tensors: 2 * L * H * d_h * S * scalar_bytes."""
    return 2 * layers * heads * head_width * positions * scalar_bytes
