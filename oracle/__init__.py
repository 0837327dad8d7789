"""CPU oracle for paged decode attention — TEST INFRASTRUCTURE, not product code.

A plain, slow, float64 implementation of what the decode path computes,
written from the pages' definitions.  Only ``tests/``, ``__graft_entry__.smoke``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code
with the HIP library (``paged_kv_cache_attention_amd``) and imports nothing from
it; the two meet only on inputs drawn by ``synth``.

Modules:

* ``oracle.attention`` — gather through a page table, softmax(q K^T / sqrt(d_h)) V,
  append-then-attend with a candidate row, the newest row of full causal
  attention, split partials and their log-sum-exp merge, K/V heads shared by
  groups of query heads, and a causal chunk of new rows over a paged prefix
  (batched prefill).
* ``oracle.counters`` — attention-score-cell counts and K/V byte accounting.
* ``oracle.transaction`` — the visible-state model of begin / append / commit /
  abort / reset on a request cache backed by a page pool (one token or a
  chunk of tokens per transaction).

Pins (tests/test_oracle_pins.py): agreement with an independent library
attention routine and with the newest row of full causal attention; closed
forms; contiguous-vs-paged and permutation invariance; split/merge identity;
the pages' printed counts.  Parity unpinned: none of the functions here (every
function has at least one pin); the pages' fixture logits are outside this
path (they need model weights the pages do not give).
"""
from .attention import (append_and_attend, attend, causal_attention, gather_prefix,
                        kv_head_of, kv_to_f64, merge_partials, paged_decode_attention,
                        prefill_attention, split_partials)
from .counters import (cached_score_cells, complete_prefix_score_cells, kv_cache_bytes,
                       qkv_projection_rows)
from .transaction import CacheModel, PoolModel, Status

__all__ = [
    "append_and_attend", "attend", "causal_attention", "gather_prefix", "kv_head_of", "kv_to_f64",
    "merge_partials", "paged_decode_attention", "prefill_attention", "split_partials",
    "cached_score_cells", "complete_prefix_score_cells", "kv_cache_bytes",
    "qkv_projection_rows", "CacheModel", "PoolModel", "Status",
]
