"""Visible-state model of the per-token cache transaction (test infrastructure only).

Sources, by page and section:

* riftco-transformer "Incremental Serving", section "Request flow": begin
  reserves the next logical position; each layer appends and attends; commit
  makes the position visible; abort leaves the visible length unchanged.
* same page, section "Paged KV-cache layout": pages are leased lazily as a
  sequence grows and return to the pool on reset or destroy.
* same page, section "Stable C and Python sessions": a session reports capacity
  exhaustion and does not crop or replay by itself.
* learn_llm ch.38, section "Prepare every block, then commit every cache
  together": every block prepares before any cache commits, so commit requires
  all layers; rejected operations leave the committed state unchanged.

Readings where the pages are silent: abort also returns the pages that this
transaction's begin leased (so pool and page table equal their state before
begin); a begin may reserve a chunk of n positions (batched prefill, which the
pages name as future work), and then commit and abort act on all n at once;
reset while a token is pending is rejected; destroy always succeeds and
returns every page, the pending one included; a call with an invalid argument
is rejected as such before the state is consulted.
"""
from __future__ import annotations

import enum


class Status(enum.IntEnum):
    OK = 0
    INVALID_ARGUMENT = 1
    BAD_STATE = 2
    OUT_OF_PAGES = 3
    CAPACITY_EXHAUSTED = 4


class PoolModel:
    def __init__(self, num_pages: int):
        self.num_pages = num_pages
        self.leased = 0

    @property
    def free(self) -> int:
        return self.num_pages - self.leased


class CacheModel:
    """One request cache: committed length, pending token, pages held."""

    def __init__(self, pool: PoolModel, layers: int, capacity: int, page_size: int):
        self.pool = pool
        self.layers = layers
        self.capacity = capacity
        self.page_size = page_size
        self.length = 0
        self.pending = None          # (position, new pages leased, appended layers, count)
        self.retained_lengths = []   # attended length of every committed token
        self.appends = 0

    @property
    def pages_held(self) -> int:
        n = -(-self.length // self.page_size)
        if self.pending is not None:
            n += self.pending[1]
        return n

    def begin(self, count: int = 1) -> Status:
        if count < 1:
            return Status.INVALID_ARGUMENT
        if self.pending is not None:
            return Status.BAD_STATE
        if self.length + count > self.capacity:
            return Status.CAPACITY_EXHAUSTED
        new_pages = -(-(self.length + count) // self.page_size) - (-(-self.length // self.page_size))
        if new_pages > self.pool.free:
            return Status.OUT_OF_PAGES
        self.pool.leased += new_pages
        self.pending = (self.length, new_pages, set(), count)
        return Status.OK

    def append(self, layer: int) -> Status:
        if not 0 <= layer < self.layers:
            return Status.INVALID_ARGUMENT
        if self.pending is None:
            return Status.BAD_STATE
        if layer in self.pending[2]:
            return Status.BAD_STATE
        self.pending[2].add(layer)
        return Status.OK

    def commit(self) -> Status:
        if self.pending is None or len(self.pending[2]) != self.layers:
            return Status.BAD_STATE
        for _ in range(self.pending[3]):
            self.length += 1
            self.retained_lengths.append(self.length)
            self.appends += self.layers
        self.pending = None
        return Status.OK

    def abort(self) -> Status:
        if self.pending is None:
            return Status.BAD_STATE
        self.pool.leased -= self.pending[1]
        self.pending = None
        return Status.OK

    def reset(self) -> Status:
        if self.pending is not None:
            return Status.BAD_STATE
        self.pool.leased -= self.pages_held
        self.length = 0
        return Status.OK

    def destroy(self) -> Status:
        self.pool.leased -= self.pages_held
        self.length = 0
        self.pending = None
        return Status.OK
