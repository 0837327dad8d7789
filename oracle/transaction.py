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

Readings where the pages are silent: abort also returns a page that this
token's begin leased (so pool and page table equal their state before begin);
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
        self.pending = None          # (position, leased_new_page, set of appended layers)
        self.retained_lengths = []   # attended length of every committed token
        self.appends = 0

    @property
    def pages_held(self) -> int:
        n = -(-self.length // self.page_size)
        if self.pending is not None and self.pending[1]:
            n += 1
        return n

    def begin(self) -> Status:
        if self.pending is not None:
            return Status.BAD_STATE
        if self.length >= self.capacity:
            return Status.CAPACITY_EXHAUSTED
        needs_page = self.length % self.page_size == 0
        if needs_page:
            if self.pool.free == 0:
                return Status.OUT_OF_PAGES
            self.pool.leased += 1
        self.pending = (self.length, needs_page, set())
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
        self.length += 1
        self.retained_lengths.append(self.length)
        self.appends += self.layers
        self.pending = None
        return Status.OK

    def abort(self) -> Status:
        if self.pending is None:
            return Status.BAD_STATE
        if self.pending[1]:
            self.pool.leased -= 1
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
