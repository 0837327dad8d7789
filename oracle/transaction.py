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

* same page, section "Current scope": paged storage alone neither shares pages
  between requests nor manages prefixes by copy-on-write; the model adds that
  mechanism as the library builds it (fork, reference counts, copy on write).

Readings where the pages are silent: abort also returns the pages that this
transaction's begin leased (so pool and page table equal their state before
begin); a begin may reserve a chunk of n positions (batched prefill, which the
pages name as future work), and then commit and abort act on all n at once; a
fork shares the pages of a committed prefix, full shared pages are never
written, and the first write into a shared partly filled page gives the
writer a private copy (abort undoes it); a page is free once no cache and no
queued copy holds it;
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
    """Pages by identity with their holders: caches, and a pending
    transaction's hold on the shared page it copied on write (kept until the
    transaction commits or aborts, so a queued copy's source stays
    allocated)."""

    def __init__(self, num_pages: int):
        self.num_pages = num_pages
        self.refs = {}        # page -> number of holders
        self.copies = []      # queued copies (source, destination)
        self._next = 0

    @property
    def leased(self) -> int:
        return len(self.refs)

    @property
    def free(self) -> int:
        return self.num_pages - len(self.refs)

    @property
    def shared(self) -> int:
        return sum(1 for r in self.refs.values() if r > 1)

    def lease(self) -> int:
        page = self._next
        self._next += 1
        self.refs[page] = 1
        return page

    def hold(self, page: int) -> None:
        self.refs[page] += 1

    def release(self, page: int) -> None:
        self.refs[page] -= 1
        if self.refs[page]:
            return
        del self.refs[page]
        # a copy queued into a page nobody holds any more is cancelled
        self.copies = [c for c in self.copies if c[1] != page]

    def flush(self) -> None:
        """The queued copies are enqueued."""
        self.copies = []


class CacheModel:
    """One request cache: committed length, pending token(s), pages held."""

    def __init__(self, pool: PoolModel, layers: int, capacity: int, page_size: int):
        self.pool = pool
        self.layers = layers
        self.capacity = capacity
        self.page_size = page_size
        self.length = 0
        self.pages = []
        # pending: (position, new pages leased, appended layers, count, copy-on-write
        # (logical page, shared page) or None)
        self.pending = None
        self.retained_lengths = []   # attended length of every committed token
        self.appends = 0

    @property
    def pages_held(self) -> int:
        return len(self.pages)

    def _needs_cow(self) -> bool:
        S = self.page_size
        return self.length % S != 0 and self.pool.refs[self.pages[self.length // S]] > 1

    def _pages_for(self, count: int) -> int:
        S = self.page_size
        return -(-(self.length + count) // S) - (-(-self.length // S)) + self._needs_cow()

    def _copy_on_write(self):
        """A private copy of the shared, partly filled last page; the hold on
        the shared page stays until the copy can no longer be undone."""
        lp = self.length // self.page_size
        old = self.pages[lp]
        new = self.pool.lease()
        self.pool.copies.append((old, new))
        self.pages[lp] = new
        return (lp, old)

    def begin(self, count: int = 1) -> Status:
        if count < 1:
            return Status.INVALID_ARGUMENT
        if self.pending is not None:
            return Status.BAD_STATE
        if self.length + count > self.capacity:
            return Status.CAPACITY_EXHAUSTED
        if self._pages_for(count) > self.pool.free:
            return Status.OUT_OF_PAGES
        cow = self._copy_on_write() if self._needs_cow() else None
        new_pages = -(-(self.length + count) // self.page_size) - len(self.pages)
        for _ in range(new_pages):
            self.pages.append(self.pool.lease())
        self.pending = (self.length, new_pages, set(), count, cow)
        return Status.OK

    def append(self, layer: int) -> Status:
        if not 0 <= layer < self.layers:
            return Status.INVALID_ARGUMENT
        if self.pending is None:
            return Status.BAD_STATE
        if layer in self.pending[2]:
            return Status.BAD_STATE
        self.pending[2].add(layer)
        self.pool.flush()
        return Status.OK

    def commit(self) -> Status:
        if self.pending is None or len(self.pending[2]) != self.layers:
            return Status.BAD_STATE
        for _ in range(self.pending[3]):
            self.length += 1
            self.retained_lengths.append(self.length)
            self.appends += self.layers
        if self.pending[4] is not None:
            self.pool.release(self.pending[4][1])
        self.pending = None
        return Status.OK

    def abort(self) -> Status:
        if self.pending is None:
            return Status.BAD_STATE
        for _ in range(self.pending[1]):
            self.pool.release(self.pages.pop())
        cow = self.pending[4]
        if cow is not None:
            lp, old = cow
            copy = self.pages[lp]
            self.pages[lp] = old
            self.pool.release(copy)
        self.pending = None
        return Status.OK

    def grow(self, n: int) -> Status:
        """Committed rows the caller writes itself; a shared last page is
        copied (and every queued copy enqueued) before the rows are written."""
        if n < 0:
            return Status.INVALID_ARGUMENT
        if self.pending is not None:
            return Status.BAD_STATE
        if self.length + n > self.capacity:
            return Status.CAPACITY_EXHAUSTED
        cow = n > 0 and self._needs_cow()
        need = -(-(self.length + n) // self.page_size) - len(self.pages)
        if need + cow > self.pool.free:
            return Status.OUT_OF_PAGES
        if cow:
            _, old = self._copy_on_write()
            self.pool.flush()
            self.pool.release(old)
        for _ in range(need):
            self.pages.append(self.pool.lease())
        self.length += n
        return Status.OK

    def fork(self, n: int, capacity: int):
        """(status, new cache sharing the first n rows' pages)."""
        if self.pending is not None:
            return Status.BAD_STATE, None
        if not 0 <= n <= self.length or capacity < n:
            return Status.INVALID_ARGUMENT, None
        other = CacheModel(self.pool, self.layers, capacity, self.page_size)
        other.pages = self.pages[:-(-n // self.page_size)]
        for page in other.pages:
            self.pool.hold(page)
        other.length = n
        return Status.OK, other

    def reset(self) -> Status:
        if self.pending is not None:
            return Status.BAD_STATE
        while self.pages:
            self.pool.release(self.pages.pop())
        self.length = 0
        return Status.OK

    def destroy(self) -> Status:
        if self.pending is not None and self.pending[4] is not None:
            self.pool.release(self.pending[4][1])
        while self.pages:
            self.pool.release(self.pages.pop())
        self.length = 0
        self.pending = None
        return Status.OK
