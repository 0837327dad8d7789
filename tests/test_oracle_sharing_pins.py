"""Pins of the oracle's prefix-sharing model (fork, copy on write, grow).

These tests call ``oracle.transaction`` only.  Each schedule's expected state
is worked out by hand from the reading of "Incremental Serving", section
"Current scope" (paged storage alone shares no pages and has no copy-on-write
prefixes; the model adds both): a fork holds the pages of a committed prefix;
full shared pages are never written, since writes go only to positions at or
past the length; the first write into a shared, partly filled page gives the
writer a private copy (a new page, its contents queued for copying) while the
transaction keeps its hold on the shared page; commit drops that hold, abort
drops the copy instead; a page is free when its last holder lets it go, and a
copy queued into a page nobody holds is cancelled.

The model leases page identities in order 0, 1, 2, ..., so every literal page
number below follows from the schedule.
"""
from __future__ import annotations

import random

import pytest

import oracle
from oracle import Status

S = 4          # rows per page in every schedule
P = 10         # pages in the pool
LAYERS = 2


def new_cache(pool, capacity=40):
    return oracle.CacheModel(pool, LAYERS, capacity, S)


def run_token(c, count=1):
    """begin (count positions), every layer, commit."""
    assert c.begin(count) == Status.OK
    for layer in range(LAYERS):
        assert c.append(layer) == Status.OK
    assert c.commit() == Status.OK


def state(pool, *caches):
    return ([(c.length, list(c.pages)) for c in caches], pool.free, pool.shared)


def test_fork_inside_a_page_then_both_write():
    pool = oracle.PoolModel(P)
    a = new_cache(pool)
    assert a.grow(10) == Status.OK                  # rows 0..9: pages 0, 1, 2 (2 rows in 2)
    st, b = a.fork(9, 40)                           # 9 rows: ceil(9/4) = 3 pages, all shared
    assert st == Status.OK
    assert state(pool, a, b) == ([(10, [0, 1, 2]), (9, [0, 1, 2])], 7, 3)
    # b writes position 9, inside shared page 2 (slot 1): private copy 3;
    # the transaction still holds page 2, so it stays shared (a + the hold)
    assert b.begin() == Status.OK
    assert pool.copies == [(2, 3)]
    assert state(pool, a, b) == ([(10, [0, 1, 2]), (9, [0, 1, 3])], 6, 3)
    assert b.append(0) == Status.OK and pool.copies == []   # the copy is enqueued
    assert b.append(1) == Status.OK and b.commit() == Status.OK
    # commit drops the hold: page 2 is a's alone
    assert state(pool, a, b) == ([(10, [0, 1, 2]), (10, [0, 1, 3])], 6, 2)
    # a writes position 10 into page 2, which only it holds now: no copy
    run_token(a)
    assert state(pool, a, b) == ([(11, [0, 1, 2]), (10, [0, 1, 3])], 6, 2)
    assert a.retained_lengths == [11] and b.retained_lengths == [10]


def test_fork_at_a_page_boundary_never_copies():
    pool = oracle.PoolModel(P)
    a = new_cache(pool)
    assert a.grow(8) == Status.OK                   # pages 0, 1, both full
    _, b = a.fork(8, 40)
    assert state(pool, a, b) == ([(8, [0, 1]), (8, [0, 1])], 8, 2)
    run_token(b)                                    # position 8 starts page 2
    run_token(a)                                    # position 8 starts page 3
    assert state(pool, a, b) == ([(9, [0, 1, 3]), (9, [0, 1, 2])], 6, 2)
    assert pool.copies == []


def test_abort_after_the_other_holders_released_the_page():
    pool = oracle.PoolModel(P)
    a = new_cache(pool)
    assert a.grow(6) == Status.OK                   # pages 0, 1 (2 rows in 1)
    _, b = a.fork(6, 40)
    assert b.begin() == Status.OK                   # position 6 in shared page 1: copy 2
    assert state(pool, a, b) == ([(6, [0, 1]), (6, [0, 2])], 7, 2)
    assert a.destroy() == Status.OK                 # a lets go of 1 and 0
    # page 1 is held by b's transaction alone, page 0 by b alone
    assert pool.refs == {0: 1, 1: 1, 2: 1} and pool.shared == 0
    assert b.abort() == Status.OK                   # back to page 1; the copy 2 is freed
    assert state(pool, b) == ([(6, [0, 1])], 8, 0)
    assert pool.refs == {0: 1, 1: 1}
    assert b.destroy() == Status.OK
    assert pool.free == P and pool.refs == {}


def test_grow_into_a_shared_page():
    pool = oracle.PoolModel(P)
    a = new_cache(pool)
    assert a.grow(5) == Status.OK                   # pages 0, 1 (1 row in 1)
    _, b = a.fork(5, 40)
    assert state(pool, a, b) == ([(5, [0, 1]), (5, [0, 1])], 8, 2)
    # b grows by 2 into shared page 1: copy 2 made at once, hold dropped at once
    assert b.grow(2) == Status.OK
    assert pool.copies == []
    assert state(pool, a, b) == ([(5, [0, 1]), (7, [0, 2])], 7, 1)
    # a grows by 4 from position 5: page 1 is its own now, then page 3
    assert a.grow(4) == Status.OK
    assert state(pool, a, b) == ([(9, [0, 1, 3]), (7, [0, 2])], 6, 1)
    # growing by nothing never copies, even on a shared page
    _, c = b.fork(7, 40)
    assert c.grow(0) == Status.OK and pool.copies == [] and pool.free == 6


def test_destroy_with_a_copy_pending_cancels_it():
    pool = oracle.PoolModel(P)
    a = new_cache(pool)
    assert a.grow(3) == Status.OK                   # page 0
    _, b = a.fork(3, 40)
    assert b.begin() == Status.OK                   # position 3 in shared page 0: copy 1
    assert pool.copies == [(0, 1)] and pool.refs == {0: 2, 1: 1}
    assert b.destroy() == Status.OK                 # before any layer ran
    assert pool.copies == [] and pool.refs == {0: 1}
    assert state(pool, a) == ([(3, [0])], 9, 0)


def test_chunk_over_a_shared_page_and_its_abort():
    pool = oracle.PoolModel(P)
    a = new_cache(pool)
    assert a.grow(6) == Status.OK                   # pages 0, 1
    _, b = a.fork(5, 40)                            # rows 0..4: pages 0, 1 (1 row in 1)
    # a chunk of 5 positions 5..9: copy of page 1 (page 2) and one new page 3
    assert b.begin(5) == Status.OK
    assert state(pool, a, b) == ([(6, [0, 1]), (5, [0, 2, 3])], 6, 2)
    assert b.abort() == Status.OK
    assert state(pool, a, b) == ([(6, [0, 1]), (5, [0, 1])], 8, 2)
    # positions 5..33 need the copy plus ceil(34/4) - 2 = 7 new pages: exactly
    # the 8 free ones; positions 5..37 need 1 + 8 = 9 and are refused whole
    assert b.begin(29) == Status.OK and pool.free == 0
    assert b.abort() == Status.OK
    assert b.begin(33) == Status.OUT_OF_PAGES
    assert state(pool, a, b) == ([(6, [0, 1]), (5, [0, 1])], 8, 2)


def test_fork_rejections_change_nothing():
    pool = oracle.PoolModel(P)
    a = new_cache(pool)
    assert a.grow(5) == Status.OK
    assert a.fork(6, 40) == (Status.INVALID_ARGUMENT, None)    # past the length
    assert a.fork(-1, 40) == (Status.INVALID_ARGUMENT, None)
    assert a.fork(4, 3) == (Status.INVALID_ARGUMENT, None)     # capacity below the prefix
    assert a.begin() == Status.OK
    assert a.fork(4, 40) == (Status.BAD_STATE, None)           # token pending
    assert a.abort() == Status.OK
    st, z = a.fork(0, 40)                                      # empty prefix: no pages
    assert st == Status.OK and z.pages == [] and z.length == 0
    assert state(pool, a) == ([(5, [0, 1])], 8, 0)


def _held(caches):
    """Pages held by caches, plus shared pages a pending copy replaced."""
    held = set()
    for c in caches:
        held.update(c.pages)
        if c.pending is not None and c.pending[4] is not None:
            held.add(c.pending[4][1])
    return held


def _refcount(caches, page):
    n = sum(c.pages.count(page) for c in caches)
    n += sum(1 for c in caches if c.pending is not None and c.pending[4] is not None
             and c.pending[4][1] == page)
    return n


@pytest.mark.parametrize("seed", range(6))
def test_random_schedules_keep_the_page_invariants(seed):
    """After every step of a random schedule: free pages plus the distinct
    pages held (by caches or by a pending copy's hold) make the pool; each
    page's count of holders is its number of holders; no cache holds a page
    twice; a queued copy's source is held and its destination is the
    writer's page; a full shared page is never a cache's write target.
    When every cache is gone, every page is free and no copy is queued."""
    rnd = random.Random(700 + seed)
    pool = oracle.PoolModel(24)
    caches = [new_cache(pool, 30)]
    for _ in range(600):
        c = rnd.choice(caches)
        op = rnd.choices(["begin", "chunk", "append", "commit", "abort", "grow", "fork",
                          "destroy", "reset"], weights=[4, 2, 6, 3, 2, 1, 1.5, 0.6, 0.3])[0]
        if op == "begin":
            c.begin()
        elif op == "chunk":
            c.begin(rnd.randrange(1, 7))
        elif op == "append":
            c.append(rnd.randrange(LAYERS))
        elif op == "commit":
            c.commit()
        elif op == "abort":
            c.abort()
        elif op == "grow":
            c.grow(rnd.randrange(0, 6))
        elif op == "fork" and len(caches) < 8:
            st, f = c.fork(rnd.randrange(0, c.length + 1), 30)
            if st == Status.OK:
                caches.append(f)
        elif op == "destroy" and len(caches) > 1:
            c.destroy()
            caches.remove(c)
        elif op == "reset":
            c.reset()
        held = _held(caches)
        assert pool.free + len(held) == 24, op
        assert set(pool.refs) == held
        for page in held:
            assert pool.refs[page] == _refcount(caches, page), (op, page)
        for x in caches:
            assert len(set(x.pages)) == len(x.pages)
            assert len(x.pages) == -(-(x.length + (x.pending[3] if x.pending else 0)) // S)
        for src, dst in pool.copies:
            assert src in held and pool.refs[dst] == 1
            assert any(x.pending is not None and x.pending[4] == (x.pages.index(dst), src)
                       for x in caches if dst in x.pages)
        for x in caches:
            if x.pending is not None:
                first = x.pending[0] // S
                for lp in range(first, len(x.pages)):
                    # every page a pending write lands in is the writer's own
                    assert pool.refs[x.pages[lp]] == 1, (op, lp)
    for x in list(caches):
        x.destroy()
    assert pool.free == 24 and pool.refs == {} and pool.copies == []
