"""Random transactional schedules on the GPU against the oracle.

Each schedule drives a small pool through seeded random operations -- cache
create and destroy, single-token and chunk transactions, batched
transactions over several caches, aborts at a random layer, forks at a
random prefix (shared pages, copy on write at the first write into a shared
partly filled page), resets, and the pool or a cache running out -- and
keeps, per cache and layer, the K/V rows its committed history holds.  Every
context a transaction returns is compared with ``oracle.attend`` over that
history plus the transaction's own rows (causal within a chunk); every ten
operations, and at the end, rows of every cache are read back from the pool
at the positions its page table gives and must equal the history bit for
bit.  The pool storage starts as NaN, so a read of any row outside a cache's
history would show.  Calls refused for lack of pages or capacity must leave
the history unchanged.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_attention_amd as pkv
from tests.gpu_support import record_err

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
L = 2
CONTEXT = 256
# dtype, d_h, query heads, K/V heads, page size, pages
CONFIGS = [("bf16", 128, 4, 2, 16, 64), ("f32", 64, 4, 4, 16, 48), ("bf16", 64, 8, 1, 16, 64),
           ("f32", 40, 6, 3, 16, 48), ("bf16", 128, 4, 4, 5, 200), ("f32", 64, 4, 2, 32, 32),
           ("bf16", 256, 2, 1, 16, 64), ("f32", 32, 16, 2, 16, 64)]


def _rows(rng, shape, dtype):
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32))
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def _expected(q, ks, vs, H, Hkv):
    """[H, D] context of one query row over rows ks, vs [t, Hkv, D]."""
    return np.stack([oracle.attend(q[h], ks[:, oracle.kv_head_of(h, H, Hkv)],
                                   vs[:, oracle.kv_head_of(h, H, Hkv)]) for h in range(H)])


class Schedule:
    def __init__(self, seed, dtype, D, H, Hkv, S, P):
        self.rng = np.random.default_rng(seed)
        self.dtype, self.D, self.H, self.Hkv, self.S = dtype, D, H, Hkv, S
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.kp = torch.full((L, P, Hkv, S, D), float("nan"), dtype=tdt, device="cuda")
        self.vp = torch.full_like(self.kp, float("nan"))
        d = pkv.pkv_pool_desc_init()
        d.num_layers, d.num_heads, d.head_width, d.page_size = L, H, D, S
        d.num_pages, d.max_context, d.max_caches = P, CONTEXT, 8
        d.kv_dtype = pkv.PKV_DTYPE_BF16 if dtype == "bf16" else pkv.PKV_DTYPE_F32
        d.k_storage, d.v_storage, d.free_list_seed = self.kp.data_ptr(), self.vp.data_ptr(), seed
        d.num_kv_heads = Hkv
        d.split_blocks = int(self.rng.choice([0, 1, 2]))
        self.pool = pkv.pkv_pool_create(d)
        pkv.pkv_pool_set_option(self.pool, pkv.PKV_OPT_MERGE_MODE, int(self.rng.choice([0, 1, 2])))
        self.hist = {}    # cache -> per layer list of (k [Hkv, D], v) float64 rows
        self.worst = 0.0
        self.contexts = 0

    def _history(self, c, layer):
        rows = self.hist[c][layer]
        if not rows:
            empty = np.zeros((0, self.Hkv, self.D))
            return empty, empty
        return np.stack([r[0] for r in rows]), np.stack([r[1] for r in rows])

    def check_pool(self, c):
        n = pkv.pkv_cache_size(c)
        assert n == len(self.hist[c][0])
        if n == 0:
            return
        table = pkv.pkv_cache_page_table(c)
        for p in self.rng.integers(0, n, size=min(n, 6)):
            page, slot = table[p // self.S], p % self.S
            for layer in range(L):
                k = self.kp[layer, page, :, slot, :].double().cpu().numpy()
                v = self.vp[layer, page, :, slot, :].double().cpu().numpy()
                assert np.array_equal(k, self.hist[c][layer][p][0]), ("k", layer, p)
                assert np.array_equal(v, self.hist[c][layer][p][1]), ("v", layer, p)

    def transact(self, cs, counts):
        """cs have begun counts[i] positions each: every layer appends and
        attends (some caches abort at a random layer), then the rest commit."""
        rng, H, Hkv, D, dt = self.rng, self.H, self.Hkv, self.D, self.dtype
        abort_at = {c: int(rng.integers(0, L)) if rng.random() < 0.25 else -1 for c in cs}
        rows = {c: [] for c in cs}
        live = list(cs)
        for layer in range(L):
            for c in [c for c in live if abort_at[c] == layer]:
                pkv.pkv_abort_token(c)
                live.remove(c)
            if not live:
                return
            tot = sum(counts[cs.index(c)] for c in live)
            q, k, v = (_rows(rng, (tot, h, D), dt) for h in (H, Hkv, Hkv))
            out = torch.empty((tot, H, D), device="cuda")
            if len(live) == 1 and rng.random() < 0.5:
                pkv.pkv_append_and_attend(live[0], layer, q.cuda(), k.cuda(), v.cuda(), out)
            else:
                pkv.pkv_append_and_attend_batched(live, layer, q.cuda(), k.cuda(), v.cuda(), out)
            torch.cuda.synchronize()
            got = out.cpu().numpy().astype(np.float64)
            q64, k64, v64 = (x.double().numpy() for x in (q, k, v))
            off = 0
            for c in live:
                n = counts[cs.index(c)]
                ks, vs = self._history(c, layer)
                for i in range(n):
                    ref = _expected(q64[off + i], np.concatenate([ks, k64[off:off + i + 1]]),
                                    np.concatenate([vs, v64[off:off + i + 1]]), H, Hkv)
                    err = float(np.max(np.abs(got[off + i] - ref)))
                    self.worst = max(self.worst, err)
                    self.contexts += 1
                    assert err <= TOL[dt], (layer, i, n, err)
                rows[c].append([(k64[off + i], v64[off + i]) for i in range(n)])
                off += n
        for c in live:
            pkv.pkv_commit_token(c)
            for layer in range(L):
                self.hist[c][layer].extend(rows[c][layer])

    def step(self):
        rng = self.rng
        op = rng.choice(["create", "destroy", "token", "chunk", "batched", "fork", "reset"],
                        p=[0.12, 0.05, 0.3, 0.15, 0.2, 0.12, 0.06])
        cs = list(self.hist)
        if op == "create" and len(cs) < 6:
            self.hist[pkv.pkv_cache_create(self.pool, CONTEXT)] = [[] for _ in range(L)]
        elif op == "destroy" and len(cs) > 1:
            c = cs[int(rng.integers(len(cs)))]
            pkv.pkv_cache_destroy(c)
            del self.hist[c]
        elif op in ("token", "chunk") and cs:
            c = cs[int(rng.integers(len(cs)))]
            n = 1 if op == "token" else int(rng.integers(2, 24))
            pos = pkv.pkv_begin_token(c) if n == 1 else pkv.pkv_begin_tokens(c, n)
            assert pos == len(self.hist[c][0])
            self.transact([c], [n])
        elif op == "batched" and len(cs) >= 2:
            k = int(rng.integers(2, len(cs) + 1))
            sel = [cs[i] for i in rng.choice(len(cs), size=k, replace=False)]
            counts = [1] * k if rng.random() < 0.6 else [int(rng.integers(1, 9)) for _ in sel]
            if all(x == 1 for x in counts):
                pkv.pkv_begin_token_batched(sel)
            else:
                pkv.pkv_begin_tokens_batched(sel, counts)
            self.transact(sel, counts)
        elif op == "fork" and cs and len(cs) < 6:
            c = cs[int(rng.integers(len(cs)))]
            p = int(rng.integers(0, len(self.hist[c][0]) + 1))
            f = pkv.pkv_cache_fork(c, p, CONTEXT)
            self.hist[f] = [list(self.hist[c][layer][:p]) for layer in range(L)]
        elif op == "reset" and cs:
            c = cs[int(rng.integers(len(cs)))]
            pkv.pkv_cache_reset(c)
            self.hist[c] = [[] for _ in range(L)]

    def close(self):
        for c in list(self.hist):
            self.check_pool(c)
            pkv.pkv_cache_destroy(c)
        cnt = pkv.pkv_pool_get_counters(self.pool)
        assert cnt.pages_leased == 0
        pkv.pkv_pool_destroy(self.pool)


@pytest.mark.parametrize("seed", range(16))
def test_random_transactional_schedule(seed):
    cfg = CONFIGS[seed % len(CONFIGS)]
    s = Schedule(seed, *cfg)
    for i in range(120):
        before = {c: [len(h) for h in s.hist[c]] for c in s.hist}
        try:
            s.step()
        except pkv.PkvError as e:
            # the pool or a cache ran out: nothing may have changed
            assert e.status in (pkv.PKV_ERR_OUT_OF_PAGES, pkv.PKV_ERR_CAPACITY_EXHAUSTED), str(e)
            assert {c: [len(h) for h in s.hist[c]] for c in s.hist} == before
            for c in s.hist:
                assert pkv.pkv_cache_size(c) == len(s.hist[c][0])
        if i % 10 == 9:
            for c in s.hist:
                s.check_pool(c)
    s.close()
    record_err(f"random schedule {seed} {cfg}: {s.contexts} contexts", s.worst)
