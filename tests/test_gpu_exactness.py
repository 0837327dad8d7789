"""Exact closed forms and poisoned page tails, on every kernel family.

Closed form (learn_llm ch.38, the incremental mixture): with q = 0 every
score is 0, so every weight is exp(0) = 1 -- exactly, also after rounding to
bf16 -- and the context is the plain mean of the value rows.  Value row j of
request r, K/V head g is one-hot at column (j + c[r, g]) mod d_h, so context
element d is exactly count{j < t : (j + c) mod d_h = d} / t.  Every sum is of
small integers (exact in float32), so the only error is the final division:
the bar is 1e-6.  A row dropped or counted twice moves one element by 1/t,
at least 3e-5 here -- far above the bar, where the 2e-2 bar of the random
bf16 checks would hide it.

Poisoned tails ("Incremental Serving", Paged KV-cache layout: a request's
last page is partly filled, and the bytes past its length are whatever the
slot held before): every slot at or past the attended length in each
request's last page holds NaN, +Inf and -Inf bit patterns, in both K and V
(and, for an append, the slot being written holds them until the kernel
writes it).  The rows in range are generator values; every context must be
finite and match the oracle, which never reads those slots.

Families: the vector fast path (one or two query heads per wave, padded
widths), the grouped matrix-core kernels (bf16 and float32, groups of 4 to
32), the generic kernel (other widths and page sizes), split and unsplit,
both merge modes, decode and fused append; and the prefill kernels.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from synth import workloads as W
from tests.gpu_support import (TOL, HostPages, device_pool, max_err, record_err,
                               rows_to_device, to_bits)

pytestmark = pytest.mark.gpu
pkv = pytest.importorskip("paged_kv_cache_attention_amd")

EXACT = 1e-6

FAMILIES = [
    # dtype, d_h, page size, query heads, K/V heads
    ("bf16", 128, 16, 32, 32),   # vector fast path, one query head per wave
    ("bf16", 128, 16, 32, 16),   # two query heads per wave
    ("bf16", 128, 16, 32, 8),    # grouped matrix cores, 4 heads per K/V head
    ("bf16", 128, 16, 32, 4),    # 8
    ("bf16", 128, 16, 32, 2),    # 16
    ("bf16", 128, 16, 32, 1),    # 32: two workgroups of 16 per K/V head
    ("bf16", 64, 16, 8, 2),      # grouped, d_h 64
    ("bf16", 256, 16, 8, 8),     # fast path, 512-byte rows
    ("bf16", 256, 16, 16, 1),    # grouped, d_h 256
    ("bf16", 96, 16, 4, 4),      # padded into the d_h 128 shape
    ("bf16", 100, 16, 2, 2),     # generic kernel: no fast shape
    ("bf16", 128, 8, 4, 1),      # generic kernel: 8-row pages
    ("f32", 64, 16, 12, 12),     # fast path float32
    ("f32", 64, 16, 32, 8),      # grouped float32, 4
    ("f32", 64, 16, 32, 2),      # 16
    ("f32", 128, 16, 32, 1),     # 32
    ("f32", 32, 16, 8, 1),       # 8, d_h 32
    ("f32", 40, 16, 4, 4),       # padded into the d_h 64 shape
    ("f32", 10, 16, 2, 2),       # generic kernel
]
SPLITS = [(0, 2), (2, 0), (2, 2), (-1, 2)]     # (split blocks, merge mode)
CLOSED_LENGTHS = [1, 2, 15, 16, 17, 31, 33, 100, 1000, 4097, 32768]
POISON_LENGTHS = [1, 2, 15, 16, 17, 31, 33, 100, 1000, 4097]

ONE_BITS = {"f32": np.float32(1.0).view(np.int32), "bf16": np.int16(0x3F80)}
# NaN, +Inf, -Inf
POISON_BITS = {"f32": np.array([0x7FC00000, 0x7F800000, -0x800000], dtype=np.int32),
               "bf16": np.array([0x7FC0, 0x7F80, -0x80], dtype=np.int16)}


def _int_view(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int32 if t.element_size() == 4 else torch.int16)


def _workload(name, dtype, D, S, H, Hkv, lengths, seed):
    lengths = np.asarray(lengths, dtype=np.int64)
    P = int(W.pages_needed(lengths, S).sum()) + 3
    w = W.Workload(name, seed, len(lengths), 1, H, D, S, P, dtype, lengths, appends=True,
                   kv_heads=Hkv if Hkv != H else 0)
    return W._finish(w)


def _poison_tails(w, kp, vp, first):
    """Every slot from position first[r] to the end of request r's last page
    gets NaN / +Inf / -Inf patterns (cycling over slot, head and column)."""
    S, D = w.page_size, w.head_width
    bits = torch.from_numpy(POISON_BITS[w.dtype]).cuda()
    pages, slots = [], []
    for r, t in enumerate(w.lengths.tolist()):
        end = -(-t // S) * S
        for pos in range(int(first[r]), end):
            pages.append(int(w.page_tables[r][pos // S]))
            slots.append(pos % S)
    if not pages:
        return 0
    pg = torch.tensor(pages, device="cuda")
    sl = torch.tensor(slots, device="cuda")
    h = torch.arange(w.hkv, device="cuda")
    d = torch.arange(D, device="cuda")
    idx = (sl[:, None, None] + h[None, :, None] + d[None, None, :]) % 3
    pattern = bits[idx]
    for t in (kp, vp):
        _int_view(t)[0][pg[:, None, None], h[None, :, None], sl[:, None, None],
                        d[None, None, :]] = pattern
    return len(pages)


def _one_hot_values(w, vp, upto):
    """V rows 0..upto[r]-1 of every request one-hot at (j + c) mod d_h, where
    c = 7 r + 3 g for K/V head g; everything else in those pages zero."""
    S, D = w.page_size, w.head_width
    _int_view(vp).zero_()
    rows_p, rows_s, rows_h, rows_d = [], [], [], []
    for r in range(w.n):
        j = np.arange(int(upto[r]))
        for g in range(w.hkv):
            rows_p.append(w.page_tables[r][j // S])
            rows_s.append(j % S)
            rows_h.append(np.full(len(j), g))
            rows_d.append((j + 7 * r + 3 * g) % D)
    cat = [torch.from_numpy(np.concatenate(x).astype(np.int64)).cuda()
           for x in (rows_p, rows_s, rows_h, rows_d)]
    _int_view(vp)[0][cat[0], cat[2], cat[1], cat[3]] = int(ONE_BITS[w.dtype])


def _one_hot_row(w, r, j):
    """[H_kv, D] value row j of request r in generator form."""
    row = np.zeros((w.hkv, w.head_width), dtype=np.float32)
    for g in range(w.hkv):
        row[g, (j + 7 * r + 3 * g) % w.head_width] = 1.0
    if w.dtype == "bf16":
        return (row.view(np.uint32) >> 16).astype(np.uint16)
    return row


def _expected_counts(w, r, t):
    """Exact context [H, D] over rows 0..t-1 of request r."""
    G = w.heads // w.hkv
    out = np.zeros((w.heads, w.head_width), dtype=np.float64)
    j = np.arange(t)
    for h in range(w.heads):
        g = h // G
        out[h] = np.bincount((j + 7 * r + 3 * g) % w.head_width, minlength=w.head_width) / t
    return out


def _pool(w, kp, vp, split, merge):
    d = pkv.pkv_pool_desc_init()
    d.num_layers, d.num_heads, d.head_width = 1, w.heads, w.head_width
    d.page_size, d.num_pages = w.page_size, w.num_pages
    d.max_context = w.pt_stride * w.page_size
    d.kv_dtype = pkv.PKV_DTYPE_F32 if w.dtype == "f32" else pkv.PKV_DTYPE_BF16
    d.split_blocks = split
    d.k_storage, d.v_storage = kp.data_ptr(), vp.data_ptr()
    d.num_kv_heads = w.kv_heads
    pool = pkv.pkv_pool_create(d)
    pkv.pkv_pool_set_option(pool, pkv.PKV_OPT_MERGE_MODE, merge)
    return pool


def _name(dtype, D, S, H, Hkv):
    return f"{dtype}_d{D}_s{S}_h{H}_kv{Hkv}"


@pytest.mark.parametrize("dtype,D,S,H,Hkv", FAMILIES)
@pytest.mark.parametrize("split,merge", SPLITS)
@pytest.mark.parametrize("op", ["decode", "append"])
def test_closed_form_counts_catch_a_lost_or_repeated_row(dtype, D, S, H, Hkv, split, merge, op):
    w = _workload("closed_" + _name(dtype, D, S, H, Hkv), dtype, D, S, H, Hkv, CLOSED_LENGTHS,
                  seed=61)
    kp, vp = device_pool(w)                                   # K: generator values
    last = w.lengths - 1
    upto = last if op == "append" else w.lengths
    _one_hot_values(w, vp, upto)
    _poison_tails(w, kp, vp, upto)
    pool = _pool(w, kp, vp, split, merge)
    plan = pkv.pkv_plan_create(pool)
    pkv.pkv_plan_build(plan, w.lengths.tolist(), w.pt_stride)
    if split == 2:
        assert pkv.pkv_plan_num_chunks(plan) > w.n
    q = torch.zeros((w.n, H, D), dtype=kp.dtype, device="cuda")
    out = torch.full((w.n, H, D), float("nan"), device="cuda")
    pt = torch.from_numpy(w.page_tables.copy()).cuda()
    if op == "decode":
        pkv.pkv_plan_decode_attention(plan, 0, q, pt, out)
    else:
        k_new = rows_to_device(w.k_new(0), dtype)
        v_new = rows_to_device(np.stack([_one_hot_row(w, r, int(last[r])) for r in range(w.n)]),
                               dtype)
        pkv.pkv_plan_append_and_attend(plan, 0, pt, q, k_new, v_new, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    worst = 0.0
    for r, t in enumerate(w.lengths.tolist()):
        err = float(np.max(np.abs(got[r] - _expected_counts(w, r, t))))
        worst = max(worst, err)
        assert err <= EXACT, (r, t, err)
    record_err(f"closed form {op} {_name(dtype, D, S, H, Hkv)}", worst)
    pkv.pkv_plan_destroy(plan)
    pkv.pkv_pool_destroy(pool)


@pytest.mark.parametrize("dtype,D,S,H,Hkv", FAMILIES)
@pytest.mark.parametrize("split,merge", SPLITS)
@pytest.mark.parametrize("op", ["decode", "append"])
def test_poisoned_tails_are_never_read(dtype, D, S, H, Hkv, split, merge, op):
    w = _workload("poison_" + _name(dtype, D, S, H, Hkv), dtype, D, S, H, Hkv, POISON_LENGTHS,
                  seed=67)
    kp, vp = device_pool(w)
    last = w.lengths - 1
    first = last if op == "append" else w.lengths
    assert _poison_tails(w, kp, vp, first) > 0
    pool = _pool(w, kp, vp, split, merge)
    plan = pkv.pkv_plan_create(pool)
    pkv.pkv_plan_build(plan, w.lengths.tolist(), w.pt_stride)
    qh = w.q(0)
    out = torch.full((w.n, H, D), float("nan"), device="cuda")
    pt = torch.from_numpy(w.page_tables.copy()).cuda()
    q = rows_to_device(qh, dtype)
    kh, vh = w.k_new(0), w.v_new(0)
    if op == "decode":
        pkv.pkv_plan_decode_attention(plan, 0, q, pt, out)
    else:
        pkv.pkv_plan_append_and_attend(plan, 0, pt, q, rows_to_device(kh, dtype),
                                       rows_to_device(vh, dtype), out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    kpg, vpg = HostPages(w, "k", 0), HostPages(w, "v", 0)
    worst = 0.0
    for r, t in enumerate(w.lengths.tolist()):
        if op == "decode":
            ref = oracle.paged_decode_attention(qh[r], kpg, vpg, w.page_tables[r], t, S,
                                                num_kv_heads=w.hkv)
        else:
            ref = oracle.append_and_attend(qh[r], kh[r], vh[r], kpg, vpg, w.page_tables[r],
                                           t - 1, S)
            page, slot = w.page_tables[r][(t - 1) // S], (t - 1) % S
            assert np.array_equal(to_bits(kp[0, page, :, slot, :], dtype), kh[r])
            assert np.array_equal(to_bits(vp[0, page, :, slot, :], dtype), vh[r])
        err = max_err(out[r], ref)
        worst = max(worst, err)
        assert err <= TOL[dtype], (r, t, err)
    record_err(f"poisoned tails {op} {_name(dtype, D, S, H, Hkv)}", worst)
    pkv.pkv_plan_destroy(plan)
    pkv.pkv_pool_destroy(pool)


LONG_LENGTHS = [200003, 5, 70000, 131072]


@pytest.mark.parametrize("dtype,D,S,H,Hkv", [("bf16", 128, 16, 4, 2), ("f32", 64, 16, 4, 4),
                                             ("bf16", 128, 16, 32, 1)])
@pytest.mark.parametrize("split,merge", [(0, 2), (0, 0), (-1, 2)])
def test_very_long_contexts_closed_form(dtype, D, S, H, Hkv, split, merge):
    """Contexts of up to 200,003 rows beside a short one.  The automatic plan
    cuts the long ones into hundreds of chunks (up to 391 partials merged per
    (request, head)); never splitting runs each on one workgroup.  q = 0 and
    one-hot V rows give exact expected contexts (counts / t), and the slots
    past each request's length hold NaN / Inf patterns."""
    w = _workload("long_" + _name(dtype, D, S, H, Hkv), dtype, D, S, H, Hkv, LONG_LENGTHS,
                  seed=71)
    kp, vp = device_pool(w)
    _one_hot_values(w, vp, w.lengths)
    _poison_tails(w, kp, vp, w.lengths)
    pool = _pool(w, kp, vp, split, merge)
    plan = pkv.pkv_plan_create(pool)
    pkv.pkv_plan_build(plan, w.lengths.tolist(), w.pt_stride)
    chunks = pkv.pkv_plan_num_chunks(plan)
    if split == 0 and H == 4:
        assert chunks > 300
    if split == -1:
        assert chunks == w.n
    q = torch.zeros((w.n, H, D), dtype=kp.dtype, device="cuda")
    out = torch.full((w.n, H, D), float("nan"), device="cuda")
    pt = torch.from_numpy(w.page_tables.copy()).cuda()
    pkv.pkv_plan_decode_attention(plan, 0, q, pt, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    worst = 0.0
    for r, t in enumerate(w.lengths.tolist()):
        err = float(np.max(np.abs(got[r] - _expected_counts(w, r, t))))
        worst = max(worst, err)
        assert err <= EXACT, (r, t, err)
    record_err(f"long contexts {_name(dtype, D, S, H, Hkv)} split {split} merge {merge} "
               f"({chunks} chunks)", worst)
    pkv.pkv_plan_destroy(plan)
    pkv.pkv_pool_destroy(pool)


PREFILL_FAMILIES = [
    ("bf16", 128, 16, 8, 2), ("bf16", 64, 16, 4, 4), ("bf16", 256, 16, 4, 1),
    ("bf16", 128, 32, 4, 4),
    ("f32", 64, 16, 4, 2), ("f32", 32, 16, 4, 4), ("f32", 128, 16, 4, 1),
    ("bf16", 96, 16, 2, 2),      # per-row decode kernels
]
PREFILL_CHUNKS = [(0, 1), (0, 37), (5, 20), (16, 16), (100, 70), (1000, 33), (0, 300),
                  (3000, 1100)]


def _chunk_rows(w, total):
    import synth
    out = []
    for tag, heads in ((synth.TAG_Q, w.heads), (synth.TAG_K, w.hkv), (synth.TAG_V, w.hkv)):
        key = synth.stream_key(w.seed, tag, 0, 1000)
        out.append(synth.normals(key, 0, total * heads * w.head_width, w.dtype).reshape(
            total, heads, w.head_width))
    return tuple(out)


@pytest.mark.parametrize("dtype,D,S,H,Hkv", PREFILL_FAMILIES)
@pytest.mark.parametrize("kind", ["closed", "poison"])
def test_prefill_closed_form_and_poisoned_tails(dtype, D, S, H, Hkv, kind):
    starts = [a for a, _ in PREFILL_CHUNKS]
    counts = [b for _, b in PREFILL_CHUNKS]
    w = _workload(f"prefill_{kind}_" + _name(dtype, D, S, H, Hkv), dtype, D, S, H, Hkv,
                  [a + b for a, b in PREFILL_CHUNKS], seed=71)
    kp, vp = device_pool(w)
    T = sum(counts)
    qh, kh, vh = _chunk_rows(w, T)
    if kind == "closed":
        _one_hot_values(w, vp, starts)
        qh = np.zeros_like(qh)
        vh = np.concatenate([np.stack([_one_hot_row(w, r, st + i) for i in range(n)])
                             for r, (st, n) in enumerate(PREFILL_CHUNKS)])
    _poison_tails(w, kp, vp, starts)          # the chunk's own slots too, until appended
    pool = _pool(w, kp, vp, 0, 2)
    out = torch.full((T, H, D), float("nan"), device="cuda")
    pt = torch.from_numpy(w.page_tables.copy()).cuda()
    pkv.pkv_prefill_attention(pool, 0, pt, w.pt_stride, starts, counts,
                              *(rows_to_device(x, dtype) for x in (qh, kh, vh)), out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    got = out.cpu().numpy().astype(np.float64)
    kpg, vpg = HostPages(w, "k", 0), HostPages(w, "v", 0)
    worst, off = 0.0, 0
    for r, (st, n) in enumerate(PREFILL_CHUNKS):
        sl = slice(off, off + n)
        if kind == "closed":
            ref = np.stack([_expected_counts(w, r, st + i + 1) for i in range(n)])
            bar = EXACT
        else:
            ref = oracle.prefill_attention(qh[sl], kh[sl], vh[sl], kpg, vpg, w.page_tables[r],
                                           st, S)
            bar = TOL[dtype]
        err = float(np.max(np.abs(got[sl] - ref)))
        worst = max(worst, err)
        assert err <= bar, (r, st, n, err)
        off += n
    record_err(f"prefill {kind} {_name(dtype, D, S, H, Hkv)}", worst)
    pkv.pkv_pool_destroy(pool)
