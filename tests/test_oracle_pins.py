"""Pins of the CPU oracle against facts other than itself (CPU only).

Each test names what fixes the expected value: a library routine the oracle
does not use, a closed form, an invariant the pages state, or a count the
pages print (fixtures under tests/golden/ with their citations).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import Status

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(20261202)


def _sdpa_f64(q, K, V, causal=False):
    """torch's CPU float64 scaled-dot-product attention (not used by the oracle)."""
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64))
    Kt = torch.from_numpy(np.ascontiguousarray(K, dtype=np.float64))
    Vt = torch.from_numpy(np.ascontiguousarray(V, dtype=np.float64))
    if qt.dim() == 1:
        qt = qt[None, :]
    out = torch.nn.functional.scaled_dot_product_attention(
        qt[None, None], Kt[None, None], Vt[None, None], is_causal=causal)
    return out[0, 0].numpy()


@pytest.mark.parametrize("t,d", [(1, 2), (2, 2), (37, 2), (100, 64), (513, 128)])
def test_attend_matches_library_sdpa(t, d):
    q = RNG.standard_normal(d)
    K = RNG.standard_normal((t, d))
    V = RNG.standard_normal((t, d))
    got = oracle.attend(q, K, V)
    ref = _sdpa_f64(q, K, V)[0]
    assert np.max(np.abs(got - ref)) < 1e-12


@pytest.mark.parametrize("t,d", [(1, 2), (3, 2), (4, 2), (64, 64), (300, 128)])
def test_decode_is_newest_row_of_causal_attention(t, d):
    # Cached newest-query result equals the last row of the complete-prefix
    # (full causal) computation within the pages' 2e-12 bound.
    with open(os.path.join(GOLDEN, "ch38_fixture_counts.json")) as f:
        bound = json.load(f)["max_abs_diff_bound"]
    Q = RNG.standard_normal((t, d))
    K = RNG.standard_normal((t, d))
    V = RNG.standard_normal((t, d))
    full = oracle.causal_attention(Q, K, V)
    assert np.max(np.abs(oracle.attend(Q[-1], K, V) - full[-1])) <= bound
    # the causal routine itself against the library's causal attention
    assert np.max(np.abs(full - _sdpa_f64(Q, K, V, causal=True))) < 1e-12


def test_single_row_returns_its_value_exactly():
    v = RNG.standard_normal((1, 8))
    out = oracle.attend(RNG.standard_normal(8), RNG.standard_normal((1, 8)), v)
    assert np.array_equal(out, v[0])


def test_zero_query_and_equal_keys_give_mean_value():
    V = RNG.standard_normal((50, 16))
    K = RNG.standard_normal((50, 16))
    assert np.max(np.abs(oracle.attend(np.zeros(16), K, V) - V.mean(axis=0))) < 1e-14
    Keq = np.tile(RNG.standard_normal(16), (50, 1))
    assert np.max(np.abs(oracle.attend(RNG.standard_normal(16), Keq, V) - V.mean(axis=0))) < 1e-14


@pytest.mark.parametrize("a", [-3.0, 0.5, 2.0, 7.0])
def test_two_row_closed_form(a):
    # d=2, q=(a,0), k0=(0,0), k1=(1,0): scores 0 and a/sqrt(2), so
    # p1 = 1/(1+exp(-a/sqrt(2))) and out = (1-p1) v0 + p1 v1.
    q = np.array([a, 0.0])
    K = np.array([[0.0, 0.0], [1.0, 0.0]])
    V = np.array([[1.0, -2.0], [5.0, 3.0]])
    p1 = 1.0 / (1.0 + math.exp(-a / math.sqrt(2.0)))
    ref = (1 - p1) * V[0] + p1 * V[1]
    assert np.max(np.abs(oracle.attend(q, K, V) - ref)) < 1e-15


def test_dominant_score_is_stable():
    d = 64
    K = RNG.standard_normal((200, d))
    V = RNG.standard_normal((200, d))
    q = K[123] * 1e4   # scores of order 1e5: naive exp would overflow
    out = oracle.attend(q, K, V)
    assert np.all(np.isfinite(out))
    assert np.max(np.abs(out - V[123])) < 1e-12


def test_bf16_bits_widen_exactly():
    bits = np.array([0x3F80, 0xC040, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16)
    got = oracle.kv_to_f64(bits)
    assert got[0] == 1.0 and got[1] == -3.0
    assert got[2] == 2.0 ** -133
    assert got[3] == float(np.float32(3.3895313892515355e38))
    assert got[4] == 0.0 and math.copysign(1.0, got[4]) == -1.0


def _coordinate_pool(P, H, S, D):
    # value encodes (page, head, slot, dim): any transposed index shows up
    p, h, s, d = np.meshgrid(np.arange(P), np.arange(H), np.arange(S), np.arange(D),
                             indexing="ij")
    return (1_000_000 * p + 10_000 * h + 100 * s + d).astype(np.float64)


def test_gather_follows_page_table_layout():
    P, H, S, D = 9, 3, 4, 5
    pool = _coordinate_pool(P, H, S, D)
    pt = np.array([7, 2, 5])
    t = 10
    rows = oracle.gather_prefix(pool, pt, t, S, head=1)
    for j in range(t):
        page, slot = pt[j // S], j % S
        assert rows[j].tolist() == [1_000_000 * page + 10_000 * 1 + 100 * slot + d
                                    for d in range(D)]


def _scatter(rows, page_size, page_table, num_pages):
    """Place logical rows [H, t, D] into pages per the page table."""
    H, t, D = rows.shape
    pool = np.full((num_pages, H, page_size, D), np.nan)
    for j in range(t):
        pool[page_table[j // page_size], :, j % page_size, :] = rows[:, j, :]
    return pool


@pytest.mark.parametrize("page_size", [1, 2, 3, 16])
def test_contiguous_and_paged_are_bit_identical(page_size):
    H, D, t, C = 2, 8, 45, 64
    K = RNG.standard_normal((H, t, D))
    V = RNG.standard_normal((H, t, D))
    q = RNG.standard_normal((H, D))
    # contiguous strategy: one page as long as the maximum context
    ref = oracle.paged_decode_attention(q, _scatter(K, C, [0], 1), _scatter(V, C, [0], 1),
                                        [0], t, C)
    npages = -(-t // page_size)
    P = npages + 5
    for trial in range(3):
        pt = RNG.permutation(P)[:npages]
        got = oracle.paged_decode_attention(q, _scatter(K, page_size, pt, P),
                                            _scatter(V, page_size, pt, P), pt, t, page_size)
        assert np.array_equal(got, ref)


def test_split_merge_equals_unsplit():
    d, t = 128, 1000
    q = RNG.standard_normal(d)
    K = RNG.standard_normal((t, d)) * 3
    V = RNG.standard_normal((t, d))
    ref = oracle.attend(q, K, V)
    for bounds in ([(0, t)], [(0, 1), (1, t)], [(0, 333), (333, 334), (334, 1000)],
                   [(i, min(t, i + 16)) for i in range(0, t, 16)]):
        got = oracle.merge_partials(oracle.split_partials(q, K, V, bounds))
        assert np.max(np.abs(got - ref)) < 1e-12


def test_append_and_attend_equals_write_then_attend():
    H, D, S, P, length = 3, 4, 16, 6, 21
    kp = RNG.standard_normal((P, H, S, D))
    vp = RNG.standard_normal((P, H, S, D))
    pt = np.array([4, 1])
    q, kn, vn = (RNG.standard_normal((H, D)) for _ in range(3))
    got = oracle.append_and_attend(q, kn, vn, kp, vp, pt, length, S)
    kp2, vp2 = kp.copy(), vp.copy()
    kp2[pt[length // S], :, length % S, :] = kn
    vp2[pt[length // S], :, length % S, :] = vn
    ref = oracle.paged_decode_attention(q, kp2, vp2, pt, length + 1, S)
    assert np.array_equal(got, ref)
    # length 0: the query attends to the candidate row alone
    assert np.array_equal(oracle.append_and_attend(q, kn, vn, kp, vp, pt, 0, S), vn)


def test_pages_printed_counts():
    with open(os.path.join(GOLDEN, "ch38_fixture_counts.json")) as f:
        g = json.load(f)
    fx = g["fixture"]
    lanes = fx["batch"] * fx["layers"] * fx["heads"]
    assert lanes == g["lanes"]
    cached = oracle.cached_score_cells(lanes, g["cached_retained_lengths"])
    full = oracle.complete_prefix_score_cells(lanes, g["complete_prefix_lengths"])
    assert (cached, full, full - cached) == (g["cached_scores"], g["complete_prefix_scores"],
                                            g["avoided_scores"])
    for phase in ("prefill", "decode"):
        ph = g[phase]
        assert oracle.cached_score_cells(lanes, ph["retained_lengths"]) == ph["cached_scores"]
        assert oracle.complete_prefix_score_cells(
            lanes, [ph["complete_prefix_length"]]) == ph["complete_prefix_scores"]
    assert oracle.qkv_projection_rows(fx["layers"], g["token_rows"]) == g["qkv_rows"]
    ld = g["loaded"]
    assert oracle.cached_score_cells(ld["lanes"], ld["prefixes"]) == ld["cached_scores"]
    assert oracle.complete_prefix_score_cells(ld["lanes"], ld["prefixes"]) == \
        ld["complete_prefix_scores"]


def test_kv_bytes_formula():
    with open(os.path.join(GOLDEN, "kv_bytes_formula.json")) as f:
        g = json.load(f)
    assert oracle.kv_cache_bytes(g["layers"], g["heads"], g["head_width"], g["positions"],
                                 g["scalar_bytes"]) == g["bytes"] == 1 << 30


def test_transaction_model_fixture_schedule():
    # Tiny fixture: 2 layers, capacity 4, 16-token pages, 8-page pool.
    pool = oracle.PoolModel(8)
    c = oracle.CacheModel(pool, layers=2, capacity=4, page_size=16)
    with open(os.path.join(GOLDEN, "ch38_fixture_counts.json")) as f:
        g = json.load(f)
    for _ in range(3):                      # prompt of two rows, one decoded row
        assert c.begin() == Status.OK
        assert c.append(0) == Status.OK and c.append(1) == Status.OK
        assert c.commit() == Status.OK
    assert c.appends == g["cache_appends"]
    assert oracle.cached_score_cells(g["lanes"], c.retained_lengths) == g["cached_scores"]
    assert pool.leased == 1                 # one 16-token page holds 3 rows
    assert c.begin() == Status.OK and c.append(0) == Status.OK and c.append(1) == Status.OK
    assert c.commit() == Status.OK and c.length == 4
    # capacity exhaustion is reported, not handled, and changes nothing
    assert c.begin() == Status.CAPACITY_EXHAUSTED and c.length == 4 and pool.leased == 1


def test_transaction_model_abort_and_rejections():
    pool = oracle.PoolModel(2)
    c = oracle.CacheModel(pool, layers=3, capacity=100, page_size=4)
    assert c.commit() == Status.BAD_STATE and c.abort() == Status.BAD_STATE
    assert c.begin() == Status.OK and pool.leased == 1
    assert c.begin() == Status.BAD_STATE
    assert c.append(3) == Status.INVALID_ARGUMENT
    assert c.append(0) == Status.OK and c.append(0) == Status.BAD_STATE
    assert c.commit() == Status.BAD_STATE          # layers 1, 2 missing
    assert c.reset() == Status.BAD_STATE
    assert c.abort() == Status.OK and c.length == 0 and pool.leased == 0
    for _ in range(8):
        assert c.begin() == Status.OK
        for layer in range(3):
            assert c.append(layer) == Status.OK
        assert c.commit() == Status.OK
    assert pool.leased == 2 and c.begin() == Status.OUT_OF_PAGES and c.length == 8
    assert c.reset() == Status.OK and pool.leased == 0 and c.length == 0


@pytest.mark.parametrize("H,Hkv", [(4, 1), (8, 2), (8, 4), (6, 6)])
def test_grouped_kv_heads_match_library_gqa(H, Hkv):
    # torch's SDPA with enable_gqa (not used by the oracle) shares K/V head
    # h // (H / Hkv) among consecutive query heads.
    D, t, S = 16, 45, 16
    npg = -(-t // S)
    q = RNG.standard_normal((H, D))
    K = RNG.standard_normal((Hkv, t, D))
    V = RNG.standard_normal((Hkv, t, D))
    pt = RNG.permutation(npg + 3)[:npg]
    kp, vp = _scatter(K, S, pt, npg + 3), _scatter(V, S, pt, npg + 3)
    got = oracle.paged_decode_attention(q, kp, vp, pt, t, S, num_kv_heads=Hkv)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], torch.from_numpy(K)[None], torch.from_numpy(V)[None],
        enable_gqa=True)[0, :, 0, :].numpy()
    assert np.max(np.abs(got - ref)) < 1e-12
    # the same result as multi-head attention over K/V heads repeated per group
    rep = np.repeat(np.arange(Hkv), H // Hkv)
    full = oracle.paged_decode_attention(q, _scatter(K[rep], S, pt, npg + 3),
                                         _scatter(V[rep], S, pt, npg + 3), pt, t, S)
    assert np.array_equal(got, full)
    # append-then-attend with shared new rows equals writing them then attending
    kn, vn = RNG.standard_normal((Hkv, D)), RNG.standard_normal((Hkv, D))
    got_a = oracle.append_and_attend(q, kn, vn, kp, vp, pt, t - 1, S)
    kp2, vp2 = kp.copy(), vp.copy()
    kp2[pt[(t - 1) // S], :, (t - 1) % S, :] = kn
    vp2[pt[(t - 1) // S], :, (t - 1) % S, :] = vn
    assert np.array_equal(got_a, oracle.paged_decode_attention(q, kp2, vp2, pt, t, S,
                                                               num_kv_heads=Hkv))


@pytest.mark.parametrize("start,n,H,Hkv,S", [(0, 1, 2, 2, 16), (0, 37, 2, 2, 16), (5, 20, 4, 2, 4),
                                            (33, 17, 3, 1, 16), (16, 16, 2, 2, 16)])
def test_prefill_matches_library_masked_attention(start, n, H, Hkv, S):
    # torch's float64 SDPA over the whole sequence with an explicit mask that
    # lets row start+i see rows 0..start+i; the chunk's rows are the last n.
    D, t = 16, start + n
    K = RNG.standard_normal((Hkv, t, D))
    V = RNG.standard_normal((Hkv, t, D))
    q = RNG.standard_normal((n, H, D))
    npg = -(-t // S) + 2
    pt = RNG.permutation(npg + 4)[:npg]
    kp = _scatter(K[:, :start], S, pt, npg + 4) if start else np.zeros((npg + 4, Hkv, S, D))
    vp = _scatter(V[:, :start], S, pt, npg + 4) if start else np.zeros((npg + 4, Hkv, S, D))
    got = oracle.prefill_attention(q, K[:, start:].transpose(1, 0, 2), V[:, start:].transpose(1, 0, 2),
                                   kp, vp, pt, start, S)
    allowed = torch.from_numpy(np.arange(t)[None, :] <= (start + np.arange(n))[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.transpose(1, 0, 2))[None], torch.from_numpy(K)[None],
        torch.from_numpy(V)[None], attn_mask=allowed, enable_gqa=True)[0].numpy()
    assert np.max(np.abs(got - ref.transpose(1, 0, 2))) < 1e-12
    if start == 0 and H == Hkv:
        # no prefix: the complete-prefix computation of every row
        for h in range(H):
            assert np.max(np.abs(got[:, h] - oracle.causal_attention(q[:, h], K[h], V[h]))) < 1e-12


def test_prefill_of_one_row_is_append_and_attend():
    H, D, S, P, start = 2, 8, 4, 9, 10
    kp = RNG.standard_normal((P, H, S, D))
    vp = RNG.standard_normal((P, H, S, D))
    pt = np.array([3, 7, 1])
    q, kn, vn = (RNG.standard_normal((1, H, D)) for _ in range(3))
    got = oracle.prefill_attention(q, kn, vn, kp, vp, pt, start, S)
    assert np.array_equal(got[0], oracle.append_and_attend(q[0], kn[0], vn[0], kp, vp, pt, start, S))


def test_chunk_transaction_equals_token_steps():
    # A committed chunk of n positions leaves the same visible state as n
    # committed single-token transactions (the reading of a chunked begin).
    for n in (1, 3, 4, 5, 9):
        chunk_pool, step_pool = oracle.PoolModel(10), oracle.PoolModel(10)
        chunk = oracle.CacheModel(chunk_pool, 2, 40, 4)
        steps = oracle.CacheModel(step_pool, 2, 40, 4)
        for m, counts in ((chunk, [2, n]), (steps, [1] * (2 + n))):
            for c in counts:
                assert m.begin(c) == Status.OK
                for layer in range(2):
                    assert m.append(layer) == Status.OK
                assert m.commit() == Status.OK
        assert chunk.length == steps.length == 2 + n
        assert chunk.retained_lengths == steps.retained_lengths
        assert chunk.appends == steps.appends and chunk_pool.free == step_pool.free
    m = oracle.CacheModel(oracle.PoolModel(2), 1, 40, 4)
    assert m.begin(9) == Status.OUT_OF_PAGES and m.begin(41) == Status.CAPACITY_EXHAUSTED
    assert m.begin(0) == Status.INVALID_ARGUMENT and m.pages_held == 0
