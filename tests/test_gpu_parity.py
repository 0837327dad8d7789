"""GPU parity: the HIP library through its C ABI against the float64 oracle.

Inputs are drawn by ``synth``; the device pools are filled by the generator's
device kernel and the oracle regenerates the same pages on the host.  Bars:
max abs error 1e-5 (float32 K/V) and 2e-2 (bfloat16 K/V, float32
accumulate); page writes bit-exact; page-table permutation and page-size
changes bit-identical on the device.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import workloads as W
from tests.gpu_support import (TOL, GeneratorLayer, HostPages, device_pool, max_err, record_err,
                               rows_to_device, to_bits)

pytestmark = pytest.mark.gpu
pkv = pytest.importorskip("paged_kv_cache_attention_amd")


def _pool(w, kp, vp, split=0, seed=0, max_caches=0, max_context=None, merge=0, flags=0):
    d = pkv.pkv_pool_desc_init()
    d.flags = flags
    d.num_layers, d.num_heads, d.head_width = w.layers, w.heads, w.head_width
    d.page_size, d.num_pages = w.page_size, w.num_pages
    d.max_context = max_context or w.pt_stride * w.page_size
    d.max_caches = max_caches
    d.kv_dtype = pkv.PKV_DTYPE_F32 if w.dtype == "f32" else pkv.PKV_DTYPE_BF16
    d.split_blocks = split
    d.k_storage, d.v_storage = kp.data_ptr(), vp.data_ptr()
    d.free_list_seed = seed
    d.num_kv_heads = w.kv_heads
    pool = pkv.pkv_pool_create(d)
    pkv.pkv_pool_set_option(pool, pkv.PKV_OPT_MERGE_MODE, merge)
    return pool


def _small(name, dtype, D, S, lengths, heads=3, layers=2, seed=17, extra_pages=5, kv_heads=0):
    lengths = np.asarray(lengths, dtype=np.int64)
    P = int(W.pages_needed(lengths, S).sum()) + extra_pages
    w = W.Workload(name, seed, len(lengths), layers, heads, D, S, P, dtype, lengths,
                   appends=True, kv_heads=kv_heads)
    return W._finish(w)


def _oracle_decode(w, layer, r, q_host, appended=None):
    """Oracle context of request r: over the generator pages, or with the
    newest row supplied as a candidate when the step appended it."""
    kp, vp = HostPages(w, "k", layer), HostPages(w, "v", layer)
    t = int(w.lengths[r])
    pt = w.page_tables[r]
    if appended is None:
        return oracle.paged_decode_attention(q_host[r], kp, vp, pt, t, w.page_size,
                                             num_kv_heads=w.hkv)
    k_new, v_new = appended
    return oracle.append_and_attend(q_host[r], k_new[r], v_new[r], kp, vp, pt, t - 1, w.page_size)


def _pt_device(w):
    return torch.from_numpy(w.page_tables.copy()).to("cuda")


# --------------------------------------------------------------- generator --
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_device_fill_matches_host_generator(dtype):
    from synth import gpu as sgpu
    key = synth.stream_key(99, synth.TAG_MISC, 1)
    t = torch.empty(1 << 20, dtype=sgpu.torch_dtype(dtype), device="cuda")
    sgpu.fill_normal(t, key, dtype, start=12345)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(t, dtype), synth.normals(key, 12345, 1 << 20, dtype))


# ------------------------------------------------------------ tiny fixture --
def _tiny_run(page_size, num_pages, seed=3, abort_at=None):
    """Token-at-a-time through begin / append_and_attend x L / commit on one
    request: L=2, H=2, d_h=2, lengths 1..4.  Returns the outputs per step."""
    g = W.tiny_geometry()
    L, H, D, C = g["layers"], g["heads"], g["head_width"], g["max_len"]
    shape = (L, num_pages, H, page_size, D)
    kp = torch.full(shape, float("nan"), device="cuda")
    vp = torch.full(shape, float("nan"), device="cuda")
    d = pkv.pkv_pool_desc_init()
    d.num_layers, d.num_heads, d.head_width = L, H, D
    d.page_size, d.num_pages, d.max_context = page_size, num_pages, C
    d.k_storage, d.v_storage, d.free_list_seed = kp.data_ptr(), vp.data_ptr(), seed
    pool = pkv.pkv_pool_create(d)
    cache = pkv.pkv_cache_create(pool, C)
    hist_k = np.zeros((L, 1, H, C, D), dtype=np.float32)   # contiguous strategy
    hist_v = np.zeros((L, 1, H, C, D), dtype=np.float32)
    outs = []
    for pos in range(C):
        for attempt in range(2 if abort_at == pos else 1):
            assert pkv.pkv_begin_token(cache) == pos
            step_out = []
            layers = range(L) if attempt == 1 or abort_at != pos else range(1)
            for layer in layers:
                # the aborted attempt uses different rows than the retried one
                qh, kh, vh = W.tiny_rows(g["seed"] + 100 * (attempt == 0 and abort_at == pos),
                                         layer, pos, H, D)
                q, k, v = (rows_to_device(x, "f32") for x in (qh, kh, vh))
                out = torch.empty((H, D), device="cuda")
                pkv.pkv_append_and_attend(cache, layer, q, k, v, out)
                torch.cuda.synchronize()
                step_out.append(out.cpu().numpy().copy())
                if attempt == 0 and abort_at == pos:
                    continue
                ref = oracle.append_and_attend(qh, kh, vh, hist_k[layer], hist_v[layer], [0],
                                               pos, C)
                assert max_err(out, ref) <= TOL["f32"]
                pt = pkv.pkv_cache_page_table(cache)
                page, slot = pt[pos // page_size], pos % page_size
                assert np.array_equal(to_bits(kp[layer, page, :, slot, :], "f32"), kh)
                assert np.array_equal(to_bits(vp[layer, page, :, slot, :], "f32"), vh)
                hist_k[layer, 0, :, pos, :] = kh
                hist_v[layer, 0, :, pos, :] = vh
            if attempt == 0 and abort_at == pos:
                pkv.pkv_abort_token(cache)
                assert pkv.pkv_cache_size(cache) == pos
                continue
            pkv.pkv_commit_token(cache)
            outs.append(np.stack(step_out))
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_begin_token(cache)
    assert e.value.status == pkv.PKV_ERR_CAPACITY_EXHAUSTED
    cnt = pkv.pkv_pool_get_counters(pool)
    assert cnt.cache_appends == L * C and cnt.score_cells == L * H * sum(range(1, C + 1))
    pkv.pkv_cache_destroy(cache)
    pkv.pkv_pool_destroy(pool)
    return outs


def test_tiny_fixture_transactions():
    base = _tiny_run(16, 8)
    assert len(base) == 4 and base[0].shape == (2, 2, 2)
    # lengths 1: the context is the newest value row itself, exactly
    for layer in range(2):
        _, _, vh = W.tiny_rows(W.tiny_geometry()["seed"], layer, 0, 2, 2)
        assert np.array_equal(base[0][layer], vh)
    # page size 1 and 2 (rows cross pages), and the contiguous strategy (one
    # page of the full context): bit-identical on the device
    for S, P in ((1, 8), (2, 8), (4, 2)):
        other = _tiny_run(S, P, seed=S + 7)
        for a, b in zip(base, other):
            assert np.array_equal(a, b), f"page size {S} differs"
    # an aborted token leaves no trace: the retried step equals the plain run
    aborted = _tiny_run(16, 8, abort_at=2)
    for a, b in zip(base, aborted):
        assert np.array_equal(a, b)


# -------------------------------------------------------- batched, small --
SMALL_CASES = [
    # fast path: rows of 256 bytes ...
    ("f32", 64, 16), ("bf16", 128, 16), ("bf16", 128, 32),
    # ... 128 and 512 bytes
    ("bf16", 64, 16), ("f32", 32, 16), ("bf16", 256, 16), ("f32", 128, 32),
    # ... and narrower rows padded to those (lanes past the row end idle)
    ("bf16", 96, 16), ("bf16", 80, 32), ("bf16", 48, 16), ("f32", 40, 16), ("f32", 96, 16),
    # generic path: other widths, page sizes that are not a multiple of 16
    ("bf16", 100, 16), ("f32", 10, 16), ("f32", 64, 5), ("bf16", 128, 7),
]
FAST_WIDTHS = {("f32", 32), ("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128), ("bf16", 256),
               ("bf16", 96), ("f32", 40)}
LENGTHS = [1, 15, 16, 17, 100, 333, 1000]


MERGES = [pkv.PKV_MERGE_SEPARATE, pkv.PKV_MERGE_LAST_ARRIVER]


@pytest.mark.parametrize("dtype,D,S", SMALL_CASES)
@pytest.mark.parametrize("split,merge", [(0, 0), (2, 0), (2, 2), (-1, 0)])
def test_batched_decode_small(dtype, D, S, split, merge):
    w = _small(f"small_{dtype}_{D}_{S}", dtype, D, S, LENGTHS)
    kp, vp = device_pool(w)
    pool = _pool(w, kp, vp, split=split, merge=merge)
    plan = pkv.pkv_plan_create(pool)
    pkv.pkv_plan_build(plan, w.lengths.tolist(), w.pt_stride)
    if split == 2:
        assert pkv.pkv_plan_num_chunks(plan) > w.n
    pt = _pt_device(w)
    for layer in range(w.layers):
        qh = w.q(layer)
        q = rows_to_device(qh, dtype)
        out = torch.empty((w.n, w.heads, D), device="cuda")
        pkv.pkv_plan_decode_attention(plan, layer, q, pt, out)
        torch.cuda.synchronize()
        for r in range(w.n):
            ref = _oracle_decode(w, layer, r, qh)
            assert max_err(out[r], ref) <= TOL[dtype], (layer, r, int(w.lengths[r]))
    pkv.pkv_plan_destroy(plan)
    pkv.pkv_pool_destroy(pool)


@pytest.mark.parametrize("dtype,D,S", [c for c in SMALL_CASES if (c[0], c[1]) in FAST_WIDTHS
                                        and c[2] % 16 == 0])
@pytest.mark.parametrize("split,merge", [(0, 2), (2, 2), (2, 0), (-1, 2)])
@pytest.mark.parametrize("waves", [8, 16])
def test_eight_and_sixteen_wave_workgroups(dtype, D, S, split, merge, waves):
    """Multi-head workgroups of eight and of sixteen waves (sixteen runs for
    d_h <= 64; wider rows take eight), unsplit and split, both merge modes."""
    w = _small(f"w8_{dtype}_{D}_{S}", dtype, D, S, LENGTHS, seed=29)
    kp, vp = device_pool(w)
    pool = _pool(w, kp, vp, split=split, merge=merge)
    pkv.pkv_pool_set_option(pool, pkv.PKV_OPT_WAVES, waves)
    plan = pkv.pkv_plan_create(pool)
    pkv.pkv_plan_build(plan, w.lengths.tolist(), w.pt_stride)
    pt = _pt_device(w)
    layer = 1
    qh, kh, vh = w.q(layer), w.k_new(layer), w.v_new(layer)
    q, k, v = (rows_to_device(x, dtype) for x in (qh, kh, vh))
    out = torch.empty((w.n, w.heads, D), device="cuda")
    pkv.pkv_plan_append_and_attend(plan, layer, pt, q, k, v, out)
    torch.cuda.synchronize()
    for r in range(w.n):
        ref = _oracle_decode(w, layer, r, qh, appended=(kh, vh))
        assert max_err(out[r], ref) <= TOL[dtype], (r, int(w.lengths[r]))
    pkv.pkv_plan_destroy(plan)
    pkv.pkv_pool_destroy(pool)


@pytest.mark.parametrize("dtype,D,S", SMALL_CASES)
@pytest.mark.parametrize("merge", MERGES)
def test_append_and_attend_small(dtype, D, S, merge):
    w = _small(f"append_{dtype}_{D}_{S}", dtype, D, S, LENGTHS, seed=23)
    kp, vp = device_pool(w)
    pool = _pool(w, kp, vp, split=2, merge=merge)
    plan = pkv.pkv_plan_create(pool)
    pkv.pkv_plan_build(plan, w.lengths.tolist(), w.pt_stride)
    pt = _pt_device(w)
    layer = 1
    qh, kh, vh = w.q(layer), w.k_new(layer), w.v_new(layer)
    q, k, v = (rows_to_device(x, dtype) for x in (qh, kh, vh))
    out = torch.empty((w.n, w.heads, D), device="cuda")
    pkv.pkv_plan_append_and_attend(plan, layer, pt, q, k, v, out)
    torch.cuda.synchronize()
    for r in range(w.n):
        t = int(w.lengths[r])
        page, slot = w.page_tables[r][(t - 1) // S], (t - 1) % S
        assert np.array_equal(to_bits(kp[layer, page, :, slot, :], dtype), kh[r])
        assert np.array_equal(to_bits(vp[layer, page, :, slot, :], dtype), vh[r])
        ref = _oracle_decode(w, layer, r, qh, appended=(kh, vh))
        assert max_err(out[r], ref) <= TOL[dtype], (r, t)
    # the unfused pair (append, then attend) gives bit-identical contexts
    kp2, vp2 = device_pool(w, layers=[layer])
    pool2 = _pool(w, kp2, vp2, split=2, merge=merge)
    pkv.pkv_kv_append(pool2, layer, pt, w.pt_stride, (w.lengths - 1).tolist(), k, v)
    out2 = torch.empty_like(out)
    pkv.pkv_decode_attention(pool2, layer, q, pt, w.pt_stride, w.lengths.tolist(), out2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    assert torch.equal(kp[layer], kp2[layer]) and torch.equal(vp[layer], vp2[layer])
    pkv.pkv_plan_destroy(plan)
    pkv.pkv_pool_destroy(pool)
    pkv.pkv_pool_destroy(pool2)


# ------------------------------------------------- grouped K/V heads --
GQA_CASES = [
    # dtype, D, S, H, H_kv: the fast kernels, one workgroup per K/V head for
    # groups of 2, 4, 8 and 16 ...
    ("bf16", 128, 16, 8, 4), ("bf16", 128, 16, 8, 2), ("bf16", 128, 32, 16, 2),
    ("bf16", 128, 16, 16, 1), ("f32", 64, 16, 4, 2), ("f32", 64, 16, 8, 1),
    ("f32", 64, 16, 16, 2),
    # ... several per K/V head: one K/V head under 32 query heads (16 per
    # workgroup), groups of 12 and 24 (4 and 8 per workgroup), 6 and 3 ...
    ("bf16", 128, 16, 32, 1), ("bf16", 128, 16, 24, 2), ("bf16", 128, 16, 12, 1),
    ("bf16", 128, 16, 6, 1), ("f32", 64, 16, 32, 1), ("f32", 64, 16, 6, 2),
    # ... rows of 128 and 512 bytes (512: two heads per wave, shares up to 8) ...
    ("bf16", 64, 16, 8, 1), ("f32", 32, 16, 16, 1), ("f32", 128, 16, 4, 2),
    ("bf16", 256, 16, 8, 2), ("bf16", 256, 16, 16, 1), ("bf16", 64, 32, 32, 1),
    ("bf16", 256, 16, 4, 2), ("f32", 128, 16, 8, 1), ("f32", 64, 32, 4, 1),
    # ... padded widths (shares of two heads) ...
    ("f32", 40, 16, 4, 1), ("bf16", 96, 16, 8, 2), ("bf16", 80, 16, 2, 1),
    # ... and the generic kernel: a width without a fast shape, a ragged page
    ("bf16", 100, 16, 4, 2), ("bf16", 128, 7, 8, 2),
]


@pytest.mark.parametrize("dtype,D,S,H,Hkv", GQA_CASES)
@pytest.mark.parametrize("split,merge", [(0, 2), (2, 0), (2, 2), (-1, 2)])
def test_grouped_kv_heads(dtype, D, S, H, Hkv, split, merge):
    w = _small(f"gqa_{dtype}_{D}_{S}_{H}_{Hkv}", dtype, D, S, LENGTHS, heads=H, kv_heads=Hkv,
               seed=31)
    kp, vp = device_pool(w)
    pool = _pool(w, kp, vp, split=split, merge=merge)
    plan = pkv.pkv_plan_create(pool)
    pkv.pkv_plan_build(plan, w.lengths.tolist(), w.pt_stride)
    pt = _pt_device(w)
    # layer 0: attention over the generator's rows
    qh = w.q(0)
    out = torch.empty((w.n, H, D), device="cuda")
    pkv.pkv_plan_decode_attention(plan, 0, rows_to_device(qh, dtype), pt, out)
    torch.cuda.synchronize()
    for r in range(w.n):
        assert max_err(out[r], _oracle_decode(w, 0, r, qh)) <= TOL[dtype], (r, int(w.lengths[r]))
    # layer 1: fused append of the shared K/V rows, then attention
    layer = 1
    qh, kh, vh = w.q(layer), w.k_new(layer), w.v_new(layer)
    assert kh.shape == (w.n, Hkv, D)
    q, k, v = (rows_to_device(x, dtype) for x in (qh, kh, vh))
    out = torch.empty((w.n, H, D), device="cuda")
    pkv.pkv_plan_append_and_attend(plan, layer, pt, q, k, v, out)
    torch.cuda.synchronize()
    for r in range(w.n):
        t = int(w.lengths[r])
        page, slot = w.page_tables[r][(t - 1) // S], (t - 1) % S
        assert np.array_equal(to_bits(kp[layer, page, :, slot, :], dtype), kh[r])
        assert np.array_equal(to_bits(vp[layer, page, :, slot, :], dtype), vh[r])
        ref = _oracle_decode(w, layer, r, qh, appended=(kh, vh))
        assert max_err(out[r], ref) <= TOL[dtype], (r, t)
    # the unfused pair gives bit-identical contexts and pages
    kp2, vp2 = device_pool(w, layers=[layer])
    pool2 = _pool(w, kp2, vp2, split=split, merge=merge)
    pkv.pkv_kv_append(pool2, layer, pt, w.pt_stride, (w.lengths - 1).tolist(), k, v)
    out2 = torch.empty_like(out)
    pkv.pkv_decode_attention(pool2, layer, q, pt, w.pt_stride, w.lengths.tolist(), out2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    assert torch.equal(kp[layer], kp2[layer]) and torch.equal(vp[layer], vp2[layer])
    pkv.pkv_plan_destroy(plan)
    pkv.pkv_pool_destroy(pool)
    pkv.pkv_pool_destroy(pool2)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("bf16", 256), ("f32", 64),
                                     ("f32", 32), ("f32", 128)])
@pytest.mark.parametrize("H,Hkv", [(16, 2), (16, 1), (32, 1), (24, 1), (8, 1), (4, 1)])
@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("split", [0, 3])
def test_grouped_workgroup_waves(dtype, D, H, Hkv, waves, split):
    """The matrix-core grouped kernels (bf16 head widths 64, 128, 256; float32
    32, 64, 128) with four and with eight waves per workgroup (eight is the
    default when a workgroup serves 8 or 16 query heads, except at bf16 width
    256): every context against the oracle, unsplit and split."""
    w = _small(f"gqa_waves_{dtype}_{D}_{H}_{Hkv}", dtype, D, 16, LENGTHS, heads=H, kv_heads=Hkv,
               seed=47, layers=1)
    kp, vp = device_pool(w)
    pool = _pool(w, kp, vp, split=split, merge=2)
    pkv.pkv_pool_set_option(pool, pkv.PKV_OPT_WAVES, waves)
    plan = pkv.pkv_plan_create(pool)
    pkv.pkv_plan_build(plan, w.lengths.tolist(), w.pt_stride)
    qh = w.q(0)
    out = torch.empty((w.n, H, D), device="cuda")
    pkv.pkv_plan_decode_attention(plan, 0, rows_to_device(qh, dtype), _pt_device(w), out)
    torch.cuda.synchronize()
    for r in range(w.n):
        assert max_err(out[r], _oracle_decode(w, 0, r, qh)) <= TOL[dtype], (r, int(w.lengths[r]))
    pkv.pkv_plan_destroy(plan)
    pkv.pkv_pool_destroy(pool)


@pytest.mark.parametrize("dtype,D,H,Hkv", [("bf16", 128, 8, 2), ("f32", 64, 4, 1),
                                           ("f32", 40, 6, 3), ("bf16", 128, 32, 1),
                                           ("f32", 64, 12, 2)])
@pytest.mark.parametrize("flags", [0, pkv.PKV_POOL_ADDRESS_ORDER])
def test_grouped_kv_heads_transactional(dtype, D, H, Hkv, flags):
    """begin / batched append_and_attend / abort / commit on caches whose
    pages hold H_kv heads; the aborted request retries with new rows.  Also
    with the address-order free list (the pages leased are 0, 1, 2, ...)."""
    lengths = np.array([1, 16, 17, 250, 600], dtype=np.int64)
    w = _small(f"gqa_txn_{dtype}", dtype, D, 16, lengths, heads=H, kv_heads=Hkv, layers=3,
               seed=37, extra_pages=20)
    kp, vp = device_pool(w)
    pool = _pool(w, kp, vp, seed=9, max_caches=w.n, max_context=1024, merge=2, flags=flags)
    caches = [pkv.pkv_cache_create(pool, 1024) for _ in range(w.n)]
    prefix = w.lengths - 1
    for c, n in zip(caches, prefix.tolist()):
        pkv.pkv_cache_grow(c, n)
    for c in caches:
        pkv.pkv_begin_token(c)
    tables = [pkv.pkv_cache_page_table(c) for c in caches]
    if flags:
        held = sorted(x for t in tables for x in t)
        assert held == list(range(len(held)))
    aborted, abort_layer = 3, 1
    live = list(range(w.n))
    outs = {}
    for layer in range(w.layers):
        if layer == abort_layer:
            pkv.pkv_abort_token(caches[aborted])
            live.remove(aborted)
        qa, ka, va = w.q(layer), w.k_new(layer), w.v_new(layer)
        q, k, v = (rows_to_device(x[live], dtype) for x in (qa, ka, va))
        out = torch.empty((len(live), H, D), device="cuda")
        pkv.pkv_append_and_attend_batched([caches[r] for r in live], layer, q, k, v, out)
        outs[layer] = (list(live), out)
    torch.cuda.synchronize()
    for r in live:
        pkv.pkv_commit_token(caches[r])
    for layer, (lv, out) in outs.items():
        qa, ka, va = w.q(layer), w.k_new(layer), w.v_new(layer)
        kpg, vpg = HostPages(w, "k", layer), HostPages(w, "v", layer)
        for i, r in enumerate(lv):
            ref = oracle.append_and_attend(qa[r], ka[r], va[r], kpg, vpg, tables[r],
                                           int(prefix[r]), 16)
            assert max_err(out[i], ref) <= TOL[dtype], (layer, r)
    assert pkv.pkv_cache_size(caches[aborted]) == prefix[aborted]
    # retry the aborted request with the next step's rows
    assert pkv.pkv_begin_token(caches[aborted]) == prefix[aborted]
    for layer in range(w.layers):
        qa, ka, va = w.q(layer, 1), w.k_new(layer, 1), w.v_new(layer, 1)
        q, k, v = (rows_to_device(x[[aborted]], dtype) for x in (qa, ka, va))
        out = torch.empty((1, H, D), device="cuda")
        pkv.pkv_append_and_attend_batched([caches[aborted]], layer, q, k, v, out)
        torch.cuda.synchronize()
        ref = oracle.append_and_attend(qa[aborted], ka[aborted], va[aborted],
                                       HostPages(w, "k", layer), HostPages(w, "v", layer),
                                       pkv.pkv_cache_page_table(caches[aborted]),
                                       int(prefix[aborted]), 16)
        assert max_err(out[0], ref) <= TOL[dtype], layer
    pkv.pkv_commit_token(caches[aborted])
    for c in caches:
        pkv.pkv_cache_destroy(c)
    pkv.pkv_pool_destroy(pool)


# ------------------------------------------------------- batched prefill --
def _chunk_rows(w, layer, total, step=0):
    """q [T,H,D], k and v [T,H_kv,D] for T new rows, from the generator
    (the stream keys of Workload.chunk_rows)."""
    out = []
    for tag, heads in ((synth.TAG_Q, w.heads), (synth.TAG_K, w.hkv), (synth.TAG_V, w.hkv)):
        key = synth.stream_key(w.seed, tag, layer, 1000 + step)
        out.append(synth.normals(key, 0, total * heads * w.head_width, w.dtype).reshape(
            total, heads, w.head_width))
    return tuple(out)


def _check_prefill(w, layer, starts, counts, qh, kh, vh, out, kp, vp, tables=None):
    S = w.page_size
    kpg, vpg = HostPages(w, "k", layer), HostPages(w, "v", layer)
    off = 0
    for r, (st, n) in enumerate(zip(starts, counts)):
        pt = w.page_tables[r] if tables is None else tables[r]
        sl = slice(off, off + n)
        for i in (0, n // 2, n - 1):
            pos = st + i
            page, slot = pt[pos // S], pos % S
            assert np.array_equal(to_bits(kp[layer, page, :, slot, :], w.dtype), kh[off + i])
            assert np.array_equal(to_bits(vp[layer, page, :, slot, :], w.dtype), vh[off + i])
        ref = oracle.prefill_attention(qh[sl], kh[sl], vh[sl], kpg, vpg, pt, st, S)
        err = np.max(np.abs(out[sl].cpu().numpy().astype(np.float64) - ref))
        assert err <= TOL[w.dtype], (r, st, n, err)
        off += n


PREFILL_CASES = [
    # dtype, D, S, H, H_kv: matrix-core path (16- and 32-token pages) ...
    ("bf16", 128, 16, 4, 4), ("bf16", 128, 16, 8, 2), ("bf16", 128, 32, 4, 1),
    ("bf16", 64, 16, 4, 4), ("bf16", 64, 16, 8, 2), ("bf16", 64, 32, 4, 1),
    ("bf16", 256, 16, 2, 1), ("bf16", 256, 32, 4, 2),
    ("f32", 64, 16, 3, 3), ("f32", 64, 32, 4, 2), ("f32", 32, 16, 4, 1), ("f32", 32, 32, 2, 2),
    ("f32", 128, 16, 2, 2), ("f32", 128, 32, 4, 1),
    # ... and per-row decode kernels
    ("f32", 40, 16, 2, 1), ("f32", 64, 7, 2, 2), ("bf16", 128, 7, 2, 2), ("bf16", 96, 16, 2, 2),
]
PREFILL_CHUNKS = [(0, 1), (0, 37), (5, 20), (16, 16), (100, 70), (1000, 33), (0, 300)]


@pytest.mark.parametrize("dtype,D,S,H,Hkv", PREFILL_CASES)
@pytest.mark.parametrize("merge", MERGES)
def test_prefill_attention_small(dtype, D, S, H, Hkv, merge):
    starts = [a for a, _ in PREFILL_CHUNKS]
    counts = [b for _, b in PREFILL_CHUNKS]
    w = _small(f"prefill_{dtype}_{D}_{S}_{H}_{Hkv}", dtype, D, S,
               [a + b for a, b in PREFILL_CHUNKS], heads=H, kv_heads=Hkv, layers=2, seed=41)
    kp, vp = device_pool(w)
    pool = _pool(w, kp, vp, merge=merge)
    layer = 1
    qh, kh, vh = _chunk_rows(w, layer, sum(counts))
    q, k, v = (rows_to_device(x, dtype) for x in (qh, kh, vh))
    out = torch.full((sum(counts), H, D), float("nan"), device="cuda")
    pkv.pkv_prefill_attention(pool, layer, _pt_device(w), w.pt_stride, starts, counts, q, k, v,
                              out)
    torch.cuda.synchronize()
    _check_prefill(w, layer, starts, counts, qh, kh, vh, out, kp, vp)
    pkv.pkv_pool_destroy(pool)


def test_prefill_rejects_ranges_outside_the_table():
    w = _small("prefill_rej", "f32", 64, 16, [40], heads=1, layers=1)
    kp, vp = device_pool(w)
    pool = _pool(w, kp, vp)
    q = torch.zeros((64, 1, 64), device="cuda")
    pt = _pt_device(w)
    for starts, counts in (([0], [0]), ([-1], [4]), ([w.pt_stride * 16 - 3], [4]), ([0], [1, 2])):
        with pytest.raises((pkv.PkvError, ValueError)):
            pkv.pkv_prefill_attention(pool, 0, pt, w.pt_stride, starts, counts, q, q, q, q)
    pkv.pkv_pool_destroy(pool)


@pytest.mark.parametrize("dtype,D,H,Hkv", [("bf16", 128, 4, 2), ("f32", 64, 2, 2),
                                           ("bf16", 64, 4, 1), ("bf16", 256, 2, 2),
                                           ("f32", 128, 4, 1), ("f32", 32, 2, 2)])
def test_prefill_transactional_chunks(dtype, D, H, Hkv):
    """begin_tokens chunks on several caches (one of them a single token),
    batched append_and_attend per layer, commit; an aborted chunk returns its
    pages and its retry matches the oracle; a decode step then reads the
    committed chunk."""
    chunks = [37, 1, 16, 130]
    prefix = np.array([0, 20, 16, 3], dtype=np.int64)
    w = _small(f"prefill_txn_{dtype}", dtype, D, 16, prefix + np.array(chunks) + 2, heads=H,
               kv_heads=Hkv, layers=2, seed=43, extra_pages=30)
    kp, vp = device_pool(w)
    pool = _pool(w, kp, vp, seed=5, max_caches=8, max_context=1024, merge=2)
    caches = [pkv.pkv_cache_create(pool, 1024) for _ in chunks]
    for c, n in zip(caches, prefix.tolist()):
        pkv.pkv_cache_grow(c, n)
    free0 = pkv.pkv_pool_get_counters(pool).pages_free
    assert pkv.pkv_begin_tokens_batched(caches, chunks) == prefix.tolist()
    # abort cache 3's chunk before any layer, then begin it again
    pkv.pkv_abort_token(caches[3])
    assert len(pkv.pkv_cache_page_table(caches[3])) == 1
    assert pkv.pkv_begin_tokens(caches[3], chunks[3]) == prefix[3]
    tables = [pkv.pkv_cache_page_table(c) for c in caches]
    T = sum(chunks)
    outs = []
    for layer in range(w.layers):
        qh, kh, vh = _chunk_rows(w, layer, T)
        q, k, v = (rows_to_device(x, dtype) for x in (qh, kh, vh))
        out = torch.empty((T, H, D), device="cuda")
        pkv.pkv_append_and_attend_batched(caches, layer, q, k, v, out)
        outs.append((qh, kh, vh, out))
    torch.cuda.synchronize()
    pkv.pkv_commit_token_batched(caches)
    assert [pkv.pkv_cache_size(c) for c in caches] == (prefix + np.array(chunks)).tolist()
    held = sum(-(-(int(a) + b) // 16) for a, b in zip(prefix, chunks))
    assert pkv.pkv_pool_get_counters(pool).pages_free == w.num_pages - held
    for layer, (qh, kh, vh, out) in enumerate(outs):
        _check_prefill(w, layer, prefix.tolist(), chunks, qh, kh, vh, out, kp, vp, tables)
    # one decode token on every cache reads the committed chunk
    layer = 1
    qh, kh, vh = _chunk_rows(w, layer, len(chunks), step=1)
    q, k, v = (rows_to_device(x, dtype) for x in (qh, kh, vh))
    pkv.pkv_begin_token_batched(caches)
    out = torch.empty((len(chunks), H, D), device="cuda")
    pkv.pkv_append_and_attend_batched(caches, layer, q, k, v, out)
    torch.cuda.synchronize()
    prev_q, prev_k, prev_v, _ = outs[layer]
    off = 0
    for r, c in enumerate(caches):
        sl = slice(off, off + chunks[r])
        # rows: generator prefix, the committed chunk, then the new token
        ref = oracle.prefill_attention(
            np.concatenate([prev_q[sl], qh[r:r + 1]]), np.concatenate([prev_k[sl], kh[r:r + 1]]),
            np.concatenate([prev_v[sl], vh[r:r + 1]]), HostPages(w, "k", layer),
            HostPages(w, "v", layer), pkv.pkv_cache_page_table(c), int(prefix[r]), 16)[-1]
        assert max_err(out[r], ref) <= TOL[dtype], r
        off += chunks[r]
    for c in caches:
        pkv.pkv_abort_token(c)
        pkv.pkv_cache_destroy(c)
    pkv.pkv_pool_destroy(pool)


@pytest.mark.parametrize("name", ["prefill32_bf16", "prefill32_fp32"])
def test_prefill32_full_every_request(name):
    """The full prefill workloads (32 chunks of 256-2048 rows over prefixes of
    0-2048; H=32, d_h=128, bf16, and H=12, d_h=64, fp32) in the bench's call.
    Every row of every chunk lands bit-exact in its page slot (checked on the
    device against the input rows); every request is checked against the
    oracle at rows on both sides of the 128-row tile and 64-key block edges,
    the middle and the last two rows, for five heads."""
    from synth import gpu as sgpu
    w = W.WORKLOADS[name]()
    dt = sgpu.torch_dtype(w.dtype)
    H, Hkv, D, S = w.heads, w.hkv, w.head_width, w.page_size
    T = int(w.chunks.sum())
    kp, vp = device_pool(w)
    keys = [synth.stream_key(w.seed, tag, 0, 1000) for tag in (synth.TAG_Q, synth.TAG_K,
                                                                   synth.TAG_V)]
    q = torch.empty((T, H, D), dtype=dt, device="cuda")
    k = torch.empty((T, Hkv, D), dtype=dt, device="cuda")
    v = torch.empty((T, Hkv, D), dtype=dt, device="cuda")
    for t, key in zip((q, k, v), keys):
        sgpu.fill_normal(t, key, w.dtype)
    pool = _pool(w, kp, vp)
    out = torch.full((T, H, D), float("nan"), device="cuda")
    pkv.pkv_prefill_attention(pool, 0, _pt_device(w), w.pt_stride, w.starts.tolist(),
                              w.chunks.tolist(), q, k, v, out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    offs = np.concatenate([[0], np.cumsum(w.chunks)])

    # page writes: row j of the packed input is position starts[r] + i of request r
    pos = np.concatenate([int(w.starts[r]) + np.arange(int(w.chunks[r])) for r in range(w.n)])
    req = np.repeat(np.arange(w.n), w.chunks)
    pages = torch.from_numpy(w.page_tables[req, pos // S].astype(np.int64)).to("cuda")
    slots = torch.from_numpy((pos % S).astype(np.int64)).to("cuda")
    for pool_t, rows_in in ((kp, k), (vp, v)):
        written = pool_t[0][pages, :, slots, :]          # [T, H_kv, D]
        assert torch.equal(written.view(torch.int16 if w.dtype == "bf16" else torch.int32),
                           rows_in.view(torch.int16 if w.dtype == "bf16" else torch.int32))

    kpg, vpg = HostPages(w, "k", 0), HostPages(w, "v", 0)

    def rows(key, first, n, heads, head):
        idx = (((first + np.arange(n, dtype=np.uint64))[:, None] * np.uint64(heads) +
                np.uint64(head)) * np.uint64(D) + np.arange(D, dtype=np.uint64)).ravel()
        return synth.normals_at(key, idx, w.dtype).reshape(n, D)

    heads = sorted({0, 1, H // 2, min(13, H - 1), H - 1})
    worst = 0.0
    for r in range(w.n):
        st, n = int(w.starts[r]), int(w.chunks[r])
        picks = sorted({i for i in (0, 1, 63, 64, 127, 128, 129, n // 2, n - 2, n - 1)
                        if 0 <= i < n})
        ref_rows = max(picks) + 1
        for h in heads:
            kvh = oracle.kv_head_of(h, H, Hkv)
            K = np.concatenate([
                oracle.kv_to_f64(oracle.gather_prefix(kpg, w.page_tables[r], st, S, kvh)).reshape(-1, D),
                oracle.kv_to_f64(rows(keys[1], int(offs[r]), ref_rows, Hkv, kvh))])
            V = np.concatenate([
                oracle.kv_to_f64(oracle.gather_prefix(vpg, w.page_tables[r], st, S, kvh)).reshape(-1, D),
                oracle.kv_to_f64(rows(keys[2], int(offs[r]), ref_rows, Hkv, kvh))])
            qh = rows(keys[0], int(offs[r]), ref_rows, H, h)
            got = out[int(offs[r]):int(offs[r]) + ref_rows, h].cpu().numpy().astype(np.float64)
            for i in picks:
                ref = oracle.attend(qh[i], K[:st + i + 1], V[:st + i + 1])
                err = float(np.max(np.abs(got[i] - ref)))
                worst = max(worst, err)
                assert err <= TOL[w.dtype], (r, i, h, err)
    record_err(f"{name} every request", worst)
    pkv.pkv_pool_destroy(pool)


# --------------------------------------------- prefix sharing, copy on write --
@pytest.mark.parametrize("dtype,D,H,Hkv", [("f32", 64, 2, 2), ("bf16", 128, 4, 2),
                                           ("f32", 40, 3, 3)])
def test_forked_caches_share_prefix_and_copy_on_write(dtype, D, H, Hkv):
    """A holds 37 rows; B forks at 21 (inside a page), C at 32 (a page
    boundary).  One token on each: B's write copies the shared page, C
    leases a new one, A is untouched; every context matches the oracle over
    the shared prefix plus the cache's own row.  Then an aborted copy whose
    shared page lost its other holders, and a grow into a shared page."""
    S, L = 16, 2
    w = _small(f"fork_{dtype}_{D}", dtype, D, S, [40], heads=H, kv_heads=Hkv, layers=L,
               seed=47, extra_pages=40)
    kp, vp = device_pool(w)
    pool = _pool(w, kp, vp, seed=3, max_caches=8, max_context=256, merge=2)
    A = pkv.pkv_cache_create(pool, 256)
    pkv.pkv_cache_grow(A, 37)
    tA = pkv.pkv_cache_page_table(A)
    B = pkv.pkv_cache_fork(A, 21, 256)
    C = pkv.pkv_cache_fork(A, 32, 256)
    assert pkv.pkv_cache_page_table(B) == tA[:2] and pkv.pkv_cache_page_table(C) == tA[:2]
    kA_before = kp[:, tA[1]].clone()
    caches, starts = [A, B, C], [37, 21, 32]
    assert pkv.pkv_begin_token_batched(caches) == starts
    tB, tC = pkv.pkv_cache_page_table(B), pkv.pkv_cache_page_table(C)
    assert tB[0] == tA[0] and tB[1] not in tA                      # B copied page 1
    assert tC[:2] == tA[:2] and tC[2] not in tA                    # C leased page 2
    assert pkv.pkv_pool_get_counters(pool).cow_copies == 1
    outs = []
    for layer in range(L):
        qh, kh, vh = _chunk_rows(w, layer, 3)
        q, k, v = (rows_to_device(x, dtype) for x in (qh, kh, vh))
        out = torch.empty((3, H, D), device="cuda")
        pkv.pkv_append_and_attend_batched(caches, layer, q, k, v, out)
        outs.append((qh, kh, vh, out))
    torch.cuda.synchronize()
    pkv.pkv_commit_token_batched(caches)
    for layer, (qh, kh, vh, out) in enumerate(outs):
        kpg, vpg = HostPages(w, "k", layer), HostPages(w, "v", layer)
        for r, st in enumerate(starts):
            ref = oracle.append_and_attend(qh[r], kh[r], vh[r], kpg, vpg, tA, st, S)
            assert max_err(out[r], ref) <= TOL[dtype], (layer, r)
        # B's copy: A's rows 16..20 bit-exact in every layer, then B's own row
        assert torch.equal(kp[layer, tB[1], :, :5], kA_before[layer, :, :5])
        assert np.array_equal(to_bits(kp[layer, tB[1], :, 5], dtype), kh[1])
    assert torch.equal(kp[:, tA[1]], kA_before)                    # A's page untouched
    # D forks at 21 and writes (its copy is enqueued at its first layer call);
    # every other holder of the shared page then lets it go; D aborts back to
    # that page, which its transaction kept alive, and retries.
    Dc = pkv.pkv_cache_fork(A, 21, 256)
    assert pkv.pkv_begin_token(Dc) == 21
    qh, kh, vh = _chunk_rows(w, 0, 1, step=1)
    out = torch.empty((1, H, D), device="cuda")
    pkv.pkv_append_and_attend(Dc, 0, rows_to_device(qh, dtype), rows_to_device(kh, dtype),
                              rows_to_device(vh, dtype), out)
    torch.cuda.synchronize()
    for c in (A, C):
        pkv.pkv_cache_destroy(c)
    pkv.pkv_abort_token(Dc)
    assert pkv.pkv_cache_page_table(Dc) == tA[:2]
    assert pkv.pkv_begin_token(Dc) == 21                           # sole holder: no copy
    assert pkv.pkv_cache_page_table(Dc) == tA[:2]
    for layer in range(L):
        qh, kh, vh = _chunk_rows(w, layer, 1, step=2)
        out = torch.empty((1, H, D), device="cuda")
        pkv.pkv_append_and_attend(Dc, layer, rows_to_device(qh, dtype),
                                  rows_to_device(kh, dtype), rows_to_device(vh, dtype), out)
        torch.cuda.synchronize()
        ref = oracle.append_and_attend(qh[0], kh[0], vh[0], HostPages(w, "k", layer),
                                       HostPages(w, "v", layer), tA, 21, S)
        assert max_err(out[0], ref) <= TOL[dtype], layer
    pkv.pkv_commit_token(Dc)
    # grow into a shared partly filled page: the copy is complete on return
    E = pkv.pkv_cache_fork(Dc, 22, 256)
    pkv.pkv_cache_grow(E, 3)
    tE = pkv.pkv_cache_page_table(E)
    assert tE[0] == tA[0] and tE[1] != tA[1]
    assert torch.equal(kp[:, tE[1], :, :6], kp[:, tA[1], :, :6])
    assert torch.equal(vp[:, tE[1], :, :6], vp[:, tA[1], :, :6])
    # a prefill chunk on a fork inside a shared page: the chunk's begin copies
    # the page, the append writes the copy, and every row matches the oracle
    F = pkv.pkv_cache_fork(Dc, 19, 256)
    assert pkv.pkv_begin_tokens(F, 30) == 19
    tF = pkv.pkv_cache_page_table(F)
    assert tF[0] == tA[0] and tF[1] != tA[1]
    for layer in range(L):
        qh, kh, vh = _chunk_rows(w, layer, 30, step=3)
        out = torch.empty((30, H, D), device="cuda")
        pkv.pkv_append_and_attend(F, layer, rows_to_device(qh, dtype), rows_to_device(kh, dtype),
                                  rows_to_device(vh, dtype), out)
        torch.cuda.synchronize()
        ref = oracle.prefill_attention(qh, kh, vh, HostPages(w, "k", layer),
                                       HostPages(w, "v", layer), tA, 19, S)
        assert np.max(np.abs(out.cpu().numpy().astype(np.float64) - ref)) <= TOL[dtype], layer
        assert torch.equal(kp[layer, tF[1], :, :3], kp[layer, tA[1], :, :3])
    pkv.pkv_commit_token(F)
    for c in (B, Dc, E, F):
        pkv.pkv_cache_destroy(c)
    assert pkv.pkv_pool_get_counters(pool).pages_free == w.num_pages
    pkv.pkv_pool_destroy(pool)


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 128), ("f32", 24)])
@pytest.mark.parametrize("merge", MERGES)
def test_page_table_permutation_is_bit_identical(dtype, D, merge):
    w = _small("perm", dtype, D, 16, [1, 31, 300, 777], heads=2, layers=1, extra_pages=40)
    kp, vp = device_pool(w)
    pool = _pool(w, kp, vp, split=4, merge=merge)
    q = rows_to_device(w.q(0), dtype)
    out_a = torch.empty((w.n, w.heads, D), device="cuda")
    pt_a = _pt_device(w)
    pkv.pkv_decode_attention(pool, 0, q, pt_a, w.pt_stride, w.lengths.tolist(), out_a)
    # move every used page to a new physical ID (a permutation of the pool)
    perm = torch.from_numpy(synth.shuffle(synth.stream_key(5, synth.TAG_SHUFFLE), w.num_pages)
                            .astype(np.int64)).to("cuda")
    kp_b = torch.empty_like(kp)
    vp_b = torch.empty_like(vp)
    kp_b[0, perm] = kp[0]
    vp_b[0, perm] = vp[0]
    pt_b = torch.where(pt_a >= 0, perm[pt_a.clamp(min=0).long()].int(), pt_a)
    pool_b = _pool(w, kp_b, vp_b, split=4, merge=merge)
    out_b = torch.empty_like(out_a)
    pkv.pkv_decode_attention(pool_b, 0, q, pt_b.contiguous(), w.pt_stride, w.lengths.tolist(),
                             out_b)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    pkv.pkv_pool_destroy(pool)
    pkv.pkv_pool_destroy(pool_b)


def test_split_and_unsplit_agree_and_degenerate_cases():
    w = _small("deg", "f32", 64, 16, [1, 2, 4000], heads=2, layers=1, extra_pages=0)
    kp, vp = device_pool(w)
    q = rows_to_device(w.q(0), "f32")
    pt = _pt_device(w)
    outs = []
    for split, merge in ((-1, 0), (1, 0), (3, 0), (64, 0), (1, 2), (3, 2)):
        pool = _pool(w, kp, vp, split=split, merge=merge)
        out = torch.empty((w.n, w.heads, 64), device="cuda")
        pkv.pkv_decode_attention(pool, 0, q, pt, w.pt_stride, w.lengths.tolist(), out)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
        pkv.pkv_pool_destroy(pool)
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= TOL["f32"]
    # t = 1: the context is the single value row, exactly
    page = int(w.page_tables[0][0])
    v0 = vp[0, page, :, 0, :].cpu().numpy()
    assert np.array_equal(outs[0][0], v0)
    # zero query: the mean of the value rows
    pool = _pool(w, kp, vp)
    out = torch.empty((w.n, w.heads, 64), device="cuda")
    pkv.pkv_decode_attention(pool, 0, torch.zeros_like(q), pt, w.pt_stride,
                             w.lengths.tolist(), out)
    torch.cuda.synchronize()
    for r in range(w.n):
        V = np.stack([oracle.gather_prefix(HostPages(w, "v", 0), w.page_tables[r],
                                           int(w.lengths[r]), 16, h) for h in range(2)])
        assert np.max(np.abs(out[r].cpu().numpy() - V.astype(np.float64).mean(axis=1))) <= 1e-5
    # a dominant score (q equal to one key, scaled up): finite, that value row
    big = np.zeros((w.n, w.heads, 64), dtype=np.float32)
    kpages = HostPages(w, "k", 0)
    target = 1234
    for h in range(2):
        K = oracle.gather_prefix(kpages, w.page_tables[2], 4000, 16, h)
        big[2, h] = K[target] * 40.0
    out = torch.empty((w.n, w.heads, 64), device="cuda")
    pkv.pkv_decode_attention(pool, 0, rows_to_device(big, "f32"), pt, w.pt_stride,
                             w.lengths.tolist(), out)
    torch.cuda.synchronize()
    got = out[2].cpu().numpy()
    assert np.all(np.isfinite(got))
    ref = oracle.paged_decode_attention(big[2], kpages, HostPages(w, "v", 0), w.page_tables[2],
                                        4000, 16)
    assert np.max(np.abs(got - ref)) <= 1e-5
    pkv.pkv_pool_destroy(pool)


def test_empty_and_oversized_inputs_rejected():
    w = _small("rej", "f32", 64, 16, [5], heads=1, layers=1)
    kp, vp = device_pool(w)
    pool = _pool(w, kp, vp)
    q = torch.zeros((1, 1, 64), device="cuda")
    out = torch.empty_like(q)
    pt = _pt_device(w)
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_decode_attention(pool, 0, q, pt, w.pt_stride, [], out)
    assert e.value.status == pkv.PKV_ERR_INVALID_ARGUMENT
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_decode_attention(pool, 0, q, pt, w.pt_stride, [w.pt_stride * 16 + 1], out)
    assert e.value.status == pkv.PKV_ERR_INVALID_ARGUMENT
    with pytest.raises(pkv.PkvError):
        pkv.pkv_decode_attention(pool, 0, q[..., 1:], pt, w.pt_stride, [5], out)  # misaligned
    pkv.pkv_pool_destroy(pool)


def test_debug_validation_rejects_bad_page_ids_before_any_work():
    """With PKV_OPT_VALIDATE, an entry a call would read that is not a page
    of the pool is rejected before anything is enqueued; entries past the
    rows a request reads are not looked at.  The pool is declared four pages
    smaller than its storage, so the rejected IDs (the pool's size and one
    more) still lie inside the allocation."""
    w = _small("validate", "bf16", 128, 16, [40, 17, 3], heads=4, layers=1, extra_pages=8)
    kp, vp = device_pool(w)
    d = pkv.pkv_pool_desc_init()
    d.num_layers, d.num_heads, d.head_width, d.page_size = 1, w.heads, 128, 16
    d.num_pages, d.max_context, d.kv_dtype = w.num_pages - 4, w.pt_stride * 16, pkv.PKV_DTYPE_BF16
    d.k_storage, d.v_storage = kp.data_ptr(), vp.data_ptr()
    pool = pkv.pkv_pool_create(d)
    pkv.pkv_pool_set_option(pool, pkv.PKV_OPT_VALIDATE, 1)
    good = w.page_tables.copy()
    # keep every read entry inside the declared pool
    used = sorted({int(x) for r, t in enumerate(w.lengths.tolist())
                   for x in good[r][: -(-t // 16)]})
    remap = {old: i for i, old in enumerate(used)}
    for r, t in enumerate(w.lengths.tolist()):
        for j in range(-(-t // 16)):
            good[r, j] = remap[int(good[r, j])]
    good[2, 1:] = -7                      # request 2 reads one page: the rest is unread
    q = rows_to_device(w.q(0), "bf16")
    k, v = rows_to_device(w.k_new(0), "bf16"), rows_to_device(w.v_new(0), "bf16")
    pt = torch.from_numpy(good).cuda()
    out = torch.full((w.n, w.heads, 128), float("nan"), device="cuda")
    pkv.pkv_decode_attention(pool, 0, q, pt, w.pt_stride, w.lengths.tolist(), out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    T = 12
    qc, kc, vc = (torch.zeros((T, w.heads, 128), dtype=torch.bfloat16, device="cuda")
                  for _ in range(3))
    for bad_value in (w.num_pages - 4, w.num_pages - 3):
        bad = good.copy()
        bad[0, 2] = bad_value             # request 0 (40 rows) reads entries 0..2
        ptb = torch.from_numpy(bad).cuda()
        sentinel = torch.full((w.n, w.heads, 128), 7.0, device="cuda")
        sentinel_c = torch.full((T, w.heads, 128), 7.0, device="cuda")
        plan = pkv.pkv_plan_create(pool)
        pkv.pkv_plan_build(plan, w.lengths.tolist(), w.pt_stride)
        calls = [
            lambda: pkv.pkv_decode_attention(pool, 0, q, ptb, w.pt_stride, w.lengths.tolist(),
                                             sentinel),
            lambda: pkv.pkv_kv_append(pool, 0, ptb, w.pt_stride, (w.lengths - 1).tolist(), k, v),
            lambda: pkv.pkv_prefill_attention(pool, 0, ptb, w.pt_stride, [30, 0, 0], [10, 1, 1],
                                              qc, kc, vc, sentinel_c),
            lambda: pkv.pkv_plan_decode_attention(plan, 0, q, ptb, sentinel),
            lambda: pkv.pkv_plan_kv_append(plan, 0, ptb, k, v),
            lambda: pkv.pkv_plan_append_and_attend(plan, 0, ptb, q, k, v, sentinel),
        ]
        for call in calls:
            with pytest.raises(pkv.PkvError) as e:
                call()
            assert e.value.status == pkv.PKV_ERR_INVALID_ARGUMENT
            assert "not a page of the pool" in str(e.value)
        torch.cuda.synchronize()
        assert bool((sentinel == 7.0).all()) and bool((sentinel_c == 7.0).all())
        pkv.pkv_plan_destroy(plan)
    pkv.pkv_pool_destroy(pool)


def test_maximum_head_width_generic():
    w = _small("wide", "f32", 1024, 16, [1, 70, 129], heads=2, layers=1)
    kp, vp = device_pool(w)
    pool = _pool(w, kp, vp, split=2)
    qh = w.q(0)
    out = torch.empty((w.n, w.heads, 1024), device="cuda")
    pkv.pkv_decode_attention(pool, 0, rows_to_device(qh, "f32"), _pt_device(w), w.pt_stride,
                             w.lengths.tolist(), out)
    torch.cuda.synchronize()
    for r in range(w.n):
        assert max_err(out[r], _oracle_decode(w, 0, r, qh)) <= TOL["f32"]
    pkv.pkv_pool_destroy(pool)


# ------------------------------------------------------ full-size configs --
def _sampled(n, extra=()):
    idx = sorted(set(list(range(0, n, max(1, n // 6))) + [n - 1] + list(extra)))
    return idx


@pytest.mark.parametrize("merge", MERGES)
@pytest.mark.parametrize("split", [0, 4])
def test_batch32_fp32_l12_full_step(merge, split):
    """32 requests x 12 layers, H=12, d_h=64, fp32, 4096-page pool: one decode
    step (fused append + attend per layer) under the plan the bench uses
    (split 0: the library's own choice, whole requests over sixteen waves
    for this batch) and under 4-block chunks (many split requests)."""
    w = W.batch32_fp32()
    kp, vp = device_pool(w)
    pool = _pool(w, kp, vp, merge=merge, split=split)
    plan = pkv.pkv_plan_create(pool)
    pkv.pkv_plan_build(plan, w.lengths.tolist(), w.pt_stride)
    pt = _pt_device(w)
    outs = []
    for layer in range(w.layers):
        q, k, v = (rows_to_device(x, "f32") for x in (w.q(layer), w.k_new(layer), w.v_new(layer)))
        out = torch.empty((w.n, w.heads, w.head_width), device="cuda")
        pkv.pkv_plan_append_and_attend(plan, layer, pt, q, k, v, out)
        outs.append(out)
    torch.cuda.synchronize()
    rows = np.arange(w.n)
    last = w.lengths - 1
    pages = w.page_tables[rows, last // 16]
    for layer in range(w.layers):
        kh, vh = w.k_new(layer), w.v_new(layer)
        got_k = to_bits(kp[layer][torch.from_numpy(pages).long(), :, torch.from_numpy(last % 16)
                                  .long(), :], "f32")
        got_v = to_bits(vp[layer][torch.from_numpy(pages).long(), :, torch.from_numpy(last % 16)
                                  .long(), :], "f32")
        assert np.array_equal(got_k, kh) and np.array_equal(got_v, vh)
    worst = 0.0
    for layer in range(w.layers):
        qh, kh, vh = w.q(layer), w.k_new(layer), w.v_new(layer)
        kg, vg = GeneratorLayer(w, "k", layer), GeneratorLayer(w, "v", layer)
        if layer == 0:
            kg.spot_check(w.page_tables[:, 0])
        for r in range(w.n):
            t = int(w.lengths[r])
            ref = oracle.append_and_attend(qh[r], kh[r], vh[r], kg, vg, w.page_tables[r], t - 1,
                                           w.page_size)
            err = max_err(outs[layer][r], ref)
            worst = max(worst, err)
            assert err <= TOL["f32"], (layer, r)
    record_err(f"batch32_fp32_l12 full step split {split} merge {merge}", worst)
    pkv.pkv_plan_destroy(plan)
    pkv.pkv_pool_destroy(pool)


def test_last_arriver_merge_is_bitwise_separate_merge():
    """Both merge modes run the same second pass in the same split order, so
    their contexts agree bit for bit; repeated launches in last-arriver mode
    (every 16-row block its own chunk: up to 64 arrivals per counter) must
    never read a stale partial."""
    w = W.batch32_fp32()
    kp, vp = device_pool(w, layers=[0])
    q = rows_to_device(w.q(0), "f32")
    pt = _pt_device(w)
    outs = {}
    for merge in MERGES:
        pool = _pool(w, kp, vp, split=1, merge=merge)
        plan = pkv.pkv_plan_create(pool)
        pkv.pkv_plan_build(plan, w.lengths.tolist(), w.pt_stride)
        assert pkv.pkv_plan_num_chunks(plan) == int(W.pages_needed(w.lengths, 16).sum())
        got = []
        for _ in range(25 if merge == pkv.PKV_MERGE_LAST_ARRIVER else 1):
            out = torch.full((w.n, w.heads, w.head_width), float("nan"), device="cuda")
            pkv.pkv_plan_decode_attention(plan, 0, q, pt, out)
            got.append(out)
        torch.cuda.synchronize()
        outs[merge] = got
        pkv.pkv_plan_destroy(plan)
        pkv.pkv_pool_destroy(pool)
    ref = outs[pkv.PKV_MERGE_SEPARATE][0]
    for o in outs[pkv.PKV_MERGE_LAST_ARRIVER]:
        assert torch.equal(o, ref)
    qh = w.q(0)
    for r in range(w.n):
        assert max_err(ref[r], _oracle_decode(w, 0, r, qh)) <= TOL["f32"]


@pytest.mark.parametrize("merge", MERGES)
def test_plan_decode_replays_from_a_hip_graph(merge):
    """A multi-layer decode on a prebuilt plan, captured once in a HIP graph
    and replayed: every replay (with eager work and synchronisation between
    replays) equals the eager launch bit for bit.  The split-merge counters
    return to zero by themselves, so no memset enters the graph."""
    w = _small("graph", "bf16", 128, 16, [5, 300, 1500, 2600], heads=4, layers=3)
    kp, vp = device_pool(w)
    pool = _pool(w, kp, vp, split=8, merge=merge)
    plan = pkv.pkv_plan_create(pool)
    pkv.pkv_plan_build(plan, w.lengths.tolist(), w.pt_stride)
    assert pkv.pkv_plan_num_chunks(plan) > w.n
    pt = _pt_device(w)
    qs = [rows_to_device(w.q(layer), "bf16") for layer in range(w.layers)]
    eager = [torch.empty((w.n, w.heads, 128), device="cuda") for _ in range(w.layers)]
    for layer in range(w.layers):
        pkv.pkv_plan_decode_attention(plan, layer, qs[layer], pt, eager[layer])
    torch.cuda.synchronize()
    outs = [torch.full_like(e, float("nan")) for e in eager]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for layer in range(w.layers):
            pkv.pkv_plan_decode_attention(plan, layer, qs[layer], pt, outs[layer])
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep}"
        _ = (torch.randn(1 << 20, device="cuda") * 2).sum().item()   # eager work between replays
    qh = w.q(2)
    for r in range(w.n):
        assert max_err(eager[2][r], _oracle_decode(w, 2, r, qh)) <= TOL["bf16"]
    del graph
    pkv.pkv_plan_destroy(plan)
    pkv.pkv_pool_destroy(pool)


@pytest.mark.parametrize("maker", [W.batch256_bf16, W.skewed64_bf16, W.batch256_gqa8_bf16,
                                   W.batch256_mqa_bf16])
@pytest.mark.parametrize("merge", MERGES + [pkv.PKV_MERGE_AUTO])
def test_bf16_single_layer_full(maker, merge):
    w = maker()
    kp, vp = device_pool(w)
    pool = _pool(w, kp, vp, merge=merge)
    plan = pkv.pkv_plan_create(pool)
    pkv.pkv_plan_build(plan, w.lengths.tolist(), w.pt_stride)
    split = pkv.pkv_plan_num_chunks(plan) > w.n
    if w.lengths.max() > 4096:
        assert split   # long contexts are split
    qh = w.q(0)
    out = torch.empty((w.n, w.heads, w.head_width), device="cuda")
    pkv.pkv_pool_set_option(pool, pkv.PKV_OPT_PROFILING, 1)
    pkv.pkv_plan_decode_attention(plan, 0, rows_to_device(qh, "bf16"), _pt_device(w), out)
    torch.cuda.synchronize()
    prof = pkv.pkv_pool_get_profile(pool)
    # a separate merge launch follows a split plan in mode 0, and in the
    # automatic mode when the launch reads at least 1 GiB of K/V
    separate = merge == pkv.PKV_MERGE_SEPARATE or (
        merge == pkv.PKV_MERGE_AUTO and w.kv_bytes_per_layer() >= 1 << 30)
    assert prof.merge_launches == (1 if split and separate else 0)
    assert torch.isfinite(out).all()
    kg, vg = GeneratorLayer(w, "k", 0), GeneratorLayer(w, "v", 0)
    kg.spot_check(w.page_tables[[0, w.n - 1], 0])
    vg.spot_check(w.page_tables[[0, w.n - 1], 0])
    got = out.cpu().numpy().astype(np.float64)
    worst = 0.0
    for r in range(w.n):
        ref = oracle.paged_decode_attention(qh[r], kg, vg, w.page_tables[r], int(w.lengths[r]),
                                            w.page_size, num_kv_heads=w.hkv)
        err = float(np.max(np.abs(got[r] - ref)))
        worst = max(worst, err)
        assert err <= TOL["bf16"], (r, int(w.lengths[r]))
    record_err(f"{w.name} every request merge {merge}", worst)
    pkv.pkv_plan_destroy(plan)
    pkv.pkv_pool_destroy(pool)


def test_fullstep128_bf16_l32_transactional():
    """128 caches x 32 layers, H=32, d_h=128, bf16, every layer's pool filled
    by the generator: begin, batched append_and_attend per layer, commit;
    seeded aborts; then the aborted requests retry and match a run that never
    saw the aborted token.  Every live request is checked against the oracle
    at eight layers spread over the 32 (its new rows bit-exact in the pages
    at every layer), and every retried request at the same layers."""
    w = W.fullstep128_bf16(extra_steps=4)
    checked_layers = [0, 4, 9, 13, 18, 22, 27, 31]
    kp, vp = device_pool(w)
    pool = _pool(w, kp, vp, seed=55, max_caches=w.n, max_context=4096)
    caches = [pkv.pkv_cache_create(pool, 4096) for _ in range(w.n)]
    prefix = w.lengths - 1
    for c, n in zip(caches, prefix.tolist()):
        pkv.pkv_cache_grow(c, n)
    tables = [pkv.pkv_cache_page_table(c) for c in caches]
    flat = [p for t in tables for p in t]
    assert len(flat) == len(set(flat)) and all(0 <= p < w.num_pages for p in flat)
    # find a step with at least one abort
    step = next(s for s in range(100) if (w.abort_layer(s) >= 0).any())
    abort = w.abort_layer(step)
    for c in caches:
        pkv.pkv_begin_token(c)
    tables = [pkv.pkv_cache_page_table(c) for c in caches]
    outs, lives = {}, {}
    live = list(range(w.n))
    for layer in range(w.layers):
        for r in [r for r in live if abort[r] == layer]:
            pkv.pkv_abort_token(caches[r])
        live = [r for r in live if abort[r] != layer]
        qa, ka, va = w.q(layer, step), w.k_new(layer, step), w.v_new(layer, step)
        q, k, v = (rows_to_device(x[live], "bf16") for x in (qa, ka, va))
        out = torch.empty((len(live), w.heads, w.head_width), device="cuda")
        pkv.pkv_append_and_attend_batched([caches[r] for r in live], layer, q, k, v, out)
        lives[layer] = list(live)
        if layer in checked_layers:
            outs[layer] = out
    torch.cuda.synchronize()
    for r in live:
        pkv.pkv_commit_token(caches[r])
    aborted = [r for r in range(w.n) if abort[r] >= 0]
    assert aborted
    for r in range(w.n):
        assert pkv.pkv_cache_size(caches[r]) == prefix[r] + (0 if r in aborted else 1)
    # the committed requests' new rows, bit-exact in the pages of every layer
    committed = list(live)
    rows = torch.tensor([tables[r][int(prefix[r]) // 16] for r in committed], device="cuda")
    slots = torch.tensor([int(prefix[r]) % 16 for r in committed], device="cuda")
    for layer in range(w.layers):
        ka, va = w.k_new(layer, step), w.v_new(layer, step)
        got_k = to_bits(kp[layer][rows, :, slots, :], "bf16")
        got_v = to_bits(vp[layer][rows, :, slots, :], "bf16")
        assert np.array_equal(got_k, ka[committed]) and np.array_equal(got_v, va[committed]), layer
    # the retry of the aborted requests, with the next step's rows
    retry = step + 1
    for r in aborted:
        assert pkv.pkv_begin_token(caches[r]) == prefix[r]
    retry_outs = {}
    for layer in range(w.layers):
        qa, ka, va = w.q(layer, retry), w.k_new(layer, retry), w.v_new(layer, retry)
        q, k, v = (rows_to_device(x[aborted], "bf16") for x in (qa, ka, va))
        out = torch.empty((len(aborted), w.heads, w.head_width), device="cuda")
        pkv.pkv_append_and_attend_batched([caches[r] for r in aborted], layer, q, k, v, out)
        if layer in checked_layers:
            retry_outs[layer] = out
    torch.cuda.synchronize()
    for r in aborted:
        pkv.pkv_commit_token(caches[r])
    retry_tables = {r: pkv.pkv_cache_page_table(caches[r]) for r in aborted}
    worst = 0.0
    for layer in checked_layers:
        kg, vg = GeneratorLayer(w, "k", layer), GeneratorLayer(w, "v", layer)
        if layer == checked_layers[-1]:
            kg.spot_check(tables[0][:2])
        got = outs[layer].cpu().numpy().astype(np.float64)
        qa, ka, va = w.q(layer, step), w.k_new(layer, step), w.v_new(layer, step)
        for i, r in enumerate(lives[layer]):
            ref = oracle.append_and_attend(qa[r], ka[r], va[r], kg, vg, tables[r],
                                           int(prefix[r]), 16)
            err = float(np.max(np.abs(got[i] - ref)))
            worst = max(worst, err)
            assert err <= TOL["bf16"], (layer, r)
        got = retry_outs[layer].cpu().numpy().astype(np.float64)
        qa, ka, va = w.q(layer, retry), w.k_new(layer, retry), w.v_new(layer, retry)
        for i, r in enumerate(aborted):
            ref = oracle.append_and_attend(qa[r], ka[r], va[r], kg, vg, retry_tables[r],
                                           int(prefix[r]), 16)
            err = float(np.max(np.abs(got[i] - ref)))
            worst = max(worst, err)
            assert err <= TOL["bf16"], ("retry", layer, r)
        del kg, vg
    record_err("fullstep128_bf16_l32 live and retried requests", worst)
    cnt = pkv.pkv_pool_get_counters(pool)
    assert cnt.committed_tokens == w.n and cnt.aborted_tokens == len(aborted)
    for c in caches:
        pkv.pkv_cache_destroy(c)
    pkv.pkv_pool_destroy(pool)


# ------------------------------------------------------ randomized sweep --
LARGE_PLANS = [
    # dtype, d_h, H, H_kv, n, length recipe, op, merge; whole = requests kept whole
    ("bf16", 128, 32, 32, 96, "balanced", "append", pkv.PKV_MERGE_AUTO, True),
    ("f32", 64, 16, 16, 128, "one_long", "decode", pkv.PKV_MERGE_AUTO, False),
    ("bf16", 128, 32, 8, 80, "log_uniform", "decode", pkv.PKV_MERGE_SEPARATE, False),
    ("bf16", 256, 16, 16, 140, "balanced", "append", pkv.PKV_MERGE_LAST_ARRIVER, True),
]


@pytest.mark.parametrize("dtype,D,H,Hkv,n,recipe,op,merge,whole", LARGE_PLANS)
def test_large_batch_plans(dtype, D, H, Hkv, n, recipe, op, merge, whole):
    """Batches large enough for the plan's large-batch choices: a balanced
    batch of two or more resident rounds keeps requests whole (eight-wave
    workgroups on the multi-head kernel), one long request or log-uniform
    lengths split into whole chunks with the remainder last.  Every context
    against the oracle, appended rows bit-exact."""
    rng = np.random.default_rng(4100 + D + H + n)
    if recipe == "balanced":
        lengths = rng.integers(600 if D == 128 else 200, 1200 if D == 128 else 400, size=n)
    elif recipe == "one_long":
        lengths = rng.integers(300, 600, size=n)
        lengths[n // 3] = 4000
    else:
        lengths = np.minimum(6000, np.floor(16.0 * np.power(256.0, rng.random(n)))).astype(np.int64) + 1
    w = _small(f"large_{recipe}_{dtype}_{D}", dtype, D, 16, lengths.astype(np.int64), heads=H,
               kv_heads=Hkv if Hkv != H else 0, layers=1, seed=600 + n, extra_pages=8)
    kp, vp = device_pool(w)
    pool = _pool(w, kp, vp, merge=merge)
    pt = _pt_device(w)
    plan = pkv.pkv_plan_create(pool)
    pkv.pkv_plan_build(plan, w.lengths.tolist(), w.pt_stride)
    assert (pkv.pkv_plan_num_chunks(plan) == w.n) == whole
    qh = w.q(0)
    out = torch.empty((w.n, H, D), device="cuda")
    worst = 0.0
    if op == "decode":
        pkv.pkv_plan_decode_attention(plan, 0, rows_to_device(qh, dtype), pt, out)
        torch.cuda.synchronize()
        for r in range(w.n):
            err = max_err(out[r], _oracle_decode(w, 0, r, qh))
            worst = max(worst, err)
            assert err <= TOL[dtype], (r, int(w.lengths[r]))
    else:
        kh, vh = w.k_new(0), w.v_new(0)
        pkv.pkv_plan_append_and_attend(plan, 0, pt, *(rows_to_device(x, dtype)
                                                       for x in (qh, kh, vh)), out)
        torch.cuda.synchronize()
        for r in range(w.n):
            t = int(w.lengths[r])
            page, slot = w.page_tables[r][(t - 1) // 16], (t - 1) % 16
            assert np.array_equal(to_bits(kp[0, page, :, slot, :], dtype), kh[r]), r
            err = max_err(out[r], _oracle_decode(w, 0, r, qh, appended=(kh, vh)))
            worst = max(worst, err)
            assert err <= TOL[dtype], (r, t)
    record_err(f"large plan {recipe} {dtype} d{D} H{H}/{Hkv}", worst)
    pkv.pkv_plan_destroy(plan)
    pkv.pkv_pool_destroy(pool)


def _random_case(rng):
    dtype = ["f32", "bf16"][rng.integers(2)]
    D = int(rng.choice([64, 128, 40, 96, 32] if dtype == "f32" else [128, 128, 64, 80, 256]))
    S = int(rng.choice([16, 16, 32, 8, 5]))
    H = int(rng.choice([1, 2, 4, 6, 8, 16]))
    divisors = [d for d in range(1, H + 1) if H % d == 0]
    Hkv = int(rng.choice(divisors))
    n = int(rng.integers(1, 7))
    lengths = rng.integers(1, 700, size=n)
    split = int(rng.choice([0, 0, -1, 1, 3]))
    merge = int(rng.choice([0, 2]))
    op = ["decode", "append", "prefill"][rng.integers(3)]
    return dtype, D, S, H, Hkv, lengths, split, merge, op


@pytest.mark.parametrize("case", range(24))
def test_randomized_configurations(case):
    """Seeded random geometry, dtype, grouping, split and operation: every
    context against the oracle, appended rows bit-exact."""
    rng = np.random.default_rng(9000 + case)
    dtype, D, S, H, Hkv, lengths, split, merge, op = _random_case(rng)
    w = _small(f"rand{case}", dtype, D, S, lengths, heads=H, kv_heads=Hkv, layers=1,
               seed=100 + case, extra_pages=8)
    kp, vp = device_pool(w)
    pool = _pool(w, kp, vp, split=split, merge=merge)
    pt = _pt_device(w)
    info = (case, dtype, D, S, H, Hkv, lengths.tolist(), split, merge, op)
    if op == "prefill":
        counts = [int(min(t, rng.integers(1, 200))) for t in w.lengths]
        starts = [int(t) - c for t, c in zip(w.lengths, counts)]
        qh, kh, vh = _chunk_rows(w, 0, sum(counts))
        out = torch.empty((sum(counts), H, D), device="cuda")
        pkv.pkv_prefill_attention(pool, 0, pt, w.pt_stride, starts, counts,
                                  *(rows_to_device(x, dtype) for x in (qh, kh, vh)), out)
        torch.cuda.synchronize()
        _check_prefill(w, 0, starts, counts, qh, kh, vh, out, kp, vp)
    else:
        qh = w.q(0)
        out = torch.empty((w.n, H, D), device="cuda")
        plan = pkv.pkv_plan_create(pool)
        pkv.pkv_plan_build(plan, w.lengths.tolist(), w.pt_stride)
        if op == "decode":
            pkv.pkv_plan_decode_attention(plan, 0, rows_to_device(qh, dtype), pt, out)
            torch.cuda.synchronize()
            for r in range(w.n):
                assert max_err(out[r], _oracle_decode(w, 0, r, qh)) <= TOL[dtype], (info, r)
        else:
            kh, vh = w.k_new(0), w.v_new(0)
            pkv.pkv_plan_append_and_attend(plan, 0, pt, *(rows_to_device(x, dtype)
                                                           for x in (qh, kh, vh)), out)
            torch.cuda.synchronize()
            for r in range(w.n):
                t = int(w.lengths[r])
                page, slot = w.page_tables[r][(t - 1) // S], (t - 1) % S
                assert np.array_equal(to_bits(kp[0, page, :, slot, :], dtype), kh[r]), info
                ref = _oracle_decode(w, 0, r, qh, appended=(kh, vh))
                assert max_err(out[r], ref) <= TOL[dtype], (info, r)
        pkv.pkv_plan_destroy(plan)
    pkv.pkv_pool_destroy(pool)
