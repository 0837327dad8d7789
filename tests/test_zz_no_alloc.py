"""The allocation-free batched decode call (pkv_decode_attention_noalloc)
against the call it varies (pkv_decode_attention): the same plan and kernels,
so the contexts must agree bit for bit, and both must match the oracle.  Two
calls in a row on one pool, the second with a smaller input: the first plan
is above the inline limit (copied into the scratch) and splits long
requests (partials and merge counters in the scratch); the second is small
enough to travel in the kernel arguments.  Sizes beyond the scratch are
rejected before any work."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from synth import workloads as W
from tests.gpu_support import TOL, HostPages, device_pool, max_err, record_err, rows_to_device

pytestmark = pytest.mark.gpu
pkv = pytest.importorskip("paged_kv_cache_attention_amd")

CASES = [
    # dtype, d_h, query heads, K/V heads, merge mode, split blocks
    ("bf16", 128, 8, 8, pkv.PKV_MERGE_LAST_ARRIVER, 0),
    ("bf16", 128, 32, 8, pkv.PKV_MERGE_LAST_ARRIVER, 0),
    ("f32", 64, 12, 12, pkv.PKV_MERGE_SEPARATE, 4),
    ("bf16", 96, 4, 4, pkv.PKV_MERGE_LAST_ARRIVER, 2),
]


def _workload(dtype, D, H, Hkv, seed):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(1, 3000, size=96)
    lengths[:4] = [1, 16, 17, 20000]
    lengths = lengths.astype(np.int64)
    P = int(W.pages_needed(lengths, 16).sum()) + 4
    w = W.Workload(f"noalloc_{dtype}_{D}_{H}_{Hkv}", seed, len(lengths), 1, H, D, 16, P, dtype,
                   lengths, appends=False, kv_heads=Hkv if Hkv != H else 0)
    return W._finish(w)


def _pool(w, kp, vp, merge, split):
    d = pkv.pkv_pool_desc_init()
    d.num_layers, d.num_heads, d.head_width, d.num_kv_heads = 1, w.heads, w.head_width, w.kv_heads
    d.page_size, d.num_pages, d.max_context = 16, w.num_pages, w.pt_stride * 16
    d.kv_dtype = pkv.PKV_DTYPE_F32 if w.dtype == "f32" else pkv.PKV_DTYPE_BF16
    d.split_blocks = split
    d.k_storage, d.v_storage = kp.data_ptr(), vp.data_ptr()
    pool = pkv.pkv_pool_create(d)
    pkv.pkv_pool_set_option(pool, pkv.PKV_OPT_MERGE_MODE, merge)
    return pool


@pytest.mark.parametrize("dtype,D,H,Hkv,merge,split", CASES)
def test_noalloc_equals_decode_attention_on_two_calls(dtype, D, H, Hkv, merge, split):
    w = _workload(dtype, D, H, Hkv, seed=300 + D + H)
    kp, vp = device_pool(w)
    pool = _pool(w, kp, vp, merge, split)
    kpg, vpg = HostPages(w, "k", 0), HostPages(w, "v", 0)
    qh = w.q(0)
    q = rows_to_device(qh, dtype)
    pt = torch.from_numpy(w.page_tables.copy()).cuda()
    worst = 0.0
    # first call: 96 requests (above the inline limit), long ones split;
    # second call: the first 20 requests, shorter, on the same pool
    for n, cap in ((w.n, None), (20, 700)):
        lens = w.lengths[:n].copy()
        if cap is not None:
            lens = np.minimum(lens, cap)
        ref = torch.full((n, H, D), float("nan"), device="cuda")
        got = torch.full((n, H, D), float("nan"), device="cuda")
        pkv.pkv_decode_attention(pool, 0, q[:n], pt[:n], w.pt_stride, lens.tolist(), ref)
        pkv.pkv_decode_attention_noalloc(pool, 0, q[:n], pt[:n], w.pt_stride, lens.tolist(), got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), n
        for r in range(n):
            want = oracle.paged_decode_attention(qh[r], kpg, vpg, w.page_tables[r], int(lens[r]),
                                                 16, num_kv_heads=w.hkv)
            err = max_err(got[r], want)
            worst = max(worst, err)
            assert err <= TOL[dtype], (n, r, int(lens[r]))
    record_err(f"noalloc {dtype} d{D} h{H} kv{Hkv}", worst)
    pkv.pkv_pool_destroy(pool)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    H, D = 32, 128
    w = W.Workload("noalloc_big", 5, 4, 1, H, D, 16, 4 * 2048 + 4, "bf16",
                   np.full(4, 32768, dtype=np.int64), appends=False)
    W._finish(w)
    kp = torch.zeros((1, 8, H, 16, D), dtype=torch.bfloat16, device="cuda")
    d = pkv.pkv_pool_desc_init()
    d.num_layers, d.num_heads, d.head_width, d.page_size = 1, H, D, 16
    d.num_pages, d.max_context, d.kv_dtype = 8, 32768, pkv.PKV_DTYPE_BF16
    d.split_blocks = 1                       # every 16-row block its own chunk
    d.k_storage = d.v_storage = kp.data_ptr()
    pool = pkv.pkv_pool_create(d)
    q = torch.zeros((pkv.PKV_NOALLOC_MAX_REQUESTS + 1, H, D), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((pkv.PKV_NOALLOC_MAX_REQUESTS + 1, H, D), device="cuda")
    pt = torch.zeros((pkv.PKV_NOALLOC_MAX_REQUESTS + 1, 2048), dtype=torch.int32, device="cuda")
    # 4 x 2048 chunks x 32 heads x 130 floats: more partials than the scratch holds
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_decode_attention_noalloc(pool, 0, q, pt, 2048, [32768] * 4, out)
    assert e.value.status == pkv.PKV_ERR_INVALID_ARGUMENT and "scratch" in str(e.value)
    # more requests than the scratch holds
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_decode_attention_noalloc(pool, 0, q, pt, 2048,
                                         [1] * (pkv.PKV_NOALLOC_MAX_REQUESTS + 1), out)
    assert e.value.status == pkv.PKV_ERR_INVALID_ARGUMENT and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0          # nothing was enqueued
    pkv.pkv_pool_destroy(pool)
