#!/usr/bin/env python3
"""Benchmark: paged decode attention on one MI355X.

Default workload: 32 requests, 12 layers, H=12, d_h=64, 16-token pages,
attended lengths uniform in [1, 1024], a 4096-page pool with a seeded shuffled
free list, float32.  One step is the whole decode path: begin_token on every
request (lazy page lease), then per layer one batched append_and_attend (K/V
row append, paged attention, split-K merge, plan upload on the first layer),
then commit_token on every request.  Lengths grow by one per committed step;
bytes are counted per step from the actual lengths.

Prints one JSON line.  ``value`` is K/V GB/s over the timed steps (wall clock
between device synchronisations, nothing but the steps on the stream).
``roofline`` reports the attention kernel alone, from a second timed pass of
the same number of steps in which the library records HIP events on the
launch stream immediately around every attention kernel (PKV_OPT_PROFILING)
and sums each launch's algorithmic bytes.

Other workloads (--workload): batch256_bf16, skewed64_bf16 (single-layer
batched decode over existing rows), batch256_gqa8_bf16 and batch256_mqa_bf16
(the same batch with 32 query heads sharing 8 K/V heads, or one), fullstep128_bf16_l32 (32 layers, 128
requests, bf16, 1% seeded aborts), prefill32_bf16 and prefill32_fp32 (batched
prefill chunks, reported in TFLOP/s against the matrix-core peak of their
dtype) and tiny (the latency-bound fixture:
token-at-a-time steps of one request, reported in steps/s and us/step).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0

# Calibrated HBM traffic per launch of each workload's dominant kernel from
# rocprofv3 PMC runs: FETCH_SIZE and WRITE_SIZE in KiB per dispatch, scaled
# by what the same counters read for one kernel that reads and writes
# exactly 1 GiB (FETCH_SIZE x 2.000, WRITE_SIZE x 1.000 on MI355X).  Valid
# only for the kernel source they were taken from (sha256 prefix of that
# file under csrc/).
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
MEASURED_TRAFFIC = {
    "batch32_fp32_l12": {"source": "kernels.hip", "sha256_16": "290d3361ae1bcabb",
        "fetch_kib": 44294.2, "write_kib": 299.2,
        "algorithmic_bytes": 88971264},
    "batch256_bf16": {"source": "kernels.hip", "sha256_16": "290d3361ae1bcabb",
        "fetch_kib": 4761714.8, "write_kib": 4345.9,
        "algorithmic_bytes": 9718775808},
    "batch256_gqa8_bf16": {"source": "kernels.hip", "sha256_16": "290d3361ae1bcabb",
        "fetch_kib": 1194139.1, "write_kib": 4097.2,
        "algorithmic_bytes": 2434412544},
    "batch256_mqa_bf16": {"source": "kernels.hip", "sha256_16": "290d3361ae1bcabb",
        "fetch_kib": 152003.2, "write_kib": 4096.0,
        "algorithmic_bytes": 309806592},
    "prefill32_bf16": {"source": "prefill.hip", "sha256_16": "64e07feb42ad9f32",
        "fetch_kib": 724296.0, "write_kib": 518320.2,
        "algorithmic_bytes": 1854562304},
    "prefill32_fp32": {"source": "prefill.hip", "sha256_16": "64e07feb42ad9f32",
        "fetch_kib": 291189.8, "write_kib": 97857.0,
        "algorithmic_bytes": 575582208},
}


def measured_traffic(workload: str):
    """(HBM bytes per launch, algorithmic bytes of the same launches) from
    the PMC runs, or (None, None) if the kernel source changed since."""
    import hashlib
    m = MEASURED_TRAFFIC.get(workload)
    if m is None:
        return None, None
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "paged_kv_cache_attention_amd",
                       "csrc", m["source"])
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest()[:16] != m["sha256_16"]:
            return None, None
    return (int((m["fetch_kib"] * FETCH_SCALE + m["write_kib"] * WRITE_SCALE) * 1024),
            m["algorithmic_bytes"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="batch32_fp32_l12")
    ap.add_argument("--split-blocks", type=int, default=0)
    ap.add_argument("--waves", type=int, default=0,
                    help="waves per workgroup of the fast path (4, 8; 0 = per plan)")
    ap.add_argument("--merge-mode", type=int, default=2,
                    help="2: last-arriving chunk merges (default), 0: separate merge kernel")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="bound on the oracle's timed CPU work")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="time the steps without per-kernel HIP events (no roofline)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one kernel that reads and writes 1 GiB (HBM counter "
                         "calibration)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this decode path has no multi-GPU mode "
              "(requests and heads shard without communication; see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_attention_amd as pkv
    from synth import gpu as sgpu
    from synth import workloads as W

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    if args.calibrate_copy:
        # one elementwise kernel that reads 1 GiB and writes 1 GiB
        src = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    if args.workload == "tiny":
        return tiny_latency(args)
    if args.workload.startswith("prefill"):
        return prefill_bench(args, W.WORKLOADS[args.workload]())
    maker = W.WORKLOADS[args.workload]
    grow = 3 * args.steps + args.warmup + 2   # committed tokens per request over three passes
    w = maker(extra_steps=grow) if args.workload.startswith("fullstep") else maker()
    transactional = w.appends
    dt = sgpu.torch_dtype(w.dtype)
    H, D, L, n = w.heads, w.head_width, w.layers, w.n
    Hkv = w.hkv
    elt = w.elt

    # ---- pool and inputs, filled on the device by the seeded generator ----
    shape = (L, w.num_pages, Hkv, w.page_size, D)
    kp = torch.empty(shape, dtype=dt, device="cuda")
    vp = torch.empty(shape, dtype=dt, device="cuda")
    for layer in range(L):
        sgpu.fill_normal(kp[layer], w.kpool_key(layer), w.dtype)
        sgpu.fill_normal(vp[layer], w.vpool_key(layer), w.dtype)
    q_all = torch.empty((L, n, H, D), dtype=dt, device="cuda")
    k_all = torch.empty((L, n, Hkv, D), dtype=dt, device="cuda")
    v_all = torch.empty((L, n, Hkv, D), dtype=dt, device="cuda")
    for layer in range(L):
        sgpu.fill_normal(q_all[layer], w.q_key(layer), w.dtype)
        sgpu.fill_normal(k_all[layer], w.k_key(layer), w.dtype)
        sgpu.fill_normal(v_all[layer], w.v_key(layer), w.dtype)
    out = torch.empty((n, H, D), dtype=torch.float32, device="cuda")

    max_context = int(w.lengths.max()) + grow + 32
    d = pkv.pkv_pool_desc_init()
    d.num_layers, d.num_heads, d.head_width = L, H, D
    d.page_size, d.num_pages, d.max_context = w.page_size, w.num_pages, max_context
    d.max_caches = max(n, 1)
    d.kv_dtype = pkv.PKV_DTYPE_F32 if w.dtype == "f32" else pkv.PKV_DTYPE_BF16
    d.split_blocks = args.split_blocks
    d.k_storage, d.v_storage = kp.data_ptr(), vp.data_ptr()
    d.free_list_seed = w.seed
    d.num_kv_heads = Hkv
    pool = pkv.pkv_pool_create(d)
    pkv.pkv_pool_set_option(pool, pkv.PKV_OPT_MERGE_MODE, args.merge_mode)
    pkv.pkv_pool_set_option(pool, pkv.PKV_OPT_WAVES, args.waves)

    step_kv_bytes = []

    if transactional:
        caches = [pkv.pkv_cache_create(pool, max_context) for _ in range(n)]
        for c, t in zip(caches, w.lengths.tolist()):
            pkv.pkv_cache_grow(c, t - 1)
        all_caches = pkv.pkv_cache_array(caches)
        lens = [t - 1 for t in w.lengths.tolist()]   # committed lengths
        sh = stream.cuda_stream
        step_no = [0]

        def step(timed: bool):
            s = step_no[0]
            step_no[0] += 1
            abort = w.abort_layer(s)
            pkv.pkv_begin_token_batched(all_caches)
            live = list(range(n))
            live_arr = all_caches
            idx = None
            kv_bytes = 0
            t_sum = sum(lens) + n
            for layer in range(L):
                if (abort == layer).any():
                    for r in [r for r in live if abort[r] == layer]:
                        pkv.pkv_abort_token(caches[r])
                    live = [r for r in live if abort[r] != layer]
                    live_arr = pkv.pkv_cache_array([caches[r] for r in live])
                    t_sum = sum(lens[r] + 1 for r in live)
                    # the live rows' index, uploaded once per abort from
                    # pinned memory without waiting for the stream (a
                    # pageable upload would drain it at every later layer)
                    idx = torch.tensor(live, dtype=torch.int64).pin_memory().to(
                        "cuda", non_blocking=True)
                if len(live) == n:
                    q, k, v, o = q_all[layer], k_all[layer], v_all[layer], out
                else:
                    q, k, v = q_all[layer][idx], k_all[layer][idx], v_all[layer][idx]
                    o = out[:len(live)]
                kv_bytes += t_sum * Hkv * 2 * D * elt
                pkv.pkv_append_and_attend_batched(live_arr, layer, q, k, v, o, stream=sh)
            pkv.pkv_commit_token_batched(live_arr)
            for r in live:
                lens[r] += 1
            if timed:
                step_kv_bytes.append(kv_bytes)
    else:
        plan = pkv.pkv_plan_create(pool)
        pkv.pkv_plan_build(plan, w.lengths.tolist(), w.pt_stride, stream=stream)
        pt = torch.from_numpy(w.page_tables.copy()).to("cuda")
        kv_once = int(w.lengths.sum()) * Hkv * 2 * D * elt

        def step(timed: bool):
            pkv.pkv_plan_decode_attention(plan, 0, q_all[0], pt, out, stream=stream)
            if timed:
                step_kv_bytes.append(kv_once)

    for _ in range(args.warmup):
        step(False)
    # Pass 1: the timed steps, nothing else on the stream -> value.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kv_total = float(sum(step_kv_bytes))
    # Pass 2: the same number of steps with the library's HIP events around
    # every attention kernel -> the kernel's average duration (the event
    # packets lengthen a step, so they are kept out of pass 1).
    prof = None
    if not args.no_kernel_events:
        pkv.pkv_pool_get_profile(pool, reset=True)
        pkv.pkv_pool_set_option(pool, pkv.PKV_OPT_PROFILING, 1)
        for _ in range(args.steps):
            step(False)
        torch.cuda.synchronize()
        pkv.pkv_pool_set_option(pool, pkv.PKV_OPT_PROFILING, 0)
        prof = pkv.pkv_pool_get_profile(pool, reset=True)
    # Pass 3: one stream event between successive steps -> per-step spread.
    spread = step_spread(lambda: step(False), args.steps)
    launches = prof.attention_launches if prof else 0
    avg_kern_s = prof.attention_ms / max(1, launches) / 1e3 if prof else 0.0
    bytes_per_launch = prof.algorithmic_bytes / max(1, launches) if prof else 0.0
    achieved = bytes_per_launch / avg_kern_s / 1e9 if avg_kern_s > 0 else 0.0
    value = kv_total / elapsed / 1e9
    chunks = None
    if not transactional:
        chunks = pkv.pkv_plan_num_chunks(plan)

    traffic, traffic_alg = measured_traffic(w.name)
    result = {
        "metric": "paged decode attention KV GB/s (% of HBM peak) + decode-attention steps/sec",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "steps_per_sec": round(args.steps / elapsed, 2),
        "step_ms": spread,
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "requests": n, "layers": L, "heads": H, "kv_heads": Hkv, "head_width": D,
            "page_size": w.page_size, "pool_pages": w.num_pages,
            "mean_attended_len": round(kv_total / args.steps / L / (Hkv * 2 * D * elt) /
                                       max(1, n), 1),
            "kv_bytes_per_step": int(kv_total / args.steps),
            "split_blocks": args.split_blocks,
            "merge_mode": args.merge_mode,
            "waves_option": args.waves,
            "plan_chunks": chunks,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": dominant_kernel(w),
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "avg_launch_us": round(avg_kern_s * 1e6, 2),
            "bytes_per_launch": int(bytes_per_launch),
            "launches_timed": int(launches),
            "merge_launches": int(prof.merge_launches) if prof else 0,
            "merge_avg_us": round(prof.merge_ms / max(1, prof.merge_launches) * 1e3, 2)
            if prof else 0.0,
            "traffic": traffic,
            "traffic_run_algorithmic_bytes": traffic_alg,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # dense matrix-core peaks


def step_spread(step, steps: int) -> dict:
    """Median, min and max step time (ms) from one stream event recorded
    between successive steps; a separate pass, so the events do not touch the
    timed whole-job figure."""
    import statistics

    import torch

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return {"median": round(statistics.median(ms), 4), "min": round(min(ms), 4),
            "max": round(max(ms), 4), "steps": steps}


def dominant_kernel(w) -> str:
    """The attention kernel the library dispatches for a decode workload: the
    matrix-core grouped kernel for bf16 d_h of 64, 128 or 256 when a
    multiple of 4 query heads share a K/V head (template arguments: heads per
    workgroup, waves per workgroup, d_h), else the vector fast path."""
    group = w.heads // w.hkv
    D = w.head_width
    if w.dtype == "bf16" and D in (64, 128, 256) and w.page_size % 16 == 0 and group % 4 == 0:
        share = next(s for s in (16, 8, 4) if group % s == 0)
        waves = 8 if share >= 8 and D != 256 else 4
        return f"attend_group_mfma_kernel<{share},{waves},{D}>"
    return f"attend_fast_kernel<{'float' if w.dtype == 'f32' else 'bf16'},{D}>"


def prefill_bench(args, w):
    """Batched prefill of one layer: every request's chunk is appended and
    attends causally over its prefix and itself, in one pkv_prefill_attention
    call (append launch + matrix-core attention launch).  Reported in TFLOP/s
    of the score and value products (4 d_h per new row, head and attended
    row); the roofline is the attention kernel against the dense matrix-core
    peak of the pool's dtype (bf16 2.5 PFLOP/s, float32 157.3 TFLOP/s)."""
    import torch

    import paged_kv_cache_attention_amd as pkv
    from synth import gpu as sgpu

    dt = sgpu.torch_dtype(w.dtype)
    H, Hkv, D = w.heads, w.hkv, w.head_width
    T = int(w.chunks.sum())
    shape = (1, w.num_pages, Hkv, w.page_size, D)
    kp = torch.empty(shape, dtype=dt, device="cuda")
    vp = torch.empty(shape, dtype=dt, device="cuda")
    sgpu.fill_normal(kp[0], w.kpool_key(0), w.dtype)
    sgpu.fill_normal(vp[0], w.vpool_key(0), w.dtype)
    q = torch.empty((T, H, D), dtype=dt, device="cuda")
    k = torch.empty((T, Hkv, D), dtype=dt, device="cuda")
    v = torch.empty((T, Hkv, D), dtype=dt, device="cuda")
    from synth import TAG_K, TAG_Q, TAG_V, stream_key
    for t, tag in ((q, TAG_Q), (k, TAG_K), (v, TAG_V)):
        sgpu.fill_normal(t, stream_key(w.seed, tag, 0, 1000), w.dtype)
    out = torch.empty((T, H, D), dtype=torch.float32, device="cuda")
    d = pkv.pkv_pool_desc_init()
    d.num_layers, d.num_heads, d.head_width, d.num_kv_heads = 1, H, D, Hkv
    d.page_size, d.num_pages = w.page_size, w.num_pages
    d.max_context = w.pt_stride * w.page_size
    d.kv_dtype = pkv.PKV_DTYPE_F32 if w.dtype == "f32" else pkv.PKV_DTYPE_BF16
    d.k_storage, d.v_storage = kp.data_ptr(), vp.data_ptr()
    d.free_list_seed = w.seed
    pool = pkv.pkv_pool_create(d)
    pt = torch.from_numpy(w.page_tables.copy()).to("cuda")
    starts, counts = w.starts.tolist(), w.chunks.tolist()
    stream = torch.cuda.current_stream()

    def step():
        pkv.pkv_prefill_attention(pool, 0, pt, w.pt_stride, starts, counts, q, k, v, out,
                                  stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    flops = w.prefill_flops()
    value = flops * args.steps / elapsed / 1e12
    prof = None
    if not args.no_kernel_events:
        pkv.pkv_pool_get_profile(pool, reset=True)
        pkv.pkv_pool_set_option(pool, pkv.PKV_OPT_PROFILING, 1)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        pkv.pkv_pool_set_option(pool, pkv.PKV_OPT_PROFILING, 0)
        prof = pkv.pkv_pool_get_profile(pool, reset=True)
    spread = step_spread(step, args.steps)
    traffic, traffic_alg = measured_traffic(w.name)
    launches = prof.prefill_launches if prof else 0
    avg_s = prof.prefill_ms / max(1, launches) / 1e3 if prof else 0.0
    achieved = (prof.prefill_flops / max(1, launches)) / avg_s / 1e12 if avg_s > 0 else 0.0
    result = {
        "metric": "batched prefill attention TFLOP/s (score and value products)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "step_ms": spread,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "requests": w.n, "layers": 1, "heads": H, "kv_heads": Hkv,
            "head_width": D, "page_size": w.page_size, "pool_pages": w.num_pages,
            "new_rows": T, "mean_prefix": round(float(w.starts.mean()), 1),
            "flops_per_step": flops, "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "prefill_f32_kernel" if w.dtype == "f32" else "prefill_mfma_kernel",
            "achieved": round(achieved, 1),
            "peak": MFMA_PEAK_TFLOPS[w.dtype],
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_PEAK_TFLOPS[w.dtype], 4),
            "avg_launch_us": round(avg_s * 1e6, 2),
            "flops_per_launch": int(prof.prefill_flops / max(1, launches)) if prof else 0,
            "launches_timed": int(launches),
            "traffic": traffic,
            "traffic_run_algorithmic_bytes": traffic_alg,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = prefill_cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    pkv.pkv_pool_destroy(pool)


def prefill_cpu_baseline(w, budget_s: float) -> dict:
    """The oracle's prefill, one thread, over whole requests' chunks in order
    (shortest first) until the time budget is spent."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    qa, ka, va = w.chunk_rows(0)
    offs = np.concatenate([[0], np.cumsum(w.chunks)])
    order = np.argsort(w.chunks, kind="stable")
    pk, pv = {}, {}
    limiter = threadpool_limits(limits=1) if threadpool_limits else None
    done_flops, done = 0, 0
    t0 = time.perf_counter()
    try:
        for r in order.tolist():
            st, n = int(w.starts[r]), int(w.chunks[r])
            pt = w.page_tables[r]
            for p in pt[: -(-st // w.page_size)].tolist():
                if p not in pk:
                    pk[p] = w.pool_page("k", 0, p)
                    pv[p] = w.pool_page("v", 0, p)
            sl = slice(int(offs[r]), int(offs[r + 1]))
            oracle.prefill_attention(qa[sl], ka[sl], va[sl], pk, pv, pt, st, w.page_size)
            done_flops += (n * st + n * (n + 1) // 2) * w.heads * 4 * w.head_width
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
    finally:
        if limiter is not None:
            limiter.restore_original_limits()
    el = time.perf_counter() - t0
    return {"value": round(done_flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
            "kind": "oracle",
            "sample": f"layer 0 of {w.name}: {done} of {w.n} requests (shortest chunks first), "
                      f"all {w.heads} heads, {done_flops} flops in {el:.2f} s (float64, one thread, "
                      f"page generation included)"}


def tiny_latency(args):
    """Tiny fixture: 1 request, 2 layers, H=2, d_h=2, 16-token pages, 8 pages,
    float32, context 4: token-at-a-time steps (begin, append_and_attend per
    layer, commit), reset after the fourth.  Latency-bound: reports us/step."""
    import torch

    import paged_kv_cache_attention_amd as pkv
    from synth import gpu as sgpu
    from synth import workloads as W

    g = W.tiny_geometry()
    L, H, D, C = g["layers"], g["heads"], g["head_width"], g["max_len"]
    kp = torch.zeros((L, g["num_pages"], H, g["page_size"], D), device="cuda")
    vp = torch.zeros_like(kp)
    d = pkv.pkv_pool_desc_init()
    d.num_layers, d.num_heads, d.head_width = L, H, D
    d.page_size, d.num_pages, d.max_context = g["page_size"], g["num_pages"], C
    d.k_storage, d.v_storage, d.free_list_seed = kp.data_ptr(), vp.data_ptr(), g["seed"]
    pool = pkv.pkv_pool_create(d)
    cache = pkv.pkv_cache_create(pool, C)
    rows = [[tuple(sgpu.to_device(x, "f32", "cuda") for x in W.tiny_rows(g["seed"], l, p, H, D))
             for l in range(L)] for p in range(C)]
    out = torch.empty((H, D), device="cuda")
    sh = torch.cuda.current_stream().cuda_stream

    def step(i):
        pos = i % C
        if pos == 0 and pkv.pkv_cache_size(cache) == C:
            pkv.pkv_cache_reset(cache)
        pkv.pkv_begin_token(cache)
        for layer in range(L):
            q, k, v = rows[pos][layer]
            pkv.pkv_append_and_attend(cache, layer, q, k, v, out, stream=sh)
        pkv.pkv_commit_token(cache)

    for i in range(args.warmup * C):
        step(i)
    torch.cuda.synchronize()
    n = args.steps * C
    t0 = time.perf_counter()
    for i in range(n):
        step(i)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    it = iter(range(n, 2 * n))
    spread = step_spread(lambda: step(next(it)), n)
    kv = sum(t for t in range(1, C + 1)) * args.steps * L * H * 2 * D * 4
    print(json.dumps({
        "metric": "paged decode attention KV GB/s (% of HBM peak) + decode-attention steps/sec",
        "value": round(n / el, 1), "unit": "steps/s", "n_gpus": 1, "steps": n,
        "warmup": args.warmup * C, "ms_per_step": round(el / n * 1e3, 4),
        "us_per_step": round(el / n * 1e6, 2), "step_ms": spread,
        "kv_bytes_per_step_mean": kv // n,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "tiny", "requests": 1, "layers": L, "heads": H, "head_width": D,
                   "page_size": g["page_size"], "pool_pages": g["num_pages"], "context": C,
                   "parallelism": "single GPU"}}), flush=True)
    pkv.pkv_cache_destroy(cache)
    pkv.pkv_pool_destroy(pool)


def cpu_baseline(w, budget_s: float) -> dict:
    """The oracle as it is, single-threaded, on a bounded sample of the same
    workload: layer 0, requests in order, in repeated passes until the time
    budget is spent (a pass over a small layer takes well under a second).
    Page generation is done before timing; only the oracle is timed."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None

    pages_k, pages_v = {}, {}
    q = w.q(0)
    kn, vn = w.k_new(0), w.v_new(0)
    order = list(range(w.n))
    prepared = []
    t_prep = time.perf_counter()
    pt_all = w.page_tables if w.page_tables.shape[1] else None
    for r in order:
        t = int(w.lengths[r])
        npg = -(-t // w.page_size)
        pt = pt_all[r, :npg] if pt_all is not None else np.arange(r * npg, (r + 1) * npg)
        for p in pt.tolist():
            if p not in pages_k:
                pages_k[p] = w.pool_page("k", 0, p)
                pages_v[p] = w.pool_page("v", 0, p)
        prepared.append((r, t, pt))
        if time.perf_counter() - t_prep > budget_s:
            break
    limiter = threadpool_limits(limits=1) if threadpool_limits else None
    done_bytes = 0
    done = 0
    passes = 0
    out_of_time = False
    t0 = time.perf_counter()
    try:
        while not out_of_time:
            for r, t, pt in prepared:
                if w.appends:
                    # re-appending the same row at the same slot is idempotent
                    oracle.append_and_attend(q[r], kn[r], vn[r], pages_k, pages_v, pt, t - 1,
                                             w.page_size)
                else:
                    oracle.paged_decode_attention(q[r], pages_k, pages_v, pt, t, w.page_size,
                                                  num_kv_heads=w.hkv)
                done_bytes += t * w.hkv * 2 * w.head_width * w.elt
                done += 1
                if time.perf_counter() - t0 > budget_s:
                    out_of_time = True
                    break
            else:
                passes += 1
    finally:
        if limiter is not None:
            limiter.restore_original_limits()
    el = time.perf_counter() - t0
    return {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"layer 0 of {w.name}: {len(prepared)} of {w.n} requests, all {w.heads} "
                      f"heads, {passes} full passes, {done} request calls, {done_bytes} K/V "
                      f"bytes in {el:.2f} s (float64, one thread)"}


if __name__ == "__main__":
    main()
