#!/usr/bin/env python3
"""Benchmark: paged decode attention on one MI355X.

Default workload (the largest configuration that fits one GPU, and one of the
bf16 batched configurations the roofline target is set on): a full decode
step of 32 layers over 128 requests, H=32, d_h=128, 16-token pages, retained
prefixes uniform in [1536, 2560], bf16 K/V and q, float32 context, 1% of
(request, step) aborted at a seeded layer.  One step is the whole decode
path: begin_token on every request (lazy page lease), then per layer one
batched append_and_attend (K/V row append, paged attention, split-K merge,
plan upload on the first layer), aborts at their layer, then commit_token
on every live request.  Lengths grow by one per committed step; bytes are
counted per step from the actual lengths.

Prints one JSON line.  ``value`` is K/V GB/s over the timed steps (wall clock
between device synchronisations, nothing but the steps on the stream).
``roofline`` reports the attention kernel alone, from a second timed pass of
the same number of steps in which the library records HIP events on the
launch stream immediately around every attention kernel (PKV_OPT_PROFILING)
and sums each launch's algorithmic bytes (for workloads whose step is a
single launch, the duration comes instead from one event pair around
back-to-back launches, at least as many as the timed steps and at least
~50 ms of them, free of per-kernel event packets); it also repeats the
whole-step rate and says whether the kernel-only rate is at least that (for
short multi-layer launches it can fall just below: the event pair around a
launch adds about a microsecond to what it measures, e.g. 20.8 us per launch
against 19.4 us per layer of whole-step wall clock on the 12-layer float32
step).  ``cpu_baseline`` is
the float64 oracle on the host's cores, timed before the GPU is touched.

Other workloads (--workload): batch32_fp32_l12 (32 requests, 12 layers,
H=12, d_h=64, float32, lengths U[1,1024], the same step), batch256_bf16,
skewed64_bf16 (single-layer
batched decode over existing rows), batch256_gqa8_bf16 and batch256_mqa_bf16
(the same batch with 32 query heads sharing 8 K/V heads, or one), prefill32_bf16 and prefill32_fp32 (batched
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
    "fullstep128_bf16_l32": {"source": "kernels.hip", "sha256_16": "5e8a45bd1180b636",
        "fetch_kib": 2070881.5, "write_kib": 4088.8,
        "algorithmic_bytes": 4238041600},
    "batch32_fp32_l12": {"source": "kernels.hip", "sha256_16": "5e8a45bd1180b636",
        "fetch_kib": 44104.7, "write_kib": 292.0,
        "algorithmic_bytes": 88676352},
    "batch256_bf16": {"source": "kernels.hip", "sha256_16": "5e8a45bd1180b636",
        "fetch_kib": 4759798.5, "write_kib": 4113.5,
        "algorithmic_bytes": 9718775808},
    "skewed64_bf16": {"source": "kernels.hip", "sha256_16": "5e8a45bd1180b636",
        "fetch_kib": 1790272.4, "write_kib": 2576.8,
        "algorithmic_bytes": 3659710464},
    "batch256_gqa8_bf16": {"source": "kernels.hip", "sha256_16": "5e8a45bd1180b636",
        "fetch_kib": 1191767.6, "write_kib": 4096.1,
        "algorithmic_bytes": 2434412544},
    "batch256_mqa_bf16": {"source": "kernels.hip", "sha256_16": "5e8a45bd1180b636",
        "fetch_kib": 152515.3, "write_kib": 4096.0,
        "algorithmic_bytes": 309806592},
    "prefill32_bf16": {"source": "prefill.hip", "sha256_16": "c6bff56b4b013bd9",
        "fetch_kib": 753658.9, "write_kib": 518320.2,
        "algorithmic_bytes": 1854562304},
    "prefill32_fp32": {"source": "prefill.hip", "sha256_16": "c6bff56b4b013bd9",
        "fetch_kib": 281745.6, "write_kib": 97857.0,
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
    ap.add_argument("--workload", default="fullstep128_bf16_l32")
    ap.add_argument("--split-blocks", type=int, default=0)
    ap.add_argument("--waves", type=int, default=0,
                    help="waves per workgroup of the fast path (4, 8; 0 = per plan)")
    ap.add_argument("--merge-mode", type=int, default=1,
                    help="1: the library's choice per plan (default), 2: last-arriving chunk "
                         "merges, 0: separate merge kernel")
    ap.add_argument("--address-order", action="store_true",
                    help="pool allocator leases pages in address order (PKV_POOL_ADDRESS_ORDER) "
                         "instead of from the seeded shuffled free list")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="bound on the oracle's timed CPU work (all cores, then one)")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle worker processes (0: the cores this process may use, "
                         "at most 16)")
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

    from synth import workloads as W

    # The oracle's CPU baseline runs first, in worker processes forked before
    # this process has loaded the HIP runtime or touched the GPU.
    grow = 3 * args.steps + args.warmup + 2   # committed tokens per request over three passes
    baseline = None
    if not args.no_cpu_baseline and args.workload != "tiny":
        maker = W.WORKLOADS[args.workload]
        wb = maker(extra_steps=grow) if args.workload.startswith("fullstep") else maker()
        baseline = (prefill_cpu_baseline if args.workload.startswith("prefill") else cpu_baseline)(
            wb, args.cpu_seconds, args.cpu_workers)

    import numpy as np
    import torch

    import paged_kv_cache_attention_amd as pkv
    from synth import gpu as sgpu

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
        return prefill_bench(args, W.WORKLOADS[args.workload](), baseline)
    maker = W.WORKLOADS[args.workload]
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
    if args.address_order:
        d.flags = pkv.PKV_POOL_ADDRESS_ORDER
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
    # Pass 2b, steps that are one attention launch each: one pair of events
    # on the launch stream around all the launches, back to back -> device
    # time per launch with no event packet between them (per-kernel events
    # cost a few microseconds each).  Multi-layer steps keep the per-kernel
    # events: host work and other kernels sit between their launches.
    # At least ~50 ms of launches, so a step of tens of microseconds is not
    # timed over a couple of milliseconds only.
    batch_s = None
    batch_launches = 0
    if not args.no_kernel_events and not transactional:
        batch_launches = max(args.steps, int(0.05 / max(elapsed / args.steps, 1e-6)) + 1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(batch_launches):
            step(False)
        e1.record(stream)
        torch.cuda.synchronize()
        batch_s = e0.elapsed_time(e1) / 1e3 / batch_launches
    # Pass 3: one stream event between successive steps -> per-step spread.
    spread = step_spread(lambda: step(False), args.steps)
    launches = prof.attention_launches if prof else 0
    event_kern_s = prof.attention_ms / max(1, launches) / 1e3 if prof else 0.0
    if batch_s is not None:
        avg_kern_s, timing = batch_s, "one event pair around back-to-back launches"
    else:
        avg_kern_s, timing = event_kern_s, "event pair around each attention launch"
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
            "page_allocator": ("address order" if args.address_order else "seeded shuffle")
            if transactional else "synthetic shuffled page tables",
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": dominant_kernel(w),
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "step_rate_gbs": round(value, 1),
            "step_frac": round(value / HBM_PEAK_GBS, 4),
            "kernel_rate_at_least_step_rate": bool(achieved >= value),
            "avg_launch_us": round(avg_kern_s * 1e6, 2),
            "launch_timing": timing,
            "avg_launch_us_per_kernel_events": round(event_kern_s * 1e6, 2),
            "bytes_per_launch": int(bytes_per_launch),
            "launches_timed": int(batch_launches if batch_s is not None else launches),
            "merge_launches": int(prof.merge_launches) if prof else 0,
            "merge_avg_us": round(prof.merge_ms / max(1, prof.merge_launches) * 1e3, 2)
            if prof else 0.0,
            "traffic": traffic,
            "traffic_run_algorithmic_bytes": traffic_alg,
        },
    }
    if baseline is not None:
        result["cpu_baseline"] = baseline
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
    """The attention kernel the library dispatches for a decode workload: a
    grouped matrix-core kernel when a multiple of 4 query heads share a K/V
    head (bf16 d_h 64/128/256, float32 d_h 32/64/128; template arguments:
    heads per workgroup, waves per workgroup, d_h), else the vector fast path
    (type, d_h); ",nt" when its K/V loads are non-temporal, which is when one
    workgroup serves all the query heads of a K/V head."""
    group = w.heads // w.hkv
    D = w.head_width
    widths = (64, 128, 256) if w.dtype == "bf16" else (32, 64, 128)
    if D in widths and w.page_size % 16 == 0 and group % 4 == 0:
        share = next(s for s in (16, 8, 4) if group % s == 0)
        nt = ",nt" if group == share else ""
        if w.dtype == "bf16":
            waves = 8 if share >= 8 and D != 256 else 4
            return f"attend_group_mfma_kernel<{share},{waves},{D}{nt}>"
        waves = 8 if share >= 8 else 4
        return f"attend_group_f32_kernel<{share},{waves},{D}{nt}>"
    row_bytes = D * (4 if w.dtype == "f32" else 2)
    share = next(s for s in ((8, 4, 2, 1) if row_bytes == 512 else (16, 8, 4, 2, 1))
                 if group % s == 0)
    nt = ",nt" if group == share else ""
    return f"attend_fast_kernel<{'float' if w.dtype == 'f32' else 'bf16'},{D}{nt}>"


def prefill_bench(args, w, baseline):
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
    if baseline is not None:
        result["cpu_baseline"] = baseline
    print(json.dumps(result), flush=True)
    pkv.pkv_pool_destroy(pool)


def _cpu_workers(requested: int) -> int:
    """Oracle worker processes: the cores this process may run on, at most 16
    (one GPU's share of the host)."""
    if requested > 0:
        return requested
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _oracle_worker(i, units, prepare, run_unit, budget_s, prep_s, barrier, results):
    """One worker process: prepares the host inputs of its units (untimed,
    within prep_s), waits for every worker, then runs its prepared units in
    repeated passes until budget_s has elapsed; reports (work, elapsed,
    units run, units prepared)."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        pass
    state, ready = prepare(units, time.perf_counter() + prep_s)
    try:
        barrier.wait(timeout=prep_s + 120)
    except Exception:  # pragma: no cover
        pass
    work, done = 0, 0
    t0 = time.perf_counter()
    while ready:
        for u in ready:
            work += run_unit(state, u)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        else:
            continue
        break
    results.put((i, work, time.perf_counter() - t0, done, len(ready)))


def _run_oracle_workers(units, prepare, run_unit, workers: int, budget_s: float, prep_s: float):
    """The oracle in `workers` forked processes (forked before this process
    has touched the GPU), each over a contiguous slice of `units`.  Returns
    (total work, longest elapsed, units run, units prepared)."""
    import multiprocessing as mp
    ctx = mp.get_context("fork")
    barrier = ctx.Barrier(workers)
    results = ctx.Queue()
    n = len(units)
    procs = []
    for i in range(workers):
        part = units[i * n // workers:(i + 1) * n // workers]
        pr = ctx.Process(target=_oracle_worker,
                         args=(i, part, prepare, run_unit, budget_s, prep_s, barrier, results))
        pr.start()
        procs.append(pr)
    got = [results.get(timeout=budget_s + prep_s + 300) for _ in procs]
    for pr in procs:
        pr.join()
    work = sum(g[1] for g in got)
    elapsed = max(g[2] for g in got)
    return work, elapsed, sum(g[3] for g in got), sum(g[4] for g in got)


class _HeadPages:
    """Physical pages narrowed to one K/V head: page p -> [1, S, D]."""

    def __init__(self, pages, head: int):
        self.pages, self.head = pages, head

    def __getitem__(self, p):
        return self.pages[p][self.head:self.head + 1]


def prefill_cpu_baseline(w, budget_s: float, workers: int = 0) -> dict:
    """The float64 oracle's prefill (oracle.prefill_attention) on the host's
    cores, one (request, query head) lane per call -- the lane's query rows
    with its K/V head's new rows and pages -- in contiguous slices over worker
    processes, repeated passes for the time budget, then with one process.
    Reported in TFLOP/s of the score and value products (4 d_h per new row,
    head and attended row)."""
    import numpy as np

    import oracle

    qa, ka, va = w.chunk_rows(0)
    offs = np.concatenate([[0], np.cumsum(w.chunks)])
    H, Hkv = w.heads, w.hkv

    def prepare(lanes, deadline):
        pk, pv, ready, seen = {}, {}, [], set()
        for r, h in lanes:
            if r not in seen:
                if time.perf_counter() > deadline and ready:
                    break
                st = int(w.starts[r])
                for p in w.page_tables[r][: -(-st // w.page_size)].tolist():
                    pk[p] = w.pool_page("k", 0, p)
                    pv[p] = w.pool_page("v", 0, p)
                seen.add(r)
            ready.append((r, h))
        return (pk, pv), ready

    def run_unit(state, lane):
        pk, pv = state
        r, h = lane
        kvh = oracle.kv_head_of(h, H, Hkv)
        st, n = int(w.starts[r]), int(w.chunks[r])
        sl = slice(int(offs[r]), int(offs[r + 1]))
        oracle.prefill_attention(qa[sl, h:h + 1], ka[sl, kvh:kvh + 1], va[sl, kvh:kvh + 1],
                                 _HeadPages(pk, kvh), _HeadPages(pv, kvh), w.page_tables[r], st,
                                 w.page_size)
        return (n * st + n * (n + 1) // 2) * 4 * w.head_width

    order = np.argsort(w.chunks, kind="stable").tolist()   # shortest chunks first
    lanes = [(r, h) for r in order for h in range(H)]
    nw = _cpu_workers(workers)
    multi = _run_oracle_workers(lanes, prepare, run_unit, nw, budget_s * 0.6, budget_s)
    single = _run_oracle_workers(lanes[:H], prepare, run_unit, 1, budget_s * 0.4, budget_s * 0.5)
    return {"value": round(multi[0] / multi[1] / 1e12, 6), "unit": "TFLOP/s", "cores": nw,
            "kind": "oracle",
            "sample": f"layer 0 of {w.name}: {multi[3]} of {len(lanes)} (request, head) lanes "
                      f"prepared over {nw} worker processes (contiguous slices, shortest "
                      f"chunks first), {multi[2]} lane calls, {int(multi[0])} flops in "
                      f"{multi[1]:.2f} s (float64)",
            "single_process": {"value": round(single[0] / single[1] / 1e12, 6),
                               "unit": "TFLOP/s", "cores": 1,
                               "sample": f"lanes of the shortest chunk, {single[2]} lane "
                                         f"calls in {single[1]:.2f} s"}}


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


def cpu_baseline(w, budget_s: float, workers: int = 0) -> dict:
    """The float64 oracle as it is, on the host's cores: layer 0 of the same
    workload, split into (request, query head) lanes -- gather the head's
    prefix through the page table, then softmax(q K^T / sqrt(d_h)) V
    (oracle.gather_prefix, oracle.attend) -- in contiguous slices over worker
    processes, each running its lanes in repeated passes for the time budget;
    then the same with one process.  Pages are regenerated before timing.
    Workloads that append write the new row into its host page first:
    attending over t rows then equals the oracle's append-then-attend, bit
    for bit.  The rate counts the K/V bytes the GPU path counts: t * H_kv *
    2 * d_h * elt per request (a lane of a grouped head is 1/G of that)."""
    import numpy as np

    import oracle

    H, Hkv, D, S = w.heads, w.hkv, w.head_width, w.page_size
    G = H // Hkv
    q = w.q(0)
    kn, vn = (w.k_new(0), w.v_new(0)) if w.appends else (None, None)
    # Page tables: the workload's, or (where the library's allocator assigns
    # them during the run) consecutive distinct pages per request.
    npg = -(-w.lengths.astype(np.int64) // S)
    if w.page_tables.shape[1] > 0:
        tables = [w.page_tables[r, :npg[r]] for r in range(w.n)]
    else:
        base = np.concatenate([[0], np.cumsum(npg)])
        tables = [np.arange(base[r], base[r + 1]) % w.num_pages for r in range(w.n)]

    def prepare(lanes, deadline):
        pk, pv, ready, seen = {}, {}, [], {}
        for r, h in lanes:
            if r not in seen:
                if time.perf_counter() > deadline and ready:
                    break
                t, pt = int(w.lengths[r]), tables[r]
                for p in pt.tolist():
                    pk[p] = w.pool_page("k", 0, p)
                    pv[p] = w.pool_page("v", 0, p)
                if w.appends:
                    last = int(pt[(t - 1) // S])
                    pk[last] = pk[last].copy()
                    pv[last] = pv[last].copy()
                    pk[last][:, (t - 1) % S, :] = kn[r]
                    pv[last][:, (t - 1) % S, :] = vn[r]
                seen[r] = (t, pt)
            ready.append((r, h))
        return (pk, pv, seen), ready

    lane_bytes = 2 * D * w.elt / G

    def run_unit(state, lane):
        pk, pv, seen = state
        r, h = lane
        t, pt = seen[r]
        kvh = oracle.kv_head_of(h, H, Hkv)
        K = oracle.gather_prefix(pk, pt, t, S, kvh)
        V = oracle.gather_prefix(pv, pt, t, S, kvh)
        oracle.attend(q[r, h], K, V)
        return t * lane_bytes

    lanes = [(r, h) for r in range(w.n) for h in range(H)]
    nw = _cpu_workers(workers)
    multi = _run_oracle_workers(lanes, prepare, run_unit, nw, budget_s * 0.6, budget_s)
    single = _run_oracle_workers(lanes[:8 * H], prepare, run_unit, 1, budget_s * 0.4,
                                 budget_s * 0.5)
    gbs = multi[0] / multi[1] / 1e9
    one = single[0] / single[1] / 1e9
    step_bytes = w.kv_bytes_per_layer() * w.layers
    out = {"value": round(gbs, 4), "unit": "GB/s", "cores": nw, "kind": "oracle",
           "sample": f"layer 0 of {w.name}: {multi[3]} of {len(lanes)} (request, head) lanes "
                     f"prepared, run in repeated passes by {nw} worker processes (one per "
                     f"core, contiguous lane slices): {multi[2]} lane calls, {int(multi[0])} "
                     f"K/V bytes in {multi[1]:.2f} s (float64)",
           "single_process": {"value": round(one, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"lanes of the first {single[3] // H} requests, "
                                        f"{single[2]} lane calls in {single[1]:.2f} s"}}
    if w.layers > 1:
        # a whole step is every layer: L times the layer-0 work at the same rate
        out["steps_per_sec"] = round(gbs * 1e9 / step_bytes, 5)
        out["step_note"] = (f"one step reads {step_bytes} K/V bytes over {w.layers} layers; "
                            f"steps/s = rate / step bytes (layer 0 timed, scaled x{w.layers})")
    return out


if __name__ == "__main__":
    main()
