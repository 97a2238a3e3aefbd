#!/usr/bin/env python3
"""Decode-step throughput of libpagedattn on one GPU.

A step is one pass of the whole hot path over one batch: the KV-cache write
of each sequence's new token, then paged decode attention over every
sequence's context including that token (partition kernel + log-sum-exp
merge), through paged_attention_decode_step (the cache write and the work
plan in one launch; --two-calls times reshape_and_cache and
paged_attention_decode instead, which give the same bits).  The default workload is the Llama-2-7B-shaped
layer: 64 sequences, 32 query / 32 kv heads, head_dim 128, 16-token pages,
context lengths uniform in [128, 2048], bf16 K/V/q, fp32 softmax and
accumulation, pool = 1.25x the pages needed, shuffled.

Prints one JSON line.  ``value`` is decode tokens/s (sequences / step time);
``roofline`` prices the partition kernel (the dominant kernel) against the
8 TB/s HBM peak using its algorithmic KV bytes,
sum(ctx) * kv_heads * head_dim * 2 * sizeof(bf16), and its own duration
from HIP events recorded on its stream around every launch.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak of MI355X


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="workload 1..5 (default 2)")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--partition-size", type=int, default=None,
                    help="split-K partition in tokens (default: the workload's own, else the "
                         "library default of 1024 tokens)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU-baseline budget per leg (all cores, then one core): oracle steps "
                         "are repeated until this is spent")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="decode-step: after the timed region, this many steps each preceded "
                         "by a 1 GiB read that evicts the pools from the caches; reports the "
                         "partition kernel's cold-cache duration (0: skip)")
    ap.add_argument("--probe", action="store_true", help="also measure achievable read GB/s")
    ap.add_argument("--traffic-json", default=None,
                    help="HBM bytes per partition-kernel launch measured with rocprofv3 counters "
                         "(default: profiles/traffic_pa_decode_partition_c<config>.json); used "
                         "only while the kernel source still has the hash recorded there")
    ap.add_argument("--op", choices=["decode-step", "prefill", "cache-rope", "copy", "swap-out",
                                     "swap-in"],
                    default="decode-step",
                    help="decode-step (default): the hot path; prefill: a multi-token step "
                         "(--config picks prefill workload 1..4); cache-rope: the cache write "
                         "with rotary embedding fused in, on prefill workload --config; copy / "
                         "swap-out / swap-in: copy_blocks within the device pool, to a pinned "
                         "host pool, back")
    ap.add_argument("--alibi", action="store_true",
                    help="decode-step / prefill through the ALiBi entry points (the ALiBi "
                         "paper's geometric slopes)")
    ap.add_argument("--pages", type=int, default=2048,
                    help="pages moved per copy_blocks call (--op copy/swap-*)")
    ap.add_argument("--shared-prefix", action="store_true",
                    help="decode through paged_attention_decode_shared_prefix, using the "
                         "workload's groups of samples that share prompt pages (config 5)")
    ap.add_argument("--two-calls", action="store_true",
                    help="time reshape_and_cache and paged_attention_decode (or "
                         "_shared_prefix, or paged_attention_prefill with --op prefill) as two "
                         "calls instead of the step entry paged_attention_decode_step "
                         "(_shared_prefix_step, paged_attention_prefill_step): bit for bit the "
                         "same result, one launch more")
    ap.add_argument("--graph", action="store_true",
                    help="decode-step: also capture one step (cache write + attention) in a HIP "
                         "graph and time --steps replays (graph_ms_per_step; value stays the "
                         "eager rate)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed region, run a plain device copy of this many MiB "
                         "5 times, so a counter run can scale FETCH_SIZE / WRITE_SIZE")
    return ap.parse_args()


# Sources that define each partition kernel; a recorded traffic figure is
# valid only while their combined hash is unchanged.
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "paged_kv_cache_457_amd", "csrc")
KERNEL_SOURCES = {
    "pa_prefill_gqa": ["pagedattn_prefill.hip", "pagedattn_device.h", "pagedattn_internal.h",
                       "pagedattn_prefill_launch.h"],
    "pa_decode_prefix_gqa": ["pagedattn_decode_prefix.hip", "pagedattn_device.h",
                             "pagedattn_internal.h"],
    "pa_decode_partition": ["pagedattn_decode.hip", "pagedattn_device.h", "pagedattn_internal.h"],
    "pa_decode_partition_gqa": ["pagedattn_decode_gqa.hip", "pagedattn_device.h",
                                "pagedattn_internal.h"],
}


def _percentiles(ms):
    """p10, p50 and p90 of a list of durations in ms."""
    import numpy as np
    p = np.percentile(np.asarray(ms, dtype=np.float64), [10, 50, 90])
    return {"p10": round(float(p[0]), 5), "p50": round(float(p[1]), 5),
            "p90": round(float(p[2]), 5)}


def dominant_kernel(w) -> str:
    """The partition kernel the library runs for this workload: bf16 with a
    group of query heads per kv-head goes to the matrix-core kernel."""
    return "pa_decode_partition_gqa" if (w.dtype == "bf16" and w.group >= 2) \
        else "pa_decode_partition"


def kernel_source_sha256(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(args, kernel, tag=None):
    """HBM bytes per partition-kernel launch from a committed counter run,
    or None when there is none for this workload or the kernel source has
    changed since the counters were taken."""
    path = args.traffic_json or os.path.join(
        os.path.dirname(os.path.abspath(__file__)), "profiles",
        f"traffic_{kernel}_{tag or 'c%d' % args.config}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel") != kernel or rec.get("kernel_source_sha256") != kernel_source_sha256(kernel):
        return None
    if rec.get("config_index") != args.config or rec.get("partition_size") != \
            args.effective_partition or rec.get("seed") != args.seed:
        return None
    return rec.get("bytes_per_launch")


# State the all-core leg's worker processes read (inherited through fork,
# before this process touches the GPU).
_CPU_STATE = {}
# Worker processes of the all-core leg: the host's CPU share for one GPU.
CPU_WORKERS_MAX = 16


def _oracle_unit(unit):
    """oracle.decode on one (sequence, kv-head) unit: that kv-head's query
    heads over the sequence's pages, in the pools after the step's write."""
    s, g = unit
    st = _CPU_STATE
    w = st["w"]
    G = w.group
    import oracle
    return oracle.decode(w.q[s:s + 1, g * G:(g + 1) * G], st["kp"][:, g:g + 1],
                         st["vp"][:, g:g + 1], w.block_tables[s:s + 1],
                         w.context_lens[s:s + 1], 1, w.scale, w.block_size, w.dtype).shape


def _worker_init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)      # one BLAS thread per worker process


def cpu_baseline_all_cores(w, budget_s):
    """The oracle, as it stands, on every host core this process may use (at
    most CPU_WORKERS_MAX): each step runs the oracle's cache write here and
    oracle.decode over the (sequence, kv-head) units in a pool of worker
    processes, one BLAS thread each, largest units first.  Must run before
    this process initialises the GPU (the workers are forked)."""
    import multiprocessing as mp
    import oracle
    from threadpoolctl import threadpool_limits
    n = max(1, min(CPU_WORKERS_MAX, len(os.sched_getaffinity(0))))
    kp, vp = oracle.reshape_and_cache(w.k_new, w.v_new, w.k_pool, w.v_pool, w.slot_mapping,
                                      w.block_size)
    _CPU_STATE.update(w=w, kp=kp, vp=vp)
    units = sorted(((s, g) for s in range(w.num_seqs) for g in range(w.num_kv_heads)),
                   key=lambda u: -int(w.context_lens[u[0]]))
    chunk = max(1, len(units) // (8 * n))
    runs = 0
    with mp.get_context("fork").Pool(n, initializer=_worker_init) as pool, \
            threadpool_limits(limits=1):
        list(pool.imap_unordered(_oracle_unit, units[:n], chunksize=1))   # workers up
        t0 = time.perf_counter()
        while True:
            oracle.reshape_and_cache(w.k_new, w.v_new, w.k_pool, w.v_pool, w.slot_mapping,
                                     w.block_size)
            for _ in pool.imap_unordered(_oracle_unit, units, chunksize=chunk):
                pass
            runs += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = (time.perf_counter() - t0) / runs
    _CPU_STATE.clear()
    return {
        "value": round(w.num_seqs / dt, 2),
        "unit": "tokens/s",
        "cores": n,
        "kind": "oracle",
        "sample": f"the whole batch ({w.num_seqs} sequences): per step the oracle's cache "
                  f"write in one process, then oracle.decode over {len(units)} (sequence, "
                  f"kv-head) units in {n} worker processes, one BLAS thread each; {runs} "
                  f"step(s), {dt:.3f} s/step, fp64 NumPy; host has "
                  f"{len(os.sched_getaffinity(0))} usable cores "
                  f"({platform.processor() or platform.machine()})",
    }


def cpu_baseline(w, budget_s):
    """The oracle, as it stands, on this host: cache write + decode of the
    same batch, repeated until the budget is spent (at least once)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    runs = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while True:
            kp, vp = oracle.reshape_and_cache(w.k_new, w.v_new, w.k_pool, w.v_pool,
                                              w.slot_mapping, w.block_size)
            out = oracle.decode(w.q, kp, vp, w.block_tables, w.context_lens, w.num_kv_heads,
                                w.scale, w.block_size, w.dtype)
            runs += 1
            if time.perf_counter() - t0 >= budget_s:
                break
    dt = (time.perf_counter() - t0) / runs
    assert np.all(np.isfinite(out))
    return {
        "value": round(w.num_seqs / dt, 2),
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"the whole batch ({w.num_seqs} sequences, cache write + decode), "
                  f"{runs} run(s), {dt:.2f} s/step, fp64 NumPy, BLAS limited to 1 thread; "
                  f"host has {len(os.sched_getaffinity(0))} usable cores "
                  f"({platform.processor() or platform.machine()})",
    }


def bench_copy(args):
    """copy_blocks on the workload's pool: --pages random pages per call,
    within the device pool (copy-on-write), to a pinned host pool (swap-out)
    or back (swap-in).  Bytes per call = pages * page bytes * 2 pools read
    and the same written; the call is timed with HIP events on its stream.
    For the swaps, a contiguous pinned copy of the same byte count through
    torch (one DMA transfer) is timed beside it."""
    import numpy as np
    import torch
    from paged_kv_cache_457_amd import binding
    from paged_kv_cache_457_amd.device_inputs import upload
    from paged_kv_cache_457_amd.workloads import CONFIG_NAMES, make_config

    w = make_config(args.config, args.seed)
    dw = upload(w)
    rng = np.random.default_rng(7)
    n = min(args.pages, w.num_blocks // 2)
    page_shape = tuple(w.k_pool.shape[1:])
    page_bytes = int(np.prod(page_shape)) * w.elem_bytes
    src = rng.choice(w.num_blocks, size=n, replace=False)
    if args.op == "copy":
        dst = rng.choice(np.setdiff1d(np.arange(w.num_blocks), src), size=n, replace=False)
        ks, vs, kd, vd = dw.k_pool, dw.v_pool, dw.k_pool, dw.v_pool
    else:
        hk = torch.empty((n,) + page_shape, dtype=dw.k_pool.dtype, pin_memory=True)
        hv = torch.empty_like(hk).pin_memory()
        if args.op == "swap-out":
            dst = np.arange(n)
            ks, vs, kd, vd = dw.k_pool, dw.v_pool, hk, hv
        else:
            src, dst = np.arange(n), src
            ks, vs, kd, vd = hk, hv, dw.k_pool, dw.v_pool
    mapping = torch.from_numpy(np.stack([src, dst], 1).astype(np.int64)).cuda()
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        binding.copy_blocks(ks, vs, kd, vd, mapping)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(args.steps):
        binding.copy_blocks(ks, vs, kd, vd, mapping)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    moved = 2 * n * page_bytes                    # K and V pages
    gbs = 2 * moved / (ms * 1e-3) / 1e9           # read + write
    result = {
        "metric": f"copy_blocks {args.op} GB/s (read + write)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": CONFIG_NAMES[args.config] + f"; {n} random pages per call",
                   "page_bytes_per_pool": page_bytes, "op": args.op},
    }
    if args.op == "copy":
        result["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                              "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        dev = torch.empty(moved // 2, dtype=torch.uint8, device="cuda")
        host = torch.empty(moved // 2, dtype=torch.uint8, pin_memory=True)
        pair = (dev, host) if args.op == "swap-out" else (host, dev)
        for _ in range(3):
            pair[1].copy_(pair[0], non_blocking=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(args.steps):
            pair[1].copy_(pair[0], non_blocking=True)
            pair[1].copy_(pair[0], non_blocking=True)
        b.record(stream)
        torch.cuda.synchronize()
        result["contiguous_dma_gbs_one_way"] = round(moved / (a.elapsed_time(b) / args.steps
                                                               * 1e-3) / 1e9, 1)
        result["paged_gbs_one_way"] = round(moved / (ms * 1e-3) / 1e9, 1)
    print(json.dumps(result), flush=True)


def prefill_cpu_baseline(w, budget_s):
    """The oracle's prefill, as it stands, on this host: eight evenly spaced
    chunk rows of every sequence (all heads), repeated until the budget is
    spent (at least once); rows per second."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    qs = w.query_start
    rows = np.unique(np.concatenate([
        np.linspace(qs[s], qs[s + 1] - 1, 8).astype(np.int64)
        for s in range(w.num_seqs) if qs[s + 1] > qs[s]]))
    kp, vp = oracle.reshape_and_cache(w.k_new, w.v_new, w.k_pool, w.v_pool, w.slot_mapping,
                                      w.block_size)
    runs = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while True:
            out = oracle.prefill(w.q, kp, vp, w.block_tables, w.context_lens, qs,
                                 w.num_kv_heads, w.scale, w.block_size, w.dtype, rows=rows)
            runs += 1
            if time.perf_counter() - t0 >= budget_s:
                break
    dt = (time.perf_counter() - t0) / runs
    assert np.all(np.isfinite(out[rows]))
    return {
        "value": round(len(rows) / dt, 2),
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{len(rows)} chunk rows (8 evenly spaced per sequence, all {w.num_heads} "
                  f"heads) of the same step, {runs} run(s), {dt:.2f} s per run, fp64 NumPy, "
                  f"BLAS limited to 1 thread; host has {len(os.sched_getaffinity(0))} usable "
                  f"cores ({platform.processor() or platform.machine()})",
    }


def alibi_slopes(H):
    """The geometric per-head slopes of the ALiBi paper."""
    import numpy as np
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], np.float32)


def bench_cache_rope(args):
    """reshape_and_cache_rope over every chunk row of a prefill workload
    (rotary dimension = head_dim, split-half pairs, positions 0..ctx-1),
    against the plain cache write of the same rows.  Bytes per call: q read
    and written, k and v read, K and V written to the pool, the table rows
    read (H, Hkv, D, T of the workload, 4-byte table entries)."""
    import numpy as np
    import torch
    from paged_kv_cache_457_amd import binding
    from paged_kv_cache_457_amd.device_inputs import upload
    from paged_kv_cache_457_amd.workloads import PREFILL_CONFIG_NAMES, make_prefill_config

    w = make_prefill_config(args.config, args.seed)
    dw = upload(w)
    qs, ctx = w.query_start, w.context_lens
    pos = np.concatenate([np.arange(ctx[s] - (qs[s + 1] - qs[s]), ctx[s])
                          for s in range(w.num_seqs)]).astype(np.int64)
    D = w.head_dim
    inv = 10000.0 ** (-np.arange(0, D, 2) / D)
    ang = np.arange(int(pos.max()) + 1)[:, None] * inv[None, :]
    table = torch.from_numpy(np.concatenate([np.cos(ang), np.sin(ang)], 1).astype(np.float32)).cuda()
    pos_d = torch.from_numpy(pos).cuda()
    q = dw.q.clone()
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    ms = timed(lambda: binding.reshape_and_cache_rope(q, dw.k_new, dw.v_new, dw.k_pool,
                                                      dw.v_pool, dw.slot_mapping, pos_d, table,
                                                      D, True))
    ms_plain = timed(lambda: binding.reshape_and_cache(dw.k_new, dw.v_new, dw.k_pool, dw.v_pool,
                                                       dw.slot_mapping))
    T, H, Hkv, e = w.num_tokens, w.num_heads, w.num_kv_heads, w.elem_bytes
    nbytes = T * H * D * e * 2 + T * Hkv * D * e * 4 + T * D * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "cache write with RoPE fused, GB/s",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": PREFILL_CONFIG_NAMES[args.config] + "; rot_dim = head_dim, "
                   "split-half pairs", "num_tokens": T, "op": "cache-rope"},
        "bytes_per_call": nbytes,
        "plain_cache_write_ms": round(ms_plain, 5),
        "plain_cache_write_gbs": round(T * Hkv * D * e * 4 / (ms_plain * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm", "kernel": "pa_reshape_and_cache_rope",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
    }), flush=True)


def bench_prefill(args):
    """Multi-token step: cache write of every chunk row, then prefill
    attention, through paged_attention_prefill_step (chunk rows and plan in
    one launch; --two-calls or --alibi: the two calls).  value = chunk tokens / step time; the roofline prices the
    attention pass against the dense bf16 matrix-core peak with its
    algorithmic flops (4 * head_dim per visible (row, key) pair and head)."""
    import numpy as np
    import torch
    from paged_kv_cache_457_amd import binding
    from paged_kv_cache_457_amd.device_inputs import upload
    from paged_kv_cache_457_amd.workloads import PREFILL_CONFIG_NAMES, make_prefill_config

    w = make_prefill_config(args.config, args.seed)
    dw = upload(w)
    stream = torch.cuda.current_stream()
    ps = args.partition_size or 0
    args.effective_partition = binding.paged_attention_prefill_partition_tokens(
        dw.q, dw.k_pool, dw.block_tables, dw.query_start, ps)
    ws = torch.empty(max(binding.paged_attention_prefill_workspace_bytes(
        dw.q, dw.k_pool, dw.block_tables, dw.query_start, ps), 16), dtype=torch.uint8,
        device="cuda")
    scale = float(w.scale)
    slopes = torch.from_numpy(alibi_slopes(w.num_heads)).cuda() if args.alibi else None

    fused = not (args.alibi or args.two_calls)

    def step(events=(None, None)):
        if fused:
            binding.paged_attention_prefill_step(
                dw.out, dw.q, dw.k_new, dw.v_new, dw.slot_mapping, dw.k_pool, dw.v_pool,
                dw.block_tables, dw.context_lens, dw.query_start, scale=scale, workspace=ws,
                timing_events=events, partition_size=ps)
            return
        binding.reshape_and_cache(dw.k_new, dw.v_new, dw.k_pool, dw.v_pool, dw.slot_mapping)
        binding.paged_attention_prefill(dw.out, dw.q, dw.k_pool, dw.v_pool, dw.block_tables,
                                        dw.context_lens, dw.query_start, scale=scale,
                                        workspace=ws, timing_events=events, alibi_slopes=slopes,
                                        partition_size=ps)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(end) / args.steps
    # the attention pass alone: K more steps with an event pair around it
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        src.fill_(3)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    flops = w.prefill_flops()
    tflops = flops / (k_ms * 1e-3) / 1e12
    kv_bytes = w.kv_bytes()
    result = {
        "metric": "prefill-attn tokens/s + matrix-core TFLOP/s (% of bf16 peak)",
        "value": round(w.num_tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": PREFILL_CONFIG_NAMES[args.config],
            "config_index": args.config,
            "seed": w.seed,
            "num_seqs": w.num_seqs,
            "num_tokens": w.num_tokens,
            "num_heads": w.num_heads,
            "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim,
            "block_size": w.block_size,
            "sum_context_tokens": int(w.context_lens.sum()),
            "entry": ("paged_attention_prefill_step" if fused else
                      "reshape_and_cache + paged_attention_prefill_alibi" if args.alibi else
                      "reshape_and_cache + paged_attention_prefill"),
            "partition_size": args.effective_partition,
            "parallelism": "single GPU",
        },
        "flops_per_step": flops,
        "kv_bytes_per_step": kv_bytes,
        "prefill_kernel_ms": round(k_ms, 5),
        "kv_read_gbs_kernel": round(kv_bytes / (k_ms * 1e-3) / 1e9, 1),
        "wall_s_timed_region": round(t_wall, 4),
        "roofline": {
            "bound": "mfma",
            "kernel": "pa_prefill_gqa",
            "achieved": round(tflops, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None if args.alibi else measured_traffic(args, "pa_prefill_gqa",
                                                                f"p{args.config}"),
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = prefill_cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the decode kernel shards by sequence or by kv-head with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from paged_kv_cache_457_amd import binding
    from paged_kv_cache_457_amd.device_inputs import upload
    from paged_kv_cache_457_amd.workloads import CONFIG_NAMES, make_config

    cpu_legs, w = None, None
    if args.op == "decode-step" and not args.no_cpu_baseline:
        # the oracle on the host first: the all-core leg forks worker
        # processes, which must happen before this process touches the GPU
        w = make_config(args.config, args.seed)
        cpu_legs = (cpu_baseline_all_cores(w, args.cpu_seconds),
                    cpu_baseline(w, args.cpu_seconds))
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.op == "prefill":
        bench_prefill(args)
        return
    if args.op == "cache-rope":
        bench_cache_rope(args)
        return
    if args.op != "decode-step":
        bench_copy(args)
        return
    if w is None:
        w = make_config(args.config, args.seed)
    if args.partition_size is None:
        args.partition_size = w.partition_size
    dw = upload(w)
    args.effective_partition = binding.paged_attention_decode_partition_tokens(
        dw.q, dw.k_pool, dw.block_tables, args.partition_size)
    if args.shared_prefix and not args.partition_size:
        # the shared-prefix entry's default (include/pagedattn.h)
        args.effective_partition = min(512, w.max_blocks_per_seq * w.block_size)
    stream = torch.cuda.current_stream()
    ws_bytes = binding.paged_attention_decode_workspace_bytes(dw.q, dw.k_pool, dw.block_tables,
                                                              args.partition_size)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    scale = float(w.scale)

    slopes = torch.from_numpy(alibi_slopes(w.num_heads)).cuda() if args.alibi else None
    if args.alibi and args.shared_prefix:
        print("--alibi has no shared-prefix entry point", file=sys.stderr)
        sys.exit(2)
    if args.shared_prefix:
        if "group_starts" not in w.extra:
            print("--shared-prefix needs a workload with sharing groups (config 5)",
                  file=sys.stderr)
            sys.exit(2)
        gs = torch.from_numpy(w.extra["group_starts"]).cuda()
        pl = torch.from_numpy(w.extra["prefix_lens"]).cuda()
        ws = torch.empty(max(binding.paged_attention_decode_shared_prefix_workspace_bytes(
            dw.q, dw.k_pool, dw.block_tables, args.partition_size), 16),
            dtype=torch.uint8, device="cuda")

    fused = not (args.alibi or args.two_calls)

    def step(events=(None, None)):
        if fused and args.shared_prefix:
            binding.paged_attention_decode_shared_prefix_step(
                dw.out, dw.q, dw.k_new, dw.v_new, dw.slot_mapping, dw.k_pool, dw.v_pool,
                dw.block_tables, dw.context_lens, gs, pl, scale=scale,
                partition_size=args.partition_size, workspace=ws, timing_events=events)
            return
        if fused:
            binding.paged_attention_decode_step(
                dw.out, dw.q, dw.k_new, dw.v_new, dw.slot_mapping, dw.k_pool, dw.v_pool,
                dw.block_tables, dw.context_lens, scale=scale, partition_size=args.partition_size,
                workspace=ws, timing_events=events)
            return
        binding.reshape_and_cache(dw.k_new, dw.v_new, dw.k_pool, dw.v_pool, dw.slot_mapping)
        if args.shared_prefix:
            binding.paged_attention_decode_shared_prefix(
                dw.out, dw.q, dw.k_pool, dw.v_pool, dw.block_tables, dw.context_lens, gs, pl,
                scale=scale, partition_size=args.partition_size, workspace=ws,
                timing_events=events)
            return
        binding.paged_attention_decode(dw.out, dw.q, dw.k_pool, dw.v_pool, dw.block_tables,
                                       dw.context_lens, scale=scale,
                                       partition_size=args.partition_size, workspace=ws,
                                       timing_events=events, alibi_slopes=slopes)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the timed region: K plain steps, nothing recorded inside them
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(end) / args.steps

    # then K more steps with one event pair each, recorded by the library on
    # its stream right before and after the partition kernel, and one event
    # at every step boundary (the per-step distribution)
    def event_pairs(n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for a, b in evs:
            a.record(stream)
            b.record(stream)
        return evs

    evs = event_pairs(args.steps)
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        bounds[i].record(stream)
        step(evs[i])
    bounds[-1].record(stream)
    torch.cuda.synchronize()
    k1_ms = [a.elapsed_time(b) for a, b in evs]
    k1_avg_ms = float(np.mean(k1_ms))
    step_ms = [bounds[i].elapsed_time(bounds[i + 1]) for i in range(args.steps)]

    # cold caches: before each of these steps a read of a 1 GiB buffer
    # evicts the pools from L2 and the 256 MB last-level cache; only the
    # partition kernel is timed (the library's events)
    cold_ms = None
    if args.cold_steps:
        flush = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        cev = event_pairs(args.cold_steps)
        torch.cuda.synchronize()
        for i in range(args.cold_steps):
            flush.sum()
            step(cev[i])
        torch.cuda.synchronize()
        cold_ms = [a.elapsed_time(b) for a, b in cev]
        del flush

    # the decode access pattern without its arithmetic, on the same inputs:
    # the read rate the partition kernel's loads can reach on this device
    pattern_ms = None
    if not args.shared_prefix:
        pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in pev:
            a.record(stream)
            b.record(stream)
        for _ in range(3):
            binding.paged_attention_decode_read_probe(
                dw.out, dw.q, dw.k_pool, dw.v_pool, dw.block_tables, dw.context_lens,
                partition_size=args.partition_size, workspace=ws)
        torch.cuda.synchronize()
        for a, b in pev:
            binding.paged_attention_decode_read_probe(
                dw.out, dw.q, dw.k_pool, dw.v_pool, dw.block_tables, dw.context_lens,
                partition_size=args.partition_size, workspace=ws, timing_events=(a, b))
        torch.cuda.synchronize()
        pattern_ms = float(np.mean([a.elapsed_time(b) for a, b in pev]))

    graph_ms = None
    if args.graph:
        # the same step, captured once and replayed: launches leave the host path
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        ga = torch.cuda.Event(enable_timing=True)
        gb = torch.cuda.Event(enable_timing=True)
        ga.record(stream)
        for _ in range(args.steps):
            g.replay()
        gb.record(stream)
        torch.cuda.synchronize()
        graph_ms = ga.elapsed_time(gb) / args.steps
        del g

    kv_bytes = w.kv_bytes()
    # the shared-prefix pass must read each physical page once: its
    # algorithmic bytes are the unique bytes
    kernel_bytes = w.unique_kv_bytes() if args.shared_prefix else kv_bytes
    achieved = kernel_bytes / (k1_avg_ms * 1e-3) / 1e9
    kernel = "pa_decode_prefix_gqa" if args.shared_prefix else dominant_kernel(w)
    traffic = None if args.alibi else measured_traffic(args, kernel)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        src.fill_(3)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    probe_gbs = None
    if args.probe:
        buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
        buf.fill_(1)
        sink = binding.hbm_read_probe(buf)
        torch.cuda.synchronize()
        pa, pb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        pa.record(stream)
        for _ in range(10):
            binding.hbm_read_probe(buf, sink)
        pb.record(stream)
        torch.cuda.synchronize()
        probe_gbs = buf.numel() * 10 / (pa.elapsed_time(pb) * 1e-3) / 1e9
        del buf

    result = {
        "metric": "decode-attn tokens/s + KV-read HBM GB/s (% of peak), Llama-2-7B shape, bs=64",
        "value": round(w.num_seqs / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": CONFIG_NAMES[args.config],
            "config_index": args.config,
            "seed": w.seed,
            "num_seqs": w.num_seqs,
            "num_heads": w.num_heads,
            "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim,
            "block_size": w.block_size,
            "sum_context_tokens": int(w.context_lens.sum()),
            "num_blocks": w.num_blocks,
            "partition_size": args.effective_partition,
            "decode_entry": ("paged_attention_decode_shared_prefix_step" if args.shared_prefix
                             else "paged_attention_decode_step") if fused else
            ("reshape_and_cache + " + ("paged_attention_decode_shared_prefix" if args.shared_prefix
             else "paged_attention_decode_alibi" if args.alibi else "paged_attention_decode")),
            "parallelism": "single GPU",
        },
        "kv_bytes_per_step": kv_bytes,
        "kernel_bytes_per_launch": kernel_bytes,
        "kv_read_gbs_step": round(kv_bytes / (ms_step * 1e-3) / 1e9, 1),
        "kv_read_frac_of_peak_step": round(kv_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "partition_kernel_ms": round(k1_avg_ms, 5),
        "step_ms_percentiles": _percentiles(step_ms),
        "partition_kernel_ms_percentiles": _percentiles(k1_ms),
        **({"graph_ms_per_step": round(graph_ms, 5),
            "graph_tokens_per_s": round(w.num_seqs / (graph_ms * 1e-3), 1)} if graph_ms else {}),
        "wall_s_timed_region": round(t_wall, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
    }
    if pattern_ms:
        pattern_gbs = kv_bytes / (pattern_ms * 1e-3) / 1e9
        result["decode_pattern_probe"] = {
            "kernel_ms": round(pattern_ms, 5),
            "read_gbs": round(pattern_gbs, 1),
            "partition_kernel_frac_of_probe": round(achieved / pattern_gbs, 4),
        }
    if cold_ms:
        cold_p50 = float(np.median(cold_ms))
        cold_gbs = kernel_bytes / (cold_p50 * 1e-3) / 1e9
        result["cold_cache"] = {
            "flush": "1 GiB read before each step (L2 and the 256 MB last-level cache)",
            "steps": args.cold_steps,
            "partition_kernel_ms_percentiles": _percentiles(cold_ms),
            "achieved_gbs_p50": round(cold_gbs, 1),
            "frac_of_peak_p50": round(cold_gbs / HBM_PEAK_GBS, 4),
        }
    if w.unique_kv_bytes() != kv_bytes:
        result["unique_kv_read_gbs_step"] = round(w.unique_kv_bytes() / (ms_step * 1e-3) / 1e9, 1)
    if probe_gbs is not None:
        result["probe_read_gbs"] = round(probe_gbs, 1)
    if cpu_legs:
        result["cpu_baseline"], result["cpu_baseline_one_core"] = cpu_legs
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
