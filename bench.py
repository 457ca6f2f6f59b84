#!/usr/bin/env python3
"""Verify-step latency of libswattn on one MI355X, as one JSON line.

Workload (one "step" = one swattn_verify call): a single stream's verify step
with 24 layers of KV stacked along the batch axis — 8 query heads sharing 2 KV
heads, head_dim 256, bf16 Q/K/V ~ N(0, 1), context 4096, window 188, 8 queries
(target + 7 drafts), paged KV with 16-position blocks and a shuffled block
table, seed 1.  Inputs are resident in HBM before timing starts.

Timing: ``--warmup`` untimed calls, then ``--steps`` timed calls captured in
one HIP graph (the serving loop's way of launching), each preceded by an
overwrite of 512 MiB and a read of another 512 MiB, so that the 256 MB Infinity
Cache and the L2s hold nothing of the inputs and no dirty line of the overwrite
is left to write back during the call (cold cache).  The same graph without the
calls is timed as well;
``value`` is the difference divided by the number of calls (median of 3
replays), i.e. the cold per-call time as the kernel trace sees it.  Also
reported: eager calls bracketed one by one with HIP events (adds dispatch
latency), warm back-to-back calls, and warm calls replayed from one graph.

``roofline``: algorithmic bytes (each sequence's union window of keys, both
KV heads, K and V, plus Q and the output once) over the measured time, against
MI355X's 8 TB/s HBM peak.  ``traffic`` comes from the FETCH_SIZE / WRITE_SIZE
counter summary committed under profiles/ when it was taken on the current
kernel source, else null.  ``cpu_baseline``: the float64 oracle on this host.

Usage: python bench.py [--gpus 1] [--steps 200] [--warmup 20]
       [--workload verify|decode|batched_fp8|batched_bf16|wide_verify|fullctx_*|tiny_decode|prefill_512]
       [--op attention|append_kv|accept|layer_graph|gather_ceiling|read_ceiling]
"""
import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
WORKLOAD = "verify"
DESCRIPTIONS = {
    "verify": "single-stream verify: 24 layers x (8 q heads / 2 kv heads), head_dim 256, bf16, "
              "ctx 4096, window 188, n_q 8, paged block 16 (shuffled), seed 1",
    "batched_fp8": "batched stress: 256 sequences x (8 q heads / 2 kv heads), head_dim 256, e4m3 KV "
                   "(per-head scale), bf16 Q/out, ctx ~ U[188, 4096], window 188, n_q 8, block 16, seed 4",
    "batched_bf16": "batched stress: 256 sequences x (8 q / 2 kv heads), head_dim 256, bf16, "
                    "ctx ~ U[188, 4096], window 188, n_q 8, block 16, seed 4",
    "wide_verify": "wide verify: 24 layers x (8 q / 2 kv heads), head_dim 256, bf16, ctx 4096, window 188, "
                   "n_q 64, 5% of Q rows x8, block 16, seed 3",
    "prefill_512": "chunked prefill: 24 layers x (8 q / 2 kv heads), head_dim 256, bf16, the last 512-token "
                   "chunk of a 4096-token prompt, window 188, block 16, seed 5",
    "decode": "single-stream plain decode: 24 layers x (8 q heads / 2 kv heads), head_dim 256, bf16, "
              "ctx 4096, window 188, n_q 1, paged block 16 (shuffled), seed 6",
}
# HBM-counter summaries (profiles/) of the workloads that have one
TRAFFIC_SUMMARIES = {
    "verify": os.path.join(ROOT, "profiles", "traffic_verify_24x2kv_d256_w188_nq8.txt"),
    "batched_fp8": os.path.join(ROOT, "profiles", "traffic_batched_256seq_2kv_d256_e4m3_w188_nq8.txt"),
    "batched_bf16": os.path.join(ROOT, "profiles", "traffic_batched_256seq_2kv_d256_bf16_w188_nq8.txt"),
    "decode": os.path.join(ROOT, "profiles", "traffic_decode_24x2kv_d256_w188_nq1.txt"),
    "wide_verify": os.path.join(ROOT, "profiles", "traffic_wideverify_24x2kv_d256_w188_nq64.txt"),
    "prefill_512": os.path.join(ROOT, "profiles", "traffic_prefill_24x2kv_d256_w188_nq512.txt"),
    "fullctx_4096": os.path.join(ROOT, "profiles", "traffic_fullctx_24x2kv_d256_w4096_ctx4096_nq8.txt"),
    "tiny_decode": os.path.join(ROOT, "profiles", "traffic_tinydecode_1x1kv_d64_f32_w188_nq1.txt"),
}
KERNEL_SOURCES = ["partition_mfma.hip", "partition_valu.hip", "merge.hip", "split_merge.h", "kv_access.h",
                  "swattn_internal.h", "plan.cpp", "api.cpp"]


def algorithmic_bytes(w, out_elt=None):
    """Bytes the method must move for one call: every sequence's union window of
    keys, min(ctx, window + n_q - 1) positions, for each KV head, K and V, plus Q
    and the output once (partial blocks, block table and split workspace are not
    counted)."""
    import numpy as np
    kv_elt = {"f32": 4, "bf16": 2, "e4m3": 1}[w.kv_dtype]
    q_elt = {"f32": 4, "bf16": 2}[w.q_dtype]
    o_elt = q_elt if out_elt is None else out_elt
    keys = int(np.minimum(w.ctx_len.astype(np.int64), w.window + w.n_q - 1).sum())
    return (keys * w.Hkv * w.D * kv_elt * 2 + w.B * w.n_q * w.H * w.D * q_elt
            + w.B * w.n_q * w.H * w.D * o_elt)


def _code_only(text):
    """Source text without // and /* */ comments, trailing blanks and empty lines (the
    kernel sources hold no comment markers inside string literals)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def source_hash():
    """Hash of the code (not the comments) of the sources that decide the kernels' traffic."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "speculative_verify_kv_amd", "csrc", name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload="verify"):
    """HBM bytes per call from the workload's committed counter summary, or None when
    there is none or it was taken on other kernel sources."""
    path = TRAFFIC_SUMMARIES.get(workload)
    if path is None or not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_hash") != source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def _cpu_info():
    """CPU model, CPUs this process may run on, and the cgroup CPU quota in CPUs (None
    when unlimited or unknown)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    quota = None
    try:                                          # cgroup v2: "<quota> <period>" or "max <period>"
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, per = f.read().split()[:2]
            if q != "max":
                quota = float(q) / float(per)
    except (OSError, ValueError):
        try:                                      # cgroup v1
            with open("/sys/fs/cgroup/cpu/cpu.cfs_quota_us") as f:
                q = float(f.read())
            with open("/sys/fs/cgroup/cpu/cpu.cfs_period_us") as f:
                per = float(f.read())
            if q > 0:
                quota = q / per
        except (OSError, ValueError):
            pass
    return model, len(os.sched_getaffinity(0)), quota


_POOL_W = None


def _pool_init(key):
    """Worker of the CPU-baseline pool: one BLAS thread, the workload rebuilt from its seed."""
    global _POOL_W
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:
        pass
    import synth
    _POOL_W = synth.named_workload(key)
    try:                                          # numpy is loaded now: limit its BLAS too
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:
        pass


def _pool_slice(b0, b1):
    import oracle
    w = _POOL_W
    oracle.attend(w.q[b0:b1], w.k_cache, w.v_cache, w.block_table[b0:b1], w.ctx_len[b0:b1], w.n_q, w.window,
                  w.scale, q_format=w.q_format, kv_format=w.kv_format, k_scale=w.k_scale, v_scale=w.v_scale)
    return b1 - b0


def _time_reps(fn, budget_s, max_reps):
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= max_reps:
            return times


def cpu_baseline(key, budget_s):
    """The float64 oracle on this host's cores, on the whole workload (one call = every
    sequence), three ways: one BLAS thread; every allowed core as BLAS threads (the
    oracle's loops are over small matrix-vector products, so few of them engage); and
    the unmodified oracle over disjoint slices of the sequences in a pool of one
    process per allowed core (at most 16).  ``value`` is the pool's wall time per call.
    Runs before the GPU is touched.  Returns None when no oracle call fits the budget."""
    import multiprocessing as mp
    import oracle
    import synth
    from threadpoolctl import threadpool_limits
    w = synth.named_workload(key)
    model, allowed, quota = _cpu_info()

    def call():
        oracle.attend(w.q, w.k_cache, w.v_cache, w.block_table, w.ctx_len, w.n_q, w.window, w.scale,
                      q_format=w.q_format, kv_format=w.kv_format, k_scale=w.k_scale, v_scale=w.v_scale)

    with threadpool_limits(limits=1):
        t1 = _time_reps(call, budget_s / 3, 5)
    with threadpool_limits(limits=allowed):
        c0 = time.process_time()
        tall = _time_reps(call, budget_s / 3, 5)
        eff = (time.process_time() - c0) / max(sum(tall), 1e-9)
    # one process per CPU the process may use: allowed CPUs, capped by the cgroup quota
    usable = allowed if quota is None else max(1, min(allowed, int(quota)))
    workers = max(1, min(usable, 16))
    per_task = max(1, -(-w.B // (4 * workers)))
    tasks = [(b, min(w.B, b + per_task)) for b in range(0, w.B, per_task)]
    # The workers are fresh interpreters: their BLAS reads its thread count from the
    # environment when numpy loads, so one thread each is set there (with 16 BLAS threads
    # per worker the pool oversubscribes the CPUs).
    thread_vars = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS")
    saved = {k: os.environ.get(k) for k in thread_vars}
    os.environ.update({k: "1" for k in thread_vars})
    try:
        with mp.get_context("spawn").Pool(workers, initializer=_pool_init, initargs=(key,)) as pool:
            pool.starmap(_pool_slice, tasks)          # every worker built its workload
            tpool = _time_reps(lambda: pool.starmap(_pool_slice, tasks), budget_s / 3, 20)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    us = lambda ts: round(statistics.median(ts) * 1e6, 1)
    return {"value": us(tpool), "unit": "us/call", "cores": workers, "kind": "oracle",
            "sample": f"whole workload per call ({w.B} sequences); process pool: {workers} processes x 1 BLAS "
                      f"thread over {len(tasks)} slices of sequences, median of {len(tpool)} calls",
            "single_thread": {"value": us(t1), "unit": "us/call", "reps": len(t1)},
            "blas_all_threads": {"value": us(tall), "unit": "us/call", "blas_threads": allowed,
                                 "effective_cores": round(eff, 2), "reps": len(tall)},
            "cpu_model": model, "host_cpus_allowed": allowed, "cgroup_cpu_quota": quota,
            "pool_speedup_vs_single_thread": round(us(t1) / max(us(tpool), 1e-9), 2)}


class ColdFlush:
    """Puts the caches in a cold, clean state before a timed call: 512 MiB written
    (twice the 256 MiB Infinity Cache, so nothing of the call's inputs stays cached),
    then one byte of every 64-byte line of another 512 MiB read, which evicts the
    written lines and makes their write-back happen here rather than inside the
    timed call.  write_only() is the first half alone."""

    def __init__(self, torch, dev):
        self.w = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        self.r = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
        self.sink = torch.empty((512 << 20) // 64, dtype=torch.uint8, device=dev)

    def write_only(self):
        self.w.zero_()

    def __call__(self):
        self.w.zero_()
        self.sink.copy_(self.r.view(-1, 64)[:, 0])


def time_calls(torch, dev, stream, launch, flush, steps, with_graph):
    """Per-call times of ``launch(stream_handle)`` (one library call):

    cold_graph: ``steps`` calls captured in one HIP graph, each after ``flush()``
    (see ColdFlush), minus the same graph without the calls, over ``steps`` (median
    of three replays); cold_graph_dirty: the same with the write half of the flush
    only, so that the write-back of 512 MiB of dirty lines overlaps the call;
    cold_eager: HIP events around each eager call (adds dispatch latency); warm:
    back to back, and replayed from a graph of 100 calls."""
    def cold_per_call(pre):
        def capture(with_calls):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cs = torch.cuda.current_stream(dev).cuda_stream
                for _ in range(steps):
                    pre()
                    if with_calls:
                        launch(cs)
            return g

        g_pair, g_flush = capture(True), capture(False)
        g_pair.replay()
        g_flush.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        per_call = []
        wall = 0.0
        for _ in range(3):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            ev[0].record(stream)
            g_pair.replay()
            ev[1].record(stream)
            torch.cuda.synchronize()
            wall += time.perf_counter() - t0
            ev[2].record(stream)
            g_flush.replay()
            ev[3].record(stream)
            torch.cuda.synchronize()
            per_call.append((ev[0].elapsed_time(ev[1]) - ev[2].elapsed_time(ev[3])) * 1e3 / steps)
        return statistics.median(per_call), per_call, wall

    cold_graph, per_call, wall = cold_per_call(flush)
    cold_dirty, _, _ = cold_per_call(flush.write_only)

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        flush()
        starts[i].record(stream)
        launch(stream.cuda_stream)
        ends[i].record(stream)
    torch.cuda.synchronize()
    cold = sorted(s_.elapsed_time(e_) * 1e3 for s_, e_ in zip(starts, ends))   # us

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        launch(stream.cuda_stream)
    e1.record(stream)
    torch.cuda.synchronize()
    warm = e0.elapsed_time(e1) * 1e3 / steps

    graph_us = None
    if with_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream(dev).cuda_stream
            for _ in range(100):
                launch(cs)
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(5):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_us = e0.elapsed_time(e1) * 1e3 / 500
    return {
        "cold_graph_us_per_call": round(cold_graph, 3),
        "cold_graph_samples_us": [round(x, 3) for x in per_call],
        "cold_graph_dirty_us_per_call": round(cold_dirty, 3),
        "cold_eager_us_median": round(statistics.median(cold), 3),
        "cold_eager_us_p10": round(cold[int(0.1 * (len(cold) - 1))], 3),
        "cold_eager_us_p90": round(cold[int(0.9 * (len(cold) - 1))], 3),
        "warm_us_back_to_back": round(warm, 3),
        "graph_us_per_call_warm": None if graph_us is None else round(graph_us, 3),
        "timed_region_wall_s": round(wall, 4),
        "note": "value = cold_graph: K calls in one HIP graph, each after a 512 MiB overwrite and "
                "a 512 MiB read (inputs in HBM only, no dirty lines pending), minus the same graph "
                "without the calls, over K; cold_graph_dirty: the overwrite alone; cold_eager = HIP "
                "events around each eager call (adds dispatch latency)",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--splits", type=int, default=0, help="force the KV split count (0 = library)")
    ap.add_argument("--workload", default=WORKLOAD, help="named synthetic workload (default: verify)")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="default workload only: skip the batched-configuration measurements")
    ap.add_argument("--op", default="attention",
                    choices=["attention", "append_kv", "accept", "layer_graph", "gather_ceiling", "read_ceiling"],
                    help="attention: swattn_verify / swattn_prefill (default); append_kv: swattn_append_kv "
                         "of the workload's new rows into its cache; accept: swattn_greedy_accept; "
                         "layer_graph: one decode step as a graph of per-layer calls; gather_ceiling: "
                         "swattn_window_gather, the workload's data movement without arithmetic; "
                         "read_ceiling: swattn_stream_read, a contiguous read of the workload's byte count")
    ap.add_argument("--vocab", type=int, default=262144, help="accept op: logits per position")
    ap.add_argument("--accept-batch", type=int, default=1, help="accept op: sequences per call")
    ap.add_argument("--gather-parts", type=int, default=1,
                    help="gather_ceiling op: workgroups per (problem, KV head), each a slice of its rows")
    ap.add_argument("--unshuffled", action="store_true",
                    help="attention and gather_ceiling ops: identity block tables (each sequence's blocks in "
                         "order) instead of the workload's shuffled ones")
    ap.add_argument("--window", type=int, default=0,
                    help="attention and gather ops: another window for the window-188 workloads (their "
                         "random recent rows follow it)")
    ap.add_argument("--read-grid", type=int, default=512,
                    help="read_ceiling op: workgroups of the contiguous read (two per CU by default)")
    ap.add_argument("--calibrate-copy", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this library runs on one GPU; multi-GPU runs are not part of it "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    # the oracle's CPU baseline runs first, before anything touches the GPU
    cpu = None
    if args.op == "attention" and not args.no_cpu_baseline and not args.calibrate_copy:
        cpu = cpu_baseline(args.workload, args.cpu_budget)

    import numpy as np
    import torch
    import speculative_verify_kv_amd as sw
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n}))
        return

    if args.op == "append_kv":
        run_append(args, torch, np, sw, synth, dev)
        return
    if args.op == "accept":
        run_accept(args, torch, np, sw, dev)
        return
    if args.op == "layer_graph":
        run_layer_graph(args, torch, np, sw, synth, dev)
        return
    if args.op == "gather_ceiling":
        r = measure_attention(args.workload, args, torch, np, sw, synth, dev, gather=True)
        line = {"metric": "data-movement floor us/call (swattn_window_gather: the verify call's algorithmic bytes "
                          "through the same paged loads, no arithmetic)",
                "value": r["value"], "unit": "us/call", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                "ms_per_step": round(r["value"] / 1e3, 6), "higher_is_better": False, "scaling": "weak",
                "vs_baseline": None, "dtype": r["dtype"], "data": "synthetic", "config": r["config"],
                "roofline": r["roofline"], "timing": r["timing"], "cpu_baseline": None,
                "gather_parts": args.gather_parts}
        print(json.dumps(line), flush=True)
        return
    if args.op == "read_ceiling":
        r = measure_read(args.workload, args, torch, np, sw, synth, dev)
        line = {"metric": "HBM read floor us/call (swattn_stream_read: a contiguous read of the verify call's "
                          "algorithmic byte count)",
                "value": r["value"], "unit": "us/call", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                "ms_per_step": round(r["value"] / 1e3, 6), "higher_is_better": False, "scaling": "weak",
                "vs_baseline": None, "dtype": "u8", "data": "synthetic", "config": r["config"],
                "roofline": r["roofline"], "timing": r["timing"], "xor_check": r["xor_check"],
                "cpu_baseline": None, "read_grid": args.read_grid}
        print(json.dumps(line), flush=True)
        if not r["xor_check"]["ok"]:
            print("bench.py: the contiguous read's xor check failed", file=sys.stderr)
            sys.exit(1)
        return

    res = measure_attention(args.workload, args, torch, np, sw, synth, dev)
    line = {
        "metric": "verify-step us/call (W=188, n_q=8) + achieved HBM GB/s as % of MI355X peak",
        "value": res["value"],
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["value"] / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": res["dtype"],
        "data": "synthetic",
        "config": res["config"],
        "roofline": res["roofline"],
        "timing": res["timing"],
        "plan": res["plan"],
        "parity_spot_check": res["parity_spot_check"],
        "cpu_baseline": cpu,
    }
    ok = res["parity_spot_check"]["ok"]
    if args.workload == WORKLOAD and not args.no_extra:
        # the same bytes without arithmetic, spread over four workgroups per (layer, KV head)
        # (the fastest spread measured; the kernel's four workgroups re-read their unit's K)
        c = measure_attention(args.workload, args, torch, np, sw, synth, dev, gather=True, gather_parts=4)
        line["gather_ceiling"] = {"value": c["value"], "unit": "us/call", "frac": c["roofline"]["frac"],
                                  "parts": 4,
                                  "what": "swattn_window_gather on the same inputs, four workgroups per "
                                          "(layer, KV head): the algorithmic bytes and paged loads, no arithmetic"}
        c = measure_read(args.workload, args, torch, np, sw, synth, dev)
        line["read_ceiling"] = _read_summary(c)
        ok = ok and c["xor_check"]["ok"]
        # the batched configuration carries the bandwidth target: measured in the same run
        line["batched"] = {}
        for key in ("batched_fp8", "batched_bf16"):
            r = measure_attention(key, args, torch, np, sw, synth, dev)
            c = measure_attention(key, args, torch, np, sw, synth, dev, gather=True, gather_parts=1)
            line["batched"][key] = {"value": r["value"], "unit": "us/call", "dtype": r["dtype"],
                                    "workload": r["config"]["workload"], "roofline": r["roofline"],
                                    "cold_eager_us_median": r["timing"]["cold_eager_us_median"],
                                    "plan": r["plan"], "parity_spot_check": r["parity_spot_check"],
                                    "gather_ceiling": {"value": c["value"], "unit": "us/call",
                                                       "frac": c["roofline"]["frac"], "parts": 1,
                                                       "what": "swattn_window_gather on the same inputs: the same "
                                                               "bytes and paged loads, no arithmetic (one "
                                                               "workgroup per unit; more measured slower)"}}
            c = measure_read(key, args, torch, np, sw, synth, dev)
            line["batched"][key]["read_ceiling"] = _read_summary(c)
            ok = ok and r["parity_spot_check"]["ok"] and c["xor_check"]["ok"]
    print(json.dumps(line), flush=True)
    if not ok:
        print("bench.py: the spot check against the oracle failed", file=sys.stderr)
        sys.exit(1)


def workload_of(key, args, synth):
    """The named workload, with the --unshuffled and --window overrides applied (tiny
    decode's single block is in order already; full context and tiny decode keep their
    windows)."""
    kw = {}
    if getattr(args, "unshuffled", False) and key != "tiny_decode":
        kw["shuffle"] = False
    if getattr(args, "window", 0):
        if key == "tiny_decode" or key.startswith("fullctx"):
            raise SystemExit(f"bench.py: --window does not apply to {key}")
        kw["window"] = args.window
    return synth.named_workload(key, **kw)


def _read_summary(c):
    return {"value": c["value"], "unit": "us/call", "frac": c["roofline"]["frac"], "grid": c["grid"],
            "what": "swattn_stream_read: a contiguous read of the same algorithmic byte count by every CU "
                    "(no block table, no per-unit workgroups): the time HBM alone sets"}


def measure_read(key, args, torch, np, sw, synth, dev):
    """Cold per-call time of swattn_stream_read over a contiguous device buffer of the
    workload's algorithmic byte count (the floor HBM sets for that many bytes), timed
    as the attention op in its read-only form; one call with the xor buffer is checked
    against the host's xor first."""
    w = workload_of(key, args, synth)
    nbytes = algorithmic_bytes(w) // 16 * 16
    grid = getattr(args, "read_grid", 512)
    host = np.random.default_rng(11).integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    x = torch.from_numpy(host.view(np.int32)).to(dev)
    xors = torch.zeros(grid * 4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def launch(cs):
        # timed without the xor buffer: the reads alone
        sw.swattn_stream_read(x, nbytes, grid, None, cs)

    # the same reads once with the workgroups' xors, checked against the host's
    sw.swattn_stream_read(x, nbytes, grid, xors, stream.cuda_stream)
    flush = ColdFlush(torch, dev)
    for _ in range(args.warmup):
        flush()
        launch(stream.cuda_stream)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(xors.cpu().numpy().view(np.uint32).reshape(grid, 4), axis=0)
    want = np.bitwise_xor.reduce(host.reshape(-1, 4), axis=0) if nbytes else np.zeros(4, np.uint32)
    t = time_calls(torch, dev, stream, launch, flush, args.steps, not args.no_graph)
    cold_graph = t["cold_graph_us_per_call"]
    achieved = nbytes / (cold_graph * 1e-6) / 1e9
    res = {"value": round(cold_graph, 3), "grid": grid,
           "config": {"workload": DESCRIPTIONS.get(key, w.name), "bytes": nbytes},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "algorithmic_bytes": nbytes,
                        "kernel": "stream_read"},
           "timing": t,
           "xor_check": {"ok": bool(np.array_equal(got, want)),
                         "what": "xor of every 16-byte chunk read, from the workgroups' results, against the host"}}
    del x, xors, flush
    torch.cuda.empty_cache()
    return res


def measure_attention(key, args, torch, np, sw, synth, dev, gather=False, gather_parts=None):
    """Cold per-call time of swattn_verify (or swattn_prefill for chunks above 64
    positions) on a named workload, its roofline fraction and an oracle spot check;
    with gather=True, of swattn_window_gather on the same inputs (no spot check)."""
    import oracle
    w = workload_of(key, args, synth)

    def to_dev(a, fmt):
        if fmt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    q = to_dev(w.q, w.q_dtype)
    k = to_dev(w.k_cache, w.kv_dtype)
    v = to_dev(w.v_cache, w.kv_dtype)
    ks = None if w.k_scale is None else torch.from_numpy(w.k_scale).to(dev)
    vs = None if w.v_scale is None else torch.from_numpy(w.v_scale).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    ctx = torch.from_numpy(w.ctx_len).to(dev)
    max_ctx = int(w.ctx_len.max())
    desc = sw.make_desc(q, k, bt, max_ctx, k_scale=ks, v_scale=vs, num_splits=args.splits)
    # a chunk of more than 64 new positions is a prefill chunk: same attention, other entry point
    prefill = w.n_q > sw.SWATTN_MAX_NQ
    plan = (sw.swattn_prefill_plan if prefill else sw.swattn_plan)(desc, w.n_q, w.window)
    call_lib = sw.swattn_prefill if prefill else sw.swattn_verify
    out = torch.empty(q.shape, dtype=torch.float32 if w.q_dtype == "f32" else torch.bfloat16, device=dev)
    ws = torch.zeros(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def launch(cs):
        if gather:
            sw.swattn_window_gather(desc, q, k, v, bt, ctx, w.n_q, w.window,
                                    args.gather_parts if gather_parts is None else gather_parts, out, cs)
        else:
            call_lib(desc, q, k, v, bt, ctx, w.n_q, w.window, w.scale, out, ws, plan.workspace_bytes, cs)

    flush = ColdFlush(torch, dev)
    for _ in range(args.warmup):
        flush()
        launch(stream.cuda_stream)
    torch.cuda.synchronize()

    # Spot check against the oracle on a few sampled sequences (every query and head).
    got = out.float().cpu().numpy()
    rng = np.random.default_rng(0)
    worst = 0.0
    for b in (rng.choice(w.B, size=min(3, w.B), replace=False) if not gather else []):
        ref = oracle.attend(w.q[b:b + 1], w.k_cache, w.v_cache, w.block_table[b:b + 1], w.ctx_len[b:b + 1], w.n_q,
                            w.window, w.scale, q_format=w.q_format, kv_format=w.kv_format,
                            k_scale=w.k_scale, v_scale=w.v_scale)
        worst = max(worst, float((np.abs(got[b:b + 1] - ref) - 1e-2 * np.abs(ref)).max()))
    parity_ok = bool(np.isfinite(worst)) and worst <= (2e-2 if w.kv_dtype == "e4m3" else 2e-3)

    t = time_calls(torch, dev, stream, launch, flush, args.steps, not args.no_graph)
    cold_graph = t["cold_graph_us_per_call"]
    nbytes = algorithmic_bytes(w)
    achieved = nbytes / (cold_graph * 1e-6) / 1e9
    config = {"workload": DESCRIPTIONS.get(key, w.name), "global_batch": w.B, "seq_len": int(max_ctx),
              "parallelism": "none (1 GPU)"}
    if not w.meta.get("shuffle", True) and key != "tiny_decode":
        config["block_table"] = "identity (--unshuffled)"
    if getattr(args, "window", 0):
        config["window"] = f"{w.window} (--window)"
    res = {
        "value": round(cold_graph, 3),
        "dtype": w.kv_dtype if w.kv_dtype != w.q_dtype else w.q_dtype,
        "config": config,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_traffic(key),
                     "algorithmic_bytes": nbytes,
                     "kernel": "window_gather" if gather else
                     "partition" + ("" if plan.num_splits == 1 or plan.fused_merge else "+merge")},
        "timing": t,
        "plan": plan.as_dict(),
        "parity_spot_check": {"ok": parity_ok, "worst_excess": worst,
                              "what": "3 sampled sequences, every query and head, |got-ref| - 1e-2|ref| "
                                      "against the absolute bound"},
    }
    del q, k, v, out, ws, flush
    torch.cuda.empty_cache()
    return res


def run_append(args, torch, np, sw, synth, dev):
    """swattn_append_kv of the workload's n_q new rows per sequence (bfloat16 K and V,
    N(0,1)) into its paged cache (the workload's cache type: bfloat16, or E4M3 with its
    per-head scales).  Same timing as the attention op; the written caches are compared
    byte for byte with the oracle."""
    import oracle
    w = synth.named_workload(args.workload)
    B, n, Hkv, D = w.B, w.n_q, w.Hkv, w.D
    rng = np.random.default_rng(7)
    x = rng.standard_normal((B, n, Hkv, D)).astype(np.float32)
    kn, vn = oracle.f32_to_bf16_rne(x), oracle.f32_to_bf16_rne(-0.5 * x)

    def dev_arr(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    k, v = dev_arr(w.k_cache), dev_arr(w.v_cache)
    kn_d, vn_d = dev_arr(kn), dev_arr(vn)
    bt, ctx = dev_arr(w.block_table), dev_arr(w.ctx_len)
    ks = None if w.k_scale is None else dev_arr(np.asarray(w.k_scale, np.float32))
    vs = None if w.v_scale is None else dev_arr(np.asarray(w.v_scale, np.float32))
    d = sw.swattn_desc_t()
    d.batch, d.num_heads, d.num_kv_heads, d.head_dim = B, w.H, Hkv, D
    d.block_size, d.max_blocks_per_seq, d.num_blocks = w.bs, w.block_table.shape[1], w.k_cache.shape[0]
    d.max_ctx_len = int(w.ctx_len.max())
    d.q_dtype, d.out_dtype = sw.SWATTN_BF16, sw.SWATTN_BF16
    d.kv_dtype = {"bf16": sw.SWATTN_BF16, "e4m3": sw.SWATTN_FP8_E4M3, "f32": sw.SWATTN_F32}[w.kv_dtype]
    d.k_scale = None if ks is None else ks.data_ptr()
    d.v_scale = None if vs is None else vs.data_ptr()
    stream = torch.cuda.current_stream(dev)

    def launch(cs):
        sw.swattn_append_kv(d, kn_d, vn_d, sw.SWATTN_BF16, bt, ctx, n, k, v, cs)

    flush = ColdFlush(torch, dev)
    for _ in range(args.warmup):
        launch(stream.cuda_stream)
    torch.cuda.synchronize()
    ek, ev = oracle.append_kv(w.k_cache, w.v_cache, w.block_table, w.ctx_len, kn, vn, n, new_format="bf16",
                              kv_format=w.kv_format, k_scale=w.k_scale, v_scale=w.v_scale,
                              max_ctx=int(w.ctx_len.max()))
    gk, gv = k.cpu().numpy(), v.cpu().numpy()
    parity_ok = (np.array_equal(gk.view(np.uint8), np.ascontiguousarray(ek).view(np.uint8)) and
                 np.array_equal(gv.view(np.uint8), np.ascontiguousarray(ev).view(np.uint8)))

    t = time_calls(torch, dev, stream, launch, flush, args.steps, not args.no_graph)
    value = t["cold_graph_us_per_call"]
    kv_elt = {"bf16": 2, "e4m3": 1, "f32": 4}[w.kv_dtype]
    nbytes = 2 * B * n * Hkv * D * (2 + kv_elt)               # read the new rows, write the cache rows
    achieved = nbytes / (value * 1e-6) / 1e9
    line = {
        "metric": "KV append us/call (n_new rows of every sequence into the paged cache)",
        "value": value, "unit": "us/call", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(value / 1e3, 6), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": f"bf16->{w.kv_dtype}", "data": "synthetic",
        "config": {"workload": "KV append of the new rows of: " + DESCRIPTIONS.get(args.workload, w.name),
                   "global_batch": B, "seq_len": int(w.ctx_len.max()), "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "algorithmic_bytes": nbytes,
                     "kernel": "kv_append"},
        "timing": t,
        "parity_check": {"ok": bool(parity_ok), "what": "whole K and V caches, byte for byte, vs oracle.append_kv"},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        times = []
        t_start = time.perf_counter()
        while time.perf_counter() - t_start < args.cpu_budget and len(times) < 5:
            t0 = time.perf_counter()
            oracle.append_kv(w.k_cache, w.v_cache, w.block_table, w.ctx_len, kn, vn, n, new_format="bf16",
                             kv_format=w.kv_format, k_scale=w.k_scale, v_scale=w.v_scale)
            times.append(time.perf_counter() - t0)
        line["cpu_baseline"] = {"value": round(statistics.median(times) * 1e6, 1), "unit": "us/call", "cores": 1,
                                "kind": "oracle", "sample": f"whole workload, {len(times)} run(s), median"}
    print(json.dumps(line), flush=True)


def run_accept(args, torch, np, sw, dev):
    """swattn_greedy_accept on one verify step's target logits: --accept-batch sequences
    x 8 positions x --vocab bfloat16 logits ~ N(0, 1), seed 6, with drafts that agree
    with the target for a random prefix.  Same timing as the attention op; the outputs
    are compared exactly with the oracle."""
    import oracle
    B, n_q, vocab = args.accept_batch, 8, args.vocab
    rng = np.random.default_rng(6)
    x = rng.standard_normal((B, n_q, vocab)).astype(np.float32)
    bits = oracle.f32_to_bf16_rne(x)
    vals = (bits.astype(np.uint32) << 16).view(np.float32)
    target = oracle.row_argmax(vals)
    drafts = target[:, :n_q - 1].astype(np.int32).copy()
    cut = rng.integers(0, n_q, B)
    for b in range(B):
        if cut[b] < n_q - 1:
            drafts[b, cut[b]] = (drafts[b, cut[b]] + 1) % vocab
    logits = torch.from_numpy(bits.view(np.int16)).to(dev)
    d = torch.from_numpy(drafts).to(dev)
    tgt = torch.empty((B, n_q), dtype=torch.int32, device=dev)
    acc = torch.empty((B,), dtype=torch.int32, device=dev)
    nxt = torch.empty((B,), dtype=torch.int32, device=dev)
    nbytes_ws = sw.swattn_greedy_accept_workspace(B, n_q, vocab)
    ws = torch.empty(max(nbytes_ws, 8) // 8, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)

    def launch(cs):
        sw.swattn_greedy_accept(logits, sw.SWATTN_BF16, B, n_q, vocab, d, tgt, acc, nxt, ws, ws.numel() * 8, cs)

    flush = ColdFlush(torch, dev)
    for _ in range(args.warmup):
        launch(stream.cuda_stream)
    torch.cuda.synchronize()
    et, ea, en = oracle.greedy_accept(vals, drafts)
    parity_ok = (np.array_equal(tgt.cpu().numpy(), et) and np.array_equal(acc.cpu().numpy(), ea)
                 and np.array_equal(nxt.cpu().numpy(), en))
    t = time_calls(torch, dev, stream, launch, flush, args.steps, not args.no_graph)
    value = t["cold_graph_us_per_call"]
    nbytes = B * n_q * vocab * 2 + B * (n_q - 1) * 4 + B * n_q * 4 + 2 * B * 4
    achieved = nbytes / (value * 1e-6) / 1e9
    line = {
        "metric": "greedy acceptance us/call (argmax of every position's logits + accepted drafts)",
        "value": value, "unit": "us/call", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(value / 1e3, 6), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"greedy acceptance: {B} sequence(s) x {n_q} positions x {vocab} bf16 logits "
                               "~ N(0,1), drafts agree for a random prefix, seed 6",
                   "global_batch": B, "seq_len": n_q, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "algorithmic_bytes": nbytes,
                     "kernel": "argmax_chunks+accept_finalize"},
        "timing": t,
        "parity_check": {"ok": bool(parity_ok), "what": "target ids, accepted counts, next tokens vs oracle"},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        times = []
        t_start = time.perf_counter()
        while time.perf_counter() - t_start < args.cpu_budget and len(times) < 20:
            t0 = time.perf_counter()
            oracle.greedy_accept(vals, drafts)
            times.append(time.perf_counter() - t0)
        line["cpu_baseline"] = {"value": round(statistics.median(times) * 1e6, 1), "unit": "us/call", "cores": 1,
                                "kind": "oracle", "sample": f"whole workload, {len(times)} run(s), median"}
    print(json.dumps(line), flush=True)


def layer_graph_inputs(w, n_slots, vocab, seed, np, torch, dev):
    """Per-slot inputs of one decode step over the verify workload's layers: bf16 Q, new
    K/V rows, the target's logits after each of the 8 inputs, and drafts that agree with
    the target's argmax for a random prefix (so acceptance is not trivially 0)."""
    import oracle
    L, n, H, Hkv, D = w.B, w.n_q, w.H, w.Hkv, w.D
    rng = np.random.default_rng(seed)
    slots = []
    for _ in range(n_slots):
        host = dict(q=oracle.f32_to_bf16_rne(rng.standard_normal((L, n, H, D)).astype(np.float32)),
                    kn=oracle.f32_to_bf16_rne(rng.standard_normal((L, n, Hkv, D)).astype(np.float32)),
                    vn=oracle.f32_to_bf16_rne(rng.standard_normal((L, n, Hkv, D)).astype(np.float32)),
                    logits=oracle.f32_to_bf16_rne(rng.standard_normal((1, n, vocab)).astype(np.float32)))
        target = oracle.row_argmax((host["logits"].astype(np.uint32) << 16).view(np.float32))
        drafts = target[:, :n - 1].astype(np.int32).copy()
        cut = int(rng.integers(0, n))
        if cut < n - 1:
            drafts[0, cut] = (drafts[0, cut] + 1) % vocab
        host["drafts"] = drafts
        dev_in = {key: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
                  for key, a in host.items() if key != "drafts"}
        dev_in["drafts"] = torch.from_numpy(drafts).to(dev)
        slots.append((host, dev_in))
    return slots


def layer_graph_expected(w, host, np):
    """Oracle result of one slot's step: caches after the append, every layer's output,
    and the acceptance."""
    import oracle
    mc = int(w.ctx_len.max())
    ek, ev = oracle.append_kv(w.k_cache, w.v_cache, w.block_table, w.ctx_len, host["kn"], host["vn"], w.n_q,
                              new_format="bf16", kv_format="bf16", max_ctx=mc)
    out = oracle.attend(host["q"], ek, ev, w.block_table, w.ctx_len, w.n_q, w.window, w.scale, q_format="bf16",
                        kv_format="bf16")
    vals = (host["logits"].astype(np.uint32) << 16).view(np.float32)
    tgt, acc, nxt = oracle.greedy_accept(vals, host["drafts"])
    return dict(k=ek, v=ev, out=out, tgt=tgt, acc=acc, nxt=nxt)


def layer_graph_errors(got, exp, np):
    """Worst excess over the verify tolerance (bf16 output: 2e-3 + 1e-2|ref|) and whether
    the acceptance matches exactly."""
    o = got["out"].float().cpu().numpy().astype(np.float64)
    excess = float((np.abs(o - exp["out"]) - 2e-3 - 1e-2 * np.abs(exp["out"])).max())
    ids = (np.array_equal(got["tgt"].cpu().numpy(), exp["tgt"]) and np.array_equal(got["acc"].cpu().numpy(), exp["acc"])
           and np.array_equal(got["nxt"].cpu().numpy(), exp["nxt"]))
    return excess, ids


def run_layer_graph(args, torch, np, sw, synth, dev):
    """One decode step of the verify workload's 24 layers as a model runs it: per layer,
    swattn_append_verify of that layer alone (its 8 new K/V rows appended and its verify,
    one launch), and at the end swattn_greedy_accept on the step's logits (8 x --vocab
    bf16).  The step is captured into one HIP graph per buffer slot (3 slots, replayed
    round-robin, 20 warm-up replays each, after the manifest's LOOPGRAPH_PINGPONG_SLOTS /
    LOOPGRAPH_WARMUP_CALLS), and compared with the same step issued with separate
    swattn_append_kv and swattn_verify calls per layer, and with all layers stacked in one
    append and one verify call.  Every slot's outputs, the cache bytes and the acceptance
    are checked against the oracle (oracle.append_kv, oracle.attend, oracle.greedy_accept)."""
    from speculative_verify_kv_amd.step_graph import FORMS, LayerStep
    w = synth.named_workload("verify")
    n_slots, vocab = 3, args.vocab
    k = torch.from_numpy(np.ascontiguousarray(w.k_cache).view(np.int16)).to(dev).view(torch.bfloat16)
    v = torch.from_numpy(np.ascontiguousarray(w.v_cache).view(np.int16)).to(dev).view(torch.bfloat16)
    bt = torch.from_numpy(w.block_table).to(dev)
    ctx = torch.from_numpy(w.ctx_len).to(dev)
    slots = layer_graph_inputs(w, n_slots, vocab, 8, np, torch, dev)
    steps_by_form = {form: LayerStep(k, v, bt, ctx, w.n_q, w.window, w.scale, w.H, vocab, form=form,
                                     num_splits=args.splits) for form in FORMS}
    outputs = {form: [steps_by_form[form].new_outputs() for _ in slots] for form in FORMS}
    graphs = {form: [steps_by_form[form].capture(dev_in, outputs[form][i]) for i, (_, dev_in) in enumerate(slots)]
              for form in FORMS}
    for form in FORMS:
        for _ in range(20):
            for g in graphs[form]:
                g.replay()
    torch.cuda.synchronize()
    # every slot of every form against the oracle; the caches hold the last replayed slot's rows
    expected = [layer_graph_expected(w, host, np) for host, _ in slots]
    worst, ids_ok = -1e30, True
    for form in FORMS:
        for i in range(n_slots):
            e, ids = layer_graph_errors(outputs[form][i], expected[i], np)
            worst, ids_ok = max(worst, e), ids_ok and ids
    last = expected[n_slots - 1]
    cache_ok = (np.array_equal(k.view(torch.int16).cpu().numpy().view(np.uint16), last["k"]) and
                np.array_equal(v.view(torch.int16).cpu().numpy().view(np.uint16), last["v"]))
    same_fused = all(torch.equal(outputs["fused"][i][key], outputs["separate"][i][key]) for i in range(n_slots)
                     for key in ("out", "tgt", "acc", "nxt"))
    parity_ok = bool(worst <= 0.0 and ids_ok and cache_ok and same_fused)

    flush = ColdFlush(torch, dev)
    stream = torch.cuda.current_stream(dev)
    res = {}
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    steps = max(args.steps // 4, 9)
    for form in FORMS:
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(steps):
            graphs[form][i % n_slots].replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        warm = ev0.elapsed_time(ev1) * 1e3 / steps
        cold = []
        for i in range(steps):
            flush()
            ev0.record(stream)
            graphs[form][i % n_slots].replay()
            ev1.record(stream)
            torch.cuda.synchronize()
            cold.append(ev0.elapsed_time(ev1) * 1e3)
        res[form] = {"warm_us_per_step": round(warm, 3), "cold_us_per_step": round(statistics.median(cold), 3)}
    value = res["fused"]["cold_us_per_step"]
    line = {
        "metric": "decode-step us (24 per-layer KV appends + verify calls + greedy acceptance, one HIP graph)",
        "value": value, "unit": "us/step", "n_gpus": 1, "steps": steps, "warmup": 20,
        "ms_per_step": round(value / 1e3, 6), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "one verify step of " + DESCRIPTIONS["verify"] + f", layer by layer, plus "
                               f"acceptance over 8 x {vocab} bf16 logits; 3 graph slots",
                   "global_batch": 1, "seq_len": int(w.ctx_len.max()), "parallelism": "none (1 GPU)"},
        "roofline": None,
        "timing": {"per_layer_graph": res["fused"], "per_layer_graph_separate_append": res["separate"],
                   "stacked_graph": res["stacked"],
                   "note": "cold = HIP events around one graph replay after a 512 MiB overwrite and read (includes "
                           "the graph launch); warm = graphs replayed back to back, round-robin over the slots"},
        "plan_per_layer": steps_by_form["fused"].plan_layer.as_dict(),
        "plan_stacked": steps_by_form["stacked"].plan_all.as_dict(),
        "parity_check": {"ok": parity_ok, "worst_excess": worst, "ids_ok": bool(ids_ok), "cache_ok": bool(cache_ok),
                         "fused_equals_separate": bool(same_fused),
                         "what": "every slot of every form vs oracle.append_kv + oracle.attend (2e-3 + 1e-2|ref|) "
                                 "and oracle.greedy_accept (exact); cache bytes vs the oracle after the last slot"},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    if not parity_ok:
        print("bench.py: the layer-graph check against the oracle failed", file=sys.stderr)
        sys.exit(1)


if __name__ == "__main__":
    main()
