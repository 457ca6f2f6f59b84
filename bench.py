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
       [--op attention|append_kv|accept|layer_graph]
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


def cpu_baseline(w, budget_s):
    """Time the float64 oracle on the same workload (single-threaded BLAS)."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:       # threadpoolctl missing: numpy may use more threads
        limiter = None
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.attend(w.q, w.k_cache, w.v_cache, w.block_table, w.ctx_len, w.n_q, w.window, w.scale,
                      q_format=w.q_format, kv_format=w.kv_format, k_scale=w.k_scale, v_scale=w.v_scale)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 5:
            break
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    return {"value": round(statistics.median(times) * 1e6, 1), "unit": "us/call", "cores": 1,
            "kind": "oracle",
            "sample": f"whole workload, {len(times)} run(s), median; float64 numpy, 1 BLAS thread"}


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
    ap.add_argument("--op", default="attention", choices=["attention", "append_kv", "accept", "layer_graph"],
                    help="attention: swattn_verify / swattn_prefill (default); append_kv: swattn_append_kv "
                         "of the workload's new rows into its cache; accept: swattn_greedy_accept; "
                         "layer_graph: one decode step as a graph of per-layer calls")
    ap.add_argument("--vocab", type=int, default=262144, help="accept op: logits per position")
    ap.add_argument("--accept-batch", type=int, default=1, help="accept op: sequences per call")
    ap.add_argument("--calibrate-copy", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this library runs on one GPU; multi-GPU runs are not part of it "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)

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

    w = synth.named_workload(args.workload)

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
        call_lib(desc, q, k, v, bt, ctx, w.n_q, w.window, w.scale, out, ws, plan.workspace_bytes, cs)

    flush = ColdFlush(torch, dev)
    for _ in range(args.warmup):
        flush()
        launch(stream.cuda_stream)
    torch.cuda.synchronize()

    # Spot check against the oracle on a few sampled (layer, query, head) rows.
    import oracle
    got = out.float().cpu().numpy()
    rng = np.random.default_rng(0)
    worst = 0.0
    for b in rng.choice(w.B, size=min(3, w.B), replace=False):
        sub = dict(q=w.q[b:b + 1], block_table=w.block_table[b:b + 1], ctx_len=w.ctx_len[b:b + 1])
        ref = oracle.attend(sub["q"], w.k_cache, w.v_cache, sub["block_table"], sub["ctx_len"], w.n_q,
                            w.window, w.scale, q_format=w.q_format, kv_format=w.kv_format,
                            k_scale=w.k_scale, v_scale=w.v_scale)
        worst = max(worst, float((np.abs(got[b:b + 1] - ref) - 1e-2 * np.abs(ref)).max()))
    parity_ok = worst <= (2e-2 if w.kv_dtype == "e4m3" else 2e-3)

    t = time_calls(torch, dev, stream, launch, flush, args.steps, not args.no_graph)
    cold_graph = t["cold_graph_us_per_call"]

    nbytes = algorithmic_bytes(w)
    achieved = nbytes / (cold_graph * 1e-6) / 1e9
    traffic = read_traffic(args.workload)
    line = {
        "metric": "verify-step us/call (W=188, n_q=8) + achieved HBM GB/s as % of MI355X peak",
        "value": round(cold_graph, 3),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(cold_graph / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kv_dtype if w.kv_dtype != w.q_dtype else w.q_dtype,
        "data": "synthetic",
        "config": {
            "workload": DESCRIPTIONS.get(args.workload, w.name),
            "global_batch": w.B, "seq_len": int(max_ctx), "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes": nbytes,
            "kernel": "partition" + ("" if plan.num_splits == 1 else "+merge"),
        },
        "timing": t,
        "plan": plan.as_dict(),
        "parity_spot_check": {"ok": parity_ok, "worst_excess": worst},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(line), flush=True)


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


def run_layer_graph(args, torch, np, sw, synth, dev):
    """One decode step of the verify workload's 24 layers as a model runs it: per layer,
    swattn_append_verify of that layer alone (B = 1: its 8 new K/V rows appended and its
    verify, one launch), and at the end swattn_greedy_accept on the step's logits (8 x
    --vocab bf16).  The step is captured into one HIP graph per buffer slot (3 slots,
    graphs replayed round-robin, 20 warm-up replays each, after the manifest's
    LOOPGRAPH_PINGPONG_SLOTS / LOOPGRAPH_WARMUP_CALLS), and compared with the same step
    with separate swattn_append_kv and swattn_verify calls per layer, and issued as
    three stacked calls (all layers in one append and one verify call).  Outputs of all
    forms must be equal bit for bit."""
    import oracle
    w = synth.named_workload("verify")
    L, n, H, Hkv, D = w.B, w.n_q, w.H, w.Hkv, w.D
    vocab, n_slots = args.vocab, 3
    rng = np.random.default_rng(8)

    def bf16_dev(x32):
        return torch.from_numpy(oracle.f32_to_bf16_rne(x32).view(np.int16)).to(dev).view(torch.bfloat16)

    k = torch.from_numpy(np.ascontiguousarray(w.k_cache).view(np.int16)).to(dev).view(torch.bfloat16)
    v = torch.from_numpy(np.ascontiguousarray(w.v_cache).view(np.int16)).to(dev).view(torch.bfloat16)
    bt = torch.from_numpy(w.block_table).to(dev)
    ctx = torch.from_numpy(w.ctx_len).to(dev)
    max_ctx = int(w.ctx_len.max())
    slots = []
    for s_ in range(n_slots):
        slot = dict(
            q=bf16_dev(rng.standard_normal((L, n, H, D)).astype(np.float32)),
            kn=bf16_dev(rng.standard_normal((L, n, Hkv, D)).astype(np.float32)),
            vn=bf16_dev(rng.standard_normal((L, n, Hkv, D)).astype(np.float32)),
            logits=bf16_dev(rng.standard_normal((1, n, vocab)).astype(np.float32)),
            drafts=torch.from_numpy(rng.integers(0, vocab, (1, n - 1)).astype(np.int32)).to(dev))
        for form in ("fused", "layers", "stacked"):
            slot[form] = dict(out=torch.empty((L, n, H, D), dtype=torch.bfloat16, device=dev),
                              tgt=torch.empty((1, n), dtype=torch.int32, device=dev),
                              acc=torch.empty((1,), dtype=torch.int32, device=dev),
                              nxt=torch.empty((1,), dtype=torch.int32, device=dev))
        slots.append(slot)
    ws_acc = torch.empty(sw.swattn_greedy_accept_workspace(1, n, vocab) // 8 + 1, dtype=torch.int64, device=dev)
    desc_all = sw.make_desc(slots[0]["q"], k, bt, max_ctx)
    desc_l = [sw.make_desc(slots[0]["q"][l:l + 1], k, bt[l:l + 1], max_ctx, num_splits=args.splits)
              for l in range(L)]
    plan_l = sw.swattn_plan(desc_l[0], n, w.window)
    plan_all = sw.swattn_plan(desc_all, n, w.window)
    assert plan_all.workspace_bytes == 0
    # the per-layer calls run one after another on the stream: one workspace serves them all
    ws_l = torch.zeros(max(plan_l.workspace_bytes, 256), dtype=torch.uint8, device=dev)

    def step(slot, form, cs):
        o = slot[form]
        if form == "fused":
            for l in range(L):
                sw.swattn_append_verify(desc_l[l], slot["q"][l:l + 1], slot["kn"][l:l + 1], slot["vn"][l:l + 1],
                                        sw.SWATTN_BF16, k, v, bt[l:l + 1], ctx[l:l + 1], n, w.window, w.scale,
                                        o["out"][l:l + 1], ws_l, plan_l.workspace_bytes, cs)
        elif form == "layers":
            for l in range(L):
                sw.swattn_append_kv(desc_l[l], slot["kn"][l:l + 1], slot["vn"][l:l + 1], sw.SWATTN_BF16,
                                    bt[l:l + 1], ctx[l:l + 1], n, k, v, cs)
                sw.swattn_verify(desc_l[l], slot["q"][l:l + 1], k, v, bt[l:l + 1], ctx[l:l + 1], n, w.window,
                                 w.scale, o["out"][l:l + 1], ws_l, plan_l.workspace_bytes, cs)
        else:
            sw.swattn_append_kv(desc_all, slot["kn"], slot["vn"], sw.SWATTN_BF16, bt, ctx, n, k, v, cs)
            sw.swattn_verify(desc_all, slot["q"], k, v, bt, ctx, n, w.window, w.scale, o["out"], None, 0, cs)
        sw.swattn_greedy_accept(slot["logits"], sw.SWATTN_BF16, 1, n, vocab, slot["drafts"], o["tgt"], o["acc"],
                                o["nxt"], ws_acc, ws_acc.numel() * 8, cs)

    stream = torch.cuda.current_stream(dev)
    graphs = {}
    for form in ("fused", "layers", "stacked"):
        graphs[form] = []
        for slot in slots:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(slot, form, torch.cuda.current_stream(dev).cuda_stream)
            graphs[form].append(g)
    for form in graphs:
        for _ in range(20):
            for g in graphs[form]:
                g.replay()
    torch.cuda.synchronize()
    same_fused = all(torch.equal(sl["fused"][key], sl["layers"][key]) for sl in slots
                     for key in ("out", "tgt", "acc", "nxt"))
    if plan_l.num_splits == plan_all.num_splits:
        same = all(torch.equal(sl["layers"][key], sl["stacked"][key]) for sl in slots
                   for key in ("out", "tgt", "acc", "nxt"))
    else:   # other split counts round differently: outputs within the verify tolerance, ids equal
        same = all(torch.equal(sl["layers"][key], sl["stacked"][key]) for sl in slots
                   for key in ("tgt", "acc", "nxt")) and all(
            float((sl["layers"]["out"].float() - sl["stacked"]["out"].float()).abs().max()) <= 2e-3
            + 1e-2 * float(sl["stacked"]["out"].float().abs().max()) for sl in slots)

    flush = ColdFlush(torch, dev)
    res = {}
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for form in graphs:
        steps = max(args.steps // 4, 9)
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
        "value": value, "unit": "us/step", "n_gpus": 1, "steps": max(args.steps // 4, 9), "warmup": 20,
        "ms_per_step": round(value / 1e3, 6), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "one verify step of " + DESCRIPTIONS["verify"] + f", layer by layer, plus "
                               f"acceptance over 8 x {vocab} bf16 logits; 3 graph slots",
                   "global_batch": 1, "seq_len": max_ctx, "parallelism": "none (1 GPU)"},
        "roofline": None,
        "timing": {"per_layer_graph": res["fused"], "per_layer_graph_separate_append": res["layers"],
                   "stacked_graph": res["stacked"],
                   "note": "cold = HIP events around one graph replay after a 512 MiB overwrite and read (includes "
                           "the graph launch); warm = graphs replayed back to back, round-robin over the slots"},
        "plan_per_layer": plan_l.as_dict(), "plan_stacked": plan_all.as_dict(),
        "parity_check": {"ok": bool(same and same_fused),
                         "what": "per-layer graph (append_verify) == per-layer graph (append_kv + verify) == "
                                 "stacked graph, outputs bit for bit"},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
