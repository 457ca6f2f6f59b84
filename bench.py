#!/usr/bin/env python3
"""Verify-step latency of libswattn on one MI355X, as one JSON line.

Workload (one "step" = one swattn_verify call): a single stream's verify step
with 24 layers of KV stacked along the batch axis — 8 query heads sharing 2 KV
heads, head_dim 256, bf16 Q/K/V ~ N(0, 1), context 4096, window 188, 8 queries
(target + 7 drafts), paged KV with 16-position blocks and a shuffled block
table, seed 1.  Inputs are resident in HBM before timing starts.

Timing: ``--warmup`` untimed calls, then ``--steps`` timed calls captured in
one HIP graph (the serving loop's way of launching), each preceded by an
overwrite of 512 MiB so the 256 MB Infinity Cache and the L2s hold nothing of
the window (cold cache).  The same graph without the calls is timed as well;
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
"""
import argparse
import hashlib
import json
import os
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
}
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_verify_24x2kv_d256_w188_nq8.txt")
KERNEL_SOURCES = ["partition_mfma.hip", "partition_valu.hip", "merge.hip", "kv_access.h",
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


def source_hash():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "speculative_verify_kv_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(calls_per_launch=1):
    """HBM bytes per call from the committed counter summary, or None when it is
    missing or was taken on other kernel sources."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    kv = {}
    with open(TRAFFIC_SUMMARY) as f:
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
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        call_lib(desc, q, k, v, bt, ctx, w.n_q, w.window, w.scale, out, ws,
                         plan.workspace_bytes, stream.cuda_stream)

    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    for _ in range(args.warmup):
        flush.zero_()
        call()
    torch.cuda.synchronize()

    # Spot check against the oracle on a few sampled (layer, query, head) rows.
    import oracle
    got = out.float().cpu().numpy()
    rng = np.random.default_rng(0)
    worst = 0.0
    for b in rng.choice(w.B, size=3, replace=False):
        sub = dict(q=w.q[b:b + 1], block_table=w.block_table[b:b + 1], ctx_len=w.ctx_len[b:b + 1])
        ref = oracle.attend(sub["q"], w.k_cache, w.v_cache, sub["block_table"], sub["ctx_len"], w.n_q,
                            w.window, w.scale, q_format=w.q_format, kv_format=w.kv_format,
                            k_scale=w.k_scale, v_scale=w.v_scale)
        worst = max(worst, float((np.abs(got[b:b + 1] - ref) - 1e-2 * np.abs(ref)).max()))
    parity_ok = worst <= (2e-2 if w.kv_dtype == "e4m3" else 2e-3)

    # ---- cold-cache timed region: K calls captured in one HIP graph, each after a
    # 512 MiB overwrite (twice the Infinity Cache); the same graph without the calls
    # is timed too, and the per-call time is the difference over K.

    def capture(with_calls):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream(dev).cuda_stream
            for _ in range(args.steps):
                flush.zero_()
                if with_calls:
                    call_lib(desc, q, k, v, bt, ctx, w.n_q, w.window, w.scale, out, ws,
                                     plan.workspace_bytes, cs)
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
        per_call.append((ev[0].elapsed_time(ev[1]) - ev[2].elapsed_time(ev[3])) * 1e3 / args.steps)
    cold_graph = statistics.median(per_call)

    # ---- cold, standalone: HIP events around each eager call (includes dispatch latency)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        flush.zero_()
        starts[i].record(stream)
        call()
        ends[i].record(stream)
    torch.cuda.synchronize()
    cold = sorted(s.elapsed_time(e) * 1e3 for s, e in zip(starts, ends))   # us
    cold_med = statistics.median(cold)
    cold_p10 = cold[int(0.1 * (len(cold) - 1))]
    cold_p90 = cold[int(0.9 * (len(cold) - 1))]

    # ---- warm, back to back ------------------------------------------------------------
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    warm = e0.elapsed_time(e1) * 1e3 / args.steps

    # ---- one HIP graph of 100 calls, replayed (warm) -----------------------------------
    graph_us = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream(dev).cuda_stream
            for _ in range(100):
                call_lib(desc, q, k, v, bt, ctx, w.n_q, w.window, w.scale, out, ws,
                                 plan.workspace_bytes, cs)
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(5):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_us = e0.elapsed_time(e1) * 1e3 / 500

    nbytes = algorithmic_bytes(w)
    achieved = nbytes / (cold_graph * 1e-6) / 1e9
    traffic = read_traffic()
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
        "timing": {
            "cold_graph_us_per_call": round(cold_graph, 3),
            "cold_graph_samples_us": [round(x, 3) for x in per_call],
            "cold_eager_us_median": round(cold_med, 3), "cold_eager_us_p10": round(cold_p10, 3),
            "cold_eager_us_p90": round(cold_p90, 3),
            "warm_us_back_to_back": round(warm, 3),
            "graph_us_per_call_warm": None if graph_us is None else round(graph_us, 3),
            "timed_region_wall_s": round(wall, 4),
            "note": "value = cold_graph: K calls in one HIP graph, each after a 512 MiB overwrite, "
                    "minus the same graph without the calls, over K; cold_eager = HIP events around "
                    "each eager call (adds dispatch latency)",
        },
        "plan": plan.as_dict(),
        "parity_spot_check": {"ok": parity_ok, "worst_excess": worst},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
