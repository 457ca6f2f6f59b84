"""GPU parity: libswattn (through its C ABI) against the float64 oracle.

Every case compares the HIP output element by element with ``oracle.attend`` on
the same seeded inputs, at the tolerance stated in tests/gpu_util.py.  The named
workloads run at full size in the launch configuration the bench times.
"""
import numpy as np
import pytest
import torch

import oracle
import speculative_verify_kv_amd as sw
import synth
import gpu_util as gu

pytestmark = pytest.mark.gpu

NAMED = list(synth.NAMED)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sw.lib()


# ---------------------------------------------------------------------------
# the named workloads, full size, default plan
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("key", NAMED)
def test_named_workload(key):
    gu.log(f"[named] {key}")
    w, ref = gu.named(key)
    got, plan = gu.run(w, prefill=w.n_q > sw.SWATTN_MAX_NQ)
    gu.log(f"  plan {plan.as_dict()}")
    gu.check(got, ref, w.kv_dtype, out_f32=(w.q_dtype == "f32"), label=key)


@pytest.mark.parametrize("key", ["verify", "decode", "wide_verify", "batched_fp8", "batched_bf16", "fullctx_1024",
                                 "fullctx_2048", "fullctx_4096", "prefill_512"])
def test_named_workload_f32_out(key):
    gu.log(f"[named f32 out] {key}")
    w, ref = gu.named(key)
    got, _ = gu.run(w, out_f32=True, prefill=w.n_q > sw.SWATTN_MAX_NQ)
    gu.check(got, ref, w.kv_dtype, out_f32=True, label=key + "/f32")


# ---------------------------------------------------------------------------
# split-count invariance and run-to-run determinism
# ---------------------------------------------------------------------------
def test_split_invariance_and_determinism_mfma():
    w, ref = gu.named("verify")
    t = gu.upload(w)
    outs = {}
    for S in (1, 2, 3, 4, 7):
        gu.log(f"[splits] S={S}")
        got, plan = gu.run(w, t, out_f32=True, num_splits=S)
        assert plan.num_splits == S and plan.variant == sw.SWATTN_VARIANT_MFMA
        gu.check(got, ref, w.kv_dtype, True, label=f"verify S={S}")
        again, _ = gu.run(w, t, out_f32=True, num_splits=S)
        assert np.array_equal(got, again), f"S={S} not bitwise deterministic"
        outs[S] = got
    for S in outs:
        assert np.abs(outs[S] - outs[1]).max() <= 2e-3


def _workload_and_reference(key):
    if key == "one_layer":
        # one layer of the verify step (2 units): every split count keeps 16-row chunks,
        # each run by four workgroups (column quarters), so a chunk waits for S x 4 arrivals
        w = synth.make_workload("one_layer", B=1, H=8, Hkv=2, D=256, n_q=8, window=188, ctx=4096, bs=16, seed=7,
                                recent=195)
        return w, gu.reference(w)
    return gu.named(key)


@pytest.mark.parametrize("key,variant", [("verify", sw.SWATTN_VARIANT_MFMA), ("one_layer", sw.SWATTN_VARIANT_MFMA),
                                         ("batched_fp8", sw.SWATTN_VARIANT_MFMA),
                                         ("tiny_decode", sw.SWATTN_VARIANT_VALU), ("verify", sw.SWATTN_VARIANT_VALU)])
def test_fused_merge_equals_merge_kernel(key, variant):
    """The last partition workgroup of a row chunk combines the partials with the same
    code as the merge kernel: identical outputs.  Calls alternate between two query
    sets on one workspace, so a partial read before its writer's stores landed, or a
    counter not reset, shows as a mismatch."""
    w, ref = _workload_and_reference(key)
    t = gu.upload(w)
    q_sets = [t["q"], (-t["q"]).contiguous()]
    S_list = (2, 3, 4, 8) if key != "batched_fp8" else (2,)
    mc = int(w.ctx_len.max())
    odt = sw.SWATTN_F32

    def call(q, S, merge, ws):
        out, plan = sw.verify(q, t["k"], t["v"], t["bt"], t["ctx"], w.n_q, w.window, w.scale, mc,
                              out_dtype=odt, k_scale=t["ks"], v_scale=t["vs"], num_splits=S,
                              variant=variant, merge=merge, workspace=ws)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64), plan

    for S in S_list:
        gu.log(f"[fused merge] {key} variant={variant} S={S}")
        kern = [call(q, S, sw.SWATTN_MERGE_KERNEL, None) for q in q_sets]
        assert kern[0][1].merge_grid > 0 and kern[0][1].fused_merge == 0
        if key == "one_layer":
            assert kern[0][1].rows_per_chunk == 16 and kern[0][1].grid == 2 * 2 * 4 * S
        gu.check(kern[0][0], ref, w.kv_dtype, True, label=f"{key} S={S} merge kernel")
        plan = kern[0][1]
        ws = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device=gu.DEV)
        for rep in range(6):
            got, fplan = call(q_sets[rep % 2], S, sw.SWATTN_MERGE_FUSED, ws)
            assert fplan.num_splits == S and fplan.variant == variant
            assert fplan.fused_merge == 1 and fplan.merge_grid == 0
            assert np.array_equal(got, kern[rep % 2][0]), f"{key} S={S} call {rep}: fused != merge kernel"
        assert int(ws[:sw.SWATTN_WORKSPACE_COUNTER_BYTES].count_nonzero()) == 0


@pytest.mark.parametrize("key,S_cycle", [("verify", (2, 4, 3, 8)), ("decode", (3, 8)), ("batched_fp8", (2,)),
                                         ("batched_bf16", (3, 2))])
def test_fused_merge_back_to_back_stress(key, S_cycle):
    """64 fused-merge launches queued back to back on one stream, with no host
    synchronisation between them, over eight query sets and a cycle of split counts on
    one workspace: every output is bit-equal to the merge kernel's for its query set and
    split count.  Hundreds of merge groups per launch, each combining partials written
    by workgroups on other XCDs: a partial read before its writer's stores were visible,
    or a counter the previous launch left non-zero, would show in some launch."""
    w = synth.named_workload(key)
    t = gu.upload(w)
    mc = int(w.ctx_len.max())
    q_sets = [(t["q"].float() * c).to(torch.bfloat16) for c in (1.0, -1.0, 0.5, -2.0, 0.25, 1.5, -0.75, 3.0)]

    def call(q, S, merge, ws=None):
        return sw.verify(q, t["k"], t["v"], t["bt"], t["ctx"], w.n_q, w.window, w.scale, mc,
                         out_dtype=sw.SWATTN_F32, k_scale=t["ks"], v_scale=t["vs"], num_splits=S,
                         merge=merge, workspace=ws)

    expect = {}
    ws_bytes = 0
    for S in S_cycle:
        for i, q in enumerate(q_sets):
            out, plan = call(q, S, sw.SWATTN_MERGE_KERNEL)
            assert plan.num_splits == S and plan.merge_grid > 0
            expect[(i, S)] = out
        ws_bytes = max(ws_bytes, plan.workspace_bytes)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=gu.DEV)
    gu.log(f"[fused stress] {key} S cycle {S_cycle}, groups per launch "
           f"{plan.grid // plan.num_splits}")
    got = []
    for n in range(64):
        i, S = n % len(q_sets), S_cycle[(n // len(q_sets)) % len(S_cycle)]
        out, plan = call(q_sets[i], S, sw.SWATTN_MERGE_FUSED, ws)
        assert plan.fused_merge == 1 and plan.merge_grid == 0
        got.append((i, S, out))
    torch.cuda.synchronize()
    bad = [(n, i, S) for n, (i, S, out) in enumerate(got) if not torch.equal(out, expect[(i, S)])]
    assert not bad, f"{key}: fused != merge kernel in launches {bad[:8]}"
    assert int(ws[:sw.SWATTN_WORKSPACE_COUNTER_BYTES].count_nonzero()) == 0


@pytest.mark.parametrize("D,n_q,window", [(64, 1, 10 ** 6), (256, 1, 10 ** 6), (256, 8, 10 ** 6), (128, 8, 5000),
                                          (256, 8, 188)])
def test_single_sequence_past_4096_keys(D, n_q, window):
    # One sequence of 8192 positions.  Past 4096 keys a launch of a few units needs more
    # than 8 splits to keep each split within its workgroup's 512-entry key table (full
    # attention: 16 splits, merged by the last workgroup where the partials are small).
    gu.log(f"[long context] D={D} n_q={n_q} window={window}")
    w = synth.make_workload("long_ctx", B=1, H=8, Hkv=2, D=D, n_q=n_q, window=window, ctx=8192, bs=16, seed=12)
    ref = gu.reference(w)
    t = gu.upload(w)
    got, plan = gu.run(w, t, out_f32=True)
    keys = min(8192, window + n_q - 1)
    assert plan.variant == sw.SWATTN_VARIANT_MFMA and plan.num_splits * 512 >= keys
    gu.check(got, ref, w.kv_dtype, True, label=f"long D={D} n_q={n_q} W={window} plan {plan.as_dict()}")
    got, _ = gu.run(w, t, out_f32=False)
    gu.check(got, ref, w.kv_dtype, False, label=f"long D={D} n_q={n_q} W={window} bf16 out")


@pytest.mark.parametrize("variant", [sw.SWATTN_VARIANT_MFMA, sw.SWATTN_VARIANT_VALU])
def test_split_invariance_decode(variant):
    # plain decode (4 rows per KV head): a 16-row matrix-core tile with 12 padding rows,
    # or the vector-ALU kernel
    w = synth.make_workload("decode", B=6, H=8, Hkv=2, D=256, n_q=1, window=188, ctx=[300, 188, 1, 4096, 189, 2000],
                            bs=16, seed=5, recent=188, max_blocks=256)
    ref = gu.reference(w)
    t = gu.upload(w)
    for S in (1, 2, 3):
        gu.log(f"[decode splits] variant {variant} S={S}")
        got, plan = gu.run(w, t, out_f32=True, num_splits=S, max_ctx=4096, variant=variant)
        assert plan.variant == variant and plan.num_splits == S
        gu.check(got, ref, w.kv_dtype, True, label=f"decode variant {variant} S={S}")
    auto, plan = gu.run(w, t, out_f32=False, max_ctx=4096)
    assert plan.variant == sw.SWATTN_VARIANT_MFMA
    gu.check(auto, ref, w.kv_dtype, False, label="decode auto")


def test_variants_agree():
    w = synth.make_workload("verify_small", B=4, H=8, Hkv=2, D=256, n_q=8, window=188, ctx=[4096, 200, 8, 1000],
                            bs=16, seed=6, max_blocks=256)
    ref = gu.reference(w)
    t = gu.upload(w)
    for variant in (sw.SWATTN_VARIANT_VALU, sw.SWATTN_VARIANT_MFMA):
        gu.log(f"[variant] {variant}")
        got, plan = gu.run(w, t, out_f32=True, variant=variant, max_ctx=4096)
        assert plan.variant == variant
        gu.check(got, ref, w.kv_dtype, True, label=f"variant {variant}")


# ---------------------------------------------------------------------------
# randomised shapes
# ---------------------------------------------------------------------------
DTYPES = [("bf16", "bf16"), ("bf16", "e4m3"), ("f32", "f32"), ("bf16", "f32"), ("f32", "bf16")]


def fuzz_cases(n=48, seed=1234):
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        n_q = int(rng.choice([1, 2, 3, 7, 8, 16, 33, 64]))
        window = int(rng.choice([1, 2, 15, 16, 17, 188, 4096]))
        bs = int(rng.choice([1, 16, 300]))
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.choice([1, 2]))
        D = int(rng.choice([64, 128, 256]))
        qd, kd = DTYPES[k % len(DTYPES)]
        B = int(rng.choice([1, 3]))
        ctx = [int(rng.integers(n_q, 700)) for _ in range(B)]
        out_f32 = bool(rng.integers(0, 2))
        S = int(rng.choice([0, 0, 1, 2, 5]))
        sentinels = bool(rng.integers(0, 2))
        cases.append(dict(idx=k, n_q=n_q, window=window, bs=bs, G=G, Hkv=Hkv, D=D, qd=qd, kd=kd,
                          B=B, ctx=ctx, out_f32=out_f32, S=S, sentinels=sentinels))
    return cases


@pytest.mark.parametrize("case", fuzz_cases(), ids=lambda c: f"fz{c['idx']}")
def test_fuzz(case):
    c = case
    gu.log(f"[fuzz] {c}")
    w = synth.make_workload(f"fz{c['idx']}", B=c["B"], H=c["G"] * c["Hkv"], Hkv=c["Hkv"], D=c["D"],
                            n_q=c["n_q"], window=c["window"], ctx=c["ctx"], bs=c["bs"],
                            seed=100 + c["idx"], q_dtype=c["qd"], kv_dtype=c["kd"],
                            recent=(c["window"] + c["n_q"] - 1) if c["sentinels"] else None)
    ref = gu.reference(w)
    got, plan = gu.run(w, out_f32=c["out_f32"] or c["qd"] == "f32", num_splits=c["S"])
    gu.log(f"  plan {plan.as_dict()}")
    gu.check(got, ref, w.kv_dtype, c["out_f32"] or c["qd"] == "f32", label=f"fz{c['idx']}")


def fuzz_long_cases(n=10, seed=4321):
    # contexts past 4096 positions: long windows need more than eight key splits
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        n_q = int(rng.choice([1, 3, 8]))
        qd, kd = DTYPES[k % len(DTYPES)]
        B = int(rng.choice([1, 2]))
        cases.append(dict(idx=k, n_q=n_q, window=int(rng.choice([188, 4500, 10 ** 6])),
                          bs=int(rng.choice([16, 64, 300])), G=int(rng.choice([1, 4, 8])),
                          Hkv=int(rng.choice([1, 2])), D=int(rng.choice([64, 128, 256])), qd=qd, kd=kd, B=B,
                          ctx=[int(rng.integers(4097, 16001)) for _ in range(B)], out_f32=True,
                          S=int(rng.choice([0, 0, 0, 40])), sentinels=False))
    return cases


@pytest.mark.parametrize("case", fuzz_long_cases(), ids=lambda c: f"fzl{c['idx']}")
def test_fuzz_long_context(case):
    test_fuzz(case)


# ---------------------------------------------------------------------------
# mask pattern: one-hot V rows turn the output into the softmax weights
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("variant", [sw.SWATTN_VARIANT_MFMA, sw.SWATTN_VARIANT_VALU])
def test_one_hot_values_expose_mask(variant):
    gu.log(f"[one-hot] variant {variant}")
    w = synth.make_workload("onehot", B=3, H=8, Hkv=2, D=256, n_q=8, window=188, ctx=[4096, 300, 195],
                            bs=16, seed=7, recent=195, max_blocks=256)
    lo, hi = oracle.window_bounds(w.ctx_len, w.n_q, w.window)
    one = synth.to_bf16_bits(np.float32([1.0]))[0]
    for b in range(w.B):
        u_lo = int(lo[b, 0])
        for j in range(u_lo, int(hi[b, -1]) + 1):
            blk = w.block_table[b, j // w.bs]
            w.v_cache[blk, :, j % w.bs, :] = 0
            w.v_cache[blk, :, j % w.bs, j - u_lo] = one
    _, weights = oracle.attend(w.q, w.k_cache, w.v_cache, w.block_table, w.ctx_len, w.n_q, w.window,
                               w.scale, q_format="bf16", kv_format="bf16", return_weights=True)
    got, _ = gu.run(w, out_f32=True, variant=variant)
    for b in range(w.B):
        u_lo, u_hi = int(lo[b, 0]), int(hi[b, -1])
        n = u_hi - u_lo + 1
        wref = weights[b, :, :, u_lo:u_hi + 1]                 # [n_q, H, n]
        g = got[b, :, :, :n]
        assert ((g == 0.0) == (wref == 0.0)).all(), "zero pattern differs from the window mask"
        assert (got[b, :, :, n:] == 0.0).all()
        np.testing.assert_allclose(g, wref, rtol=0, atol=2e-3)


# ---------------------------------------------------------------------------
# scores that grow along the window move the running max on late tiles too
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("variant", [sw.SWATTN_VARIANT_MFMA, sw.SWATTN_VARIANT_VALU])
def test_rising_scores_rescale_on_late_tiles(variant):
    w = synth.make_workload("rise", B=2, H=8, Hkv=2, D=256, n_q=8, window=188, ctx=[4096, 700],
                            bs=16, seed=12, recent=195)
    lo, hi = oracle.window_bounds(w.ctx_len, w.n_q, w.window)
    for b in range(w.B):
        u_lo = int(lo[b, 0])
        for j in range(u_lo, int(hi[b, -1]) + 1):
            # K rows grow by 2^(1/48) per position: the tile maxima of the scores rise
            # by far more than 2^8 from one 64-key tile to the next
            blk, off = w.block_table[b, j // w.bs], j % w.bs
            row = (w.k_cache[blk, :, off, :].astype(np.uint32) << 16).view(np.float32)
            w.k_cache[blk, :, off, :] = synth.to_bf16_bits(row * np.float32(2.0 ** ((j - u_lo) / 48.0)))
    ref = gu.reference(w)
    for S, out_f32 in ((1, True), (1, False), (2, True)):
        got, plan = gu.run(w, out_f32=out_f32, num_splits=S, variant=variant)
        gu.check(got, ref, w.kv_dtype, out_f32, label=f"rise S={S} f32={out_f32}")


def test_window_one_returns_own_value_row_exactly():
    w = synth.make_workload("w1", B=2, H=8, Hkv=2, D=128, n_q=8, window=1, ctx=[40, 17], bs=16, seed=8)
    for variant, out_f32 in ((sw.SWATTN_VARIANT_MFMA, False), (sw.SWATTN_VARIANT_MFMA, True),
                             (sw.SWATTN_VARIANT_VALU, True)):
        got, _ = gu.run(w, out_f32=out_f32, variant=variant)
        for b in range(w.B):
            for i in range(w.n_q):
                pos = int(w.ctx_len[b]) - w.n_q + i
                for h in range(w.H):
                    bits = w.v_cache[w.block_table[b, pos // w.bs], h // 4, pos % w.bs]
                    row = (bits.astype(np.uint32) << 16).view(np.float32)
                    assert np.array_equal(got[b, i, h], row)


def test_edge_shapes():
    cases = [
        dict(B=1, H=2, Hkv=1, D=64, n_q=1, window=1, ctx=[1], bs=1),          # one position
        dict(B=2, H=8, Hkv=1, D=64, n_q=64, window=2 ** 31 - 1, ctx=[64, 70], bs=16),   # huge window, p = 0
        dict(B=1, H=16, Hkv=2, D=128, n_q=64, window=188, ctx=[4096], bs=16),  # 512 rows, 4 row chunks
        dict(B=2, H=4, Hkv=4, D=256, n_q=5, window=3, ctx=[5, 600], bs=300),   # G = 1, big blocks
    ]
    for k, c in enumerate(cases):
        gu.log(f"[edge] {c}")
        w = synth.make_workload(f"edge{k}", seed=20 + k, **c)
        ref = gu.reference(w)
        got, plan = gu.run(w, out_f32=True)
        gu.log(f"  plan {plan.as_dict()}")
        gu.check(got, ref, w.kv_dtype, True, label=f"edge{k}")


# ---------------------------------------------------------------------------
# launches that leave CUs idle take 16-row chunks (head_dim 256, two workgroups per
# 32-row chunk): ragged row counts, both cache formats, splits, window edges
# ---------------------------------------------------------------------------
SIXTEEN = [
    dict(B=3, H=8, Hkv=2, n_q=8, window=188, ctx=[195, 700, 4096], kv="bf16", S=(1, 2, 3)),
    dict(B=2, H=8, Hkv=2, n_q=6, window=50, ctx=[6, 1000], kv="e4m3", S=(1, 2)),      # 24 rows: a ragged second chunk
    dict(B=2, H=16, Hkv=2, n_q=3, window=7, ctx=[40, 300], kv="bf16", S=(1, 4)),       # G 8, 24 rows
    dict(B=1, H=4, Hkv=1, n_q=4, window=188, ctx=[188], kv="e4m3", S=(1, 3)),          # exactly 16 rows
    dict(B=2, H=32, Hkv=2, n_q=3, window=100, ctx=[3, 2000], kv="bf16", S=(1, 2)),      # GQA 16, 48 rows
]


@pytest.mark.parametrize("k", range(len(SIXTEEN)))
def test_sixteen_row_chunks(k):
    c = dict(SIXTEEN[k])
    kv = c.pop("kv")
    splits = c.pop("S")
    w = synth.make_workload(f"sixteen{k}", D=256, bs=16, seed=60 + k,
                            kv_dtype=synth.workloads.E4M3 if kv == "e4m3" else synth.workloads.BF16, **c)
    ref = gu.reference(w)
    t = gu.upload(w)
    for S in splits:
        gu.log(f"[16-row] case {k} kv {kv} S={S}")
        got, plan = gu.run(w, t, out_f32=True, num_splits=S)
        assert plan.rows_per_chunk == 16 and plan.variant == sw.SWATTN_VARIANT_MFMA, plan.as_dict()
        gu.check(got, ref, w.kv_dtype, True, label=f"sixteen{k} S={S}")


# 16-row chunks whose launch fits the CUs twice but not four times over run without
# the column split: one workgroup per 16-row chunk, all output columns
SIXTEEN_WHOLE = [
    dict(B=48, H=8, Hkv=2, n_q=8, window=188, ctx_range=(8, 1500), kv="bf16"),     # 96 units
    dict(B=40, H=8, Hkv=2, n_q=6, window=60, ctx_range=(6, 900), kv="e4m3"),       # 24 rows: ragged chunk
]


@pytest.mark.parametrize("k", range(len(SIXTEEN_WHOLE)))
def test_sixteen_row_chunks_whole_columns(k):
    c = dict(SIXTEEN_WHOLE[k])
    kv = c.pop("kv")
    w = synth.make_workload(f"sixteenwhole{k}", D=256, bs=16, seed=90 + k, ctx=None,
                            kv_dtype=synth.workloads.E4M3 if kv == "e4m3" else synth.workloads.BF16, **c)
    ref = gu.reference(w)
    t = gu.upload(w)
    gu.log(f"[16-row whole] case {k} kv {kv}")
    for out_f32 in (True, False):
        got, plan = gu.run(w, t, out_f32=out_f32)
        assert plan.rows_per_chunk == 16 and plan.num_splits == 1, plan.as_dict()
        assert plan.grid == w.B * w.Hkv * plan.row_chunks, plan.as_dict()      # no column split
        gu.check(got, ref, w.kv_dtype, out_f32, label=f"sixteenwhole{k} f32={out_f32}")


# ---------------------------------------------------------------------------
# many rows per KV head and more 32-row chunks than CUs (head_dim 256; 32-key tiles
# for bfloat16 caches): ragged last chunks (a row block with no row), both cache
# formats, GQA 4 and 8, short contexts and narrow windows
# ---------------------------------------------------------------------------
MANY_ROWS = [
    dict(B=48, H=8, Hkv=2, n_q=20, window=188, ctx_range=(20, 1500), kv="bf16"),    # 80 rows: 32 + 32 + 16
    dict(B=48, H=8, Hkv=2, n_q=17, window=100, ctx_range=(17, 400), kv="e4m3"),     # 68 rows: 32 + 32 + 4
    dict(B=72, H=16, Hkv=2, n_q=8, window=7, ctx_range=(8, 300), kv="bf16"),        # G 8, 64 rows
    dict(B=64, H=4, Hkv=1, n_q=64, window=188, ctx_range=(64, 900), kv="e4m3"),     # 256 rows
]


@pytest.mark.parametrize("k", range(len(MANY_ROWS)))
def test_many_rows_per_kv_head(k):
    c = dict(MANY_ROWS[k])
    kv = c.pop("kv")
    w = synth.make_workload(f"manyrows{k}", D=256, bs=16, seed=80 + k, ctx=None,
                            kv_dtype=synth.workloads.E4M3 if kv == "e4m3" else synth.workloads.BF16, **c)
    ref = gu.reference(w)
    t = gu.upload(w)
    gu.log(f"[many rows] case {k} kv {kv}")
    got, plan = gu.run(w, t, out_f32=True)
    # bfloat16 caches with 64 rows or more per KV head take 64-row chunks
    rows = 64 if kv == "bf16" and w.n_q * (w.H // w.Hkv) >= 64 else 32
    assert plan.rows_per_chunk == rows and plan.num_splits == 1 and plan.variant == sw.SWATTN_VARIANT_MFMA, \
        plan.as_dict()
    gu.check(got, ref, w.kv_dtype, True, label=f"manyrows{k}")
    got16, _ = gu.run(w, t, out_f32=False)
    gu.check(got16, ref, w.kv_dtype, False, label=f"manyrows{k} bf16 out")


# ---------------------------------------------------------------------------
# launches with more units than CUs take 32-key tiles (bfloat16, head_dim 256)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("S", [1, 2, 3])
def test_many_units_32_key_tiles(S):
    w = synth.make_workload("many", B=160, H=8, Hkv=2, D=256, n_q=8, window=188, ctx=None, bs=16, seed=21,
                            recent=195, ctx_range=(8, 1200), max_blocks=80)
    ref = gu.reference(w)
    t = gu.upload(w)
    first = None
    for out_f32 in (True, False):
        got, plan = gu.run(w, t=t, out_f32=out_f32, num_splits=S)
        assert plan.grid == 160 * 2 * S
        gu.check(got, ref, w.kv_dtype, out_f32, label=f"many S={S} f32={out_f32}")
        if out_f32:
            first = got
    again, _ = gu.run(w, t=t, out_f32=True, num_splits=S)
    assert np.array_equal(first, again)


@pytest.mark.parametrize("kv,B,n_q", [("bf16", 1024, 8), ("e4m3", 1024, 8), ("bf16", 256, 64)])
def test_large_launch_sampled_sequences(kv, B, n_q):
    # Launches several times larger than the CUs hold (2,048 workgroups: four rounds at
    # two per CU), checked on a sample of sequences (first, last and spread), each
    # against the oracle run on that sequence alone through the same caches.
    gu.log(f"[large launch] {kv} B={B} n_q={n_q}")
    w = synth.make_workload(f"large_{kv}_{B}", B=B, H=8, Hkv=2, D=256, n_q=n_q, window=188, ctx=None, bs=16,
                            seed=31, kv_dtype=kv, recent=188 + n_q - 1, ctx_range=(n_q, 400), max_blocks=25)
    got, plan = gu.run(w, out_f32=True)
    gu.log(f"  plan {plan.as_dict()}")
    assert plan.grid >= 2048, plan.as_dict()
    for b in sorted({0, 1, B // 3, B // 2, 2 * B // 3, B - 2, B - 1}):
        ref = oracle.attend(w.q[b:b + 1], w.k_cache, w.v_cache, w.block_table[b:b + 1], w.ctx_len[b:b + 1],
                            w.n_q, w.window, w.scale, q_format=w.q_format, kv_format=w.kv_format,
                            k_scale=w.k_scale, v_scale=w.v_scale)
        gu.check(got[b:b + 1], ref, w.kv_dtype, True, label=f"large {kv} b={b}")


# ---------------------------------------------------------------------------
# 64-row chunks (bfloat16 caches, head_dim 256, Q^T loaded into registers; 64-key
# tiles and eight waves while the grid fits the CUs, else 32-key tiles and four waves):
# forced on shapes that span a ragged last chunk, a chunk with empty row blocks, GQA 1,
# 4 and 8, split launches with either merge, and short contexts with narrow windows
# ---------------------------------------------------------------------------
TALL = [
    dict(B=3, H=8, Hkv=2, n_q=64, window=188, ctx_range=(64, 4096), S=0, merge=0),    # 256 rows, 4 chunks
    dict(B=5, H=8, Hkv=2, n_q=17, window=100, ctx_range=(17, 700), S=0, merge=0),     # 68 rows: 64 + 4
    dict(B=7, H=8, Hkv=2, n_q=8, window=188, ctx_range=(8, 2000), S=0, merge=0),      # 32 rows of 64
    dict(B=4, H=16, Hkv=2, n_q=8, window=7, ctx_range=(8, 300), S=0, merge=0),        # G 8, 64 rows
    dict(B=2, H=2, Hkv=2, n_q=64, window=300, ctx_range=(64, 1200), S=0, merge=0),    # G 1: W + 63 keys
    dict(B=3, H=8, Hkv=2, n_q=40, window=600, ctx_range=(40, 3000), S=3, merge=sw.SWATTN_MERGE_FUSED),
    dict(B=3, H=8, Hkv=2, n_q=40, window=600, ctx_range=(40, 3000), S=3, merge=sw.SWATTN_MERGE_KERNEL),
    # more chunks than CUs: 32-key tiles, two workgroups per CU (the launches above fit
    # the CUs and take 64-key tiles)
    dict(B=160, H=8, Hkv=2, n_q=17, window=60, ctx_range=(17, 400), S=0, merge=0),    # 640 workgroups
]


@pytest.mark.parametrize("k", range(len(TALL)))
def test_sixty_four_row_chunks(k):
    c = dict(TALL[k])
    S, merge = c.pop("S"), c.pop("merge")
    w = synth.make_workload(f"tall{k}", D=256, bs=16, seed=130 + k, ctx=None, kv_dtype=synth.workloads.BF16,
                            max_blocks=256, **c)
    ref = gu.reference(w)
    t = gu.upload(w)
    gu.log(f"[64-row chunks] case {k}: {TALL[k]}")
    for out_f32 in (True, False):
        got, plan = gu.run(w, t, out_f32=out_f32, num_splits=S, merge=merge, rows_per_chunk=64)
        assert plan.rows_per_chunk == 64 and plan.col_splits == 1, plan.as_dict()
        assert plan.tile_keys == (64 if plan.grid <= 256 else 32), plan.as_dict()
        if S:
            assert plan.num_splits == S and plan.fused_merge == (merge == sw.SWATTN_MERGE_FUSED), plan.as_dict()
        gu.check(got, ref, w.kv_dtype, out_f32, label=f"tall{k} f32={out_f32}")
        if out_f32:
            again, _ = gu.run(w, t, out_f32=True, num_splits=S, merge=merge, rows_per_chunk=64)
            assert np.array_equal(got, again)


# ---------------------------------------------------------------------------
# chunked prefill: n_q above the verify cap, same semantics
# ---------------------------------------------------------------------------
PREFILL_CASES = [
    dict(B=1, H=8, Hkv=2, D=256, n_q=512, window=188, ctx=[4096], bs=16, S=0, kv="bf16", f32=False),
    dict(B=2, H=4, Hkv=4, D=128, n_q=200, window=60, ctx=[700, 200], bs=16, S=3, kv="bf16", f32=True),
    dict(B=1, H=8, Hkv=2, D=256, n_q=512, window=4096, ctx=[512], bs=16, S=0, kv="bf16", f32=True),
    dict(B=2, H=8, Hkv=2, D=256, n_q=96, window=188, ctx=[1000, 300], bs=16, S=0, kv="e4m3", f32=False),
    dict(B=1, H=6, Hkv=2, D=64, n_q=65, window=17, ctx=[65], bs=1, S=0, kv="bf16", f32=True),
    # past 4096 keys: 64-row chunks split more than eight ways, and an E4M3 cache
    dict(B=1, H=8, Hkv=2, D=256, n_q=128, window=10 ** 6, ctx=[8192], bs=16, S=0, kv="bf16", f32=True),
    dict(B=1, H=8, Hkv=2, D=256, n_q=100, window=6000, ctx=[7000], bs=16, S=0, kv="e4m3", f32=True),
]


@pytest.mark.parametrize("c", PREFILL_CASES, ids=lambda c: f"nq{c['n_q']}_W{c['window']}_{c['kv']}")
def test_prefill_matches_oracle(c):
    gu.log(f"[prefill] {c}")
    w = synth.make_workload(f"pf{c['n_q']}", B=c["B"], H=c["H"], Hkv=c["Hkv"], D=c["D"], n_q=c["n_q"],
                            window=c["window"], ctx=c["ctx"], bs=c["bs"], seed=40 + c["n_q"],
                            kv_dtype=c["kv"], recent=c["window"] + c["n_q"] - 1)
    ref = gu.reference(w)
    got, plan = gu.run(w, out_f32=c["f32"], num_splits=c["S"], prefill=True)
    gu.log(f"  plan {plan.as_dict()}")
    gu.check(got, ref, w.kv_dtype, c["f32"], label=f"prefill n_q={c['n_q']}")


def test_prefill_and_verify_agree_up_to_64_and_caps_differ():
    w, _ = gu.named("verify")
    t = gu.upload(w)
    a, _ = gu.run(w, t=t, out_f32=True)
    b, _ = gu.run(w, t=t, out_f32=True, prefill=True)
    assert np.array_equal(a, b)
    w65 = synth.make_workload("cap", B=1, H=8, Hkv=2, D=64, n_q=65, window=188, ctx=[300], bs=16, seed=13)
    t65 = gu.upload(w65)
    with pytest.raises(sw.SwattnError):
        gu.run(w65, t=t65)
    gu.run(w65, t=t65, prefill=True)


# ---------------------------------------------------------------------------
# bad device-resident inputs are turned into NaN by the kernels' own checks
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("variant", [sw.SWATTN_VARIANT_MFMA, sw.SWATTN_VARIANT_VALU])
def test_bad_ctx_and_block_ids_give_nan(variant):
    w = synth.make_workload("bad", B=4, H=8, Hkv=2, D=128, n_q=8, window=188, ctx=[300, 300, 300, 300],
                            bs=16, seed=9)
    ref = gu.reference(w)
    w.ctx_len[1] = 7                                   # < n_q
    w.ctx_len[2] = 1000                                # > max_blocks * bs (and > max_ctx_len)
    w.block_table[3, 299 // 16] = w.num_blocks + 5     # block id out of range inside the window
    t = gu.upload(w)
    desc = sw.make_desc(t["q"], t["k"], t["bt"], 300)
    assert sw.STATUS[sw.swattn_check_inputs(desc, t["bt"], t["ctx"], 8, 188)] == "SWATTN_ERR_CTX"
    out, _ = sw.verify(t["q"], t["k"], t["v"], t["bt"], t["ctx"], 8, 188, w.scale, max_ctx_len=300,
                       out_dtype=sw.SWATTN_F32, variant=variant)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    gu.check(got[0:1], ref[0:1], w.kv_dtype, True, label="good sequence")
    assert np.isnan(got[1]).all() and np.isnan(got[2]).all()
    assert np.isnan(got[3]).any()


def test_check_inputs_reports_block_errors():
    w = synth.make_workload("chk", B=2, H=8, Hkv=2, D=64, n_q=8, window=188, ctx=[300, 100], bs=16, seed=10)
    t = gu.upload(w)
    desc = sw.make_desc(t["q"], t["k"], t["bt"], 300)
    assert sw.swattn_check_inputs(desc, t["bt"], t["ctx"], 8, 188) == 0
    t["bt"][1, 3] = -1
    assert sw.STATUS[sw.swattn_check_inputs(desc, t["bt"], t["ctx"], 8, 188)] == "SWATTN_ERR_BLOCK"


# ---------------------------------------------------------------------------
# one workspace serves plans with different split counts, results reproducible
# ---------------------------------------------------------------------------
def test_workspace_reuse_across_split_counts():
    w, ref = gu.named("verify")
    t = gu.upload(w)
    big = sw.swattn_plan(sw.make_desc(t["q"], t["k"], t["bt"], 4096, num_splits=5), w.n_q, w.window)
    ws = torch.full((big.workspace_bytes,), 0x7F, dtype=torch.uint8, device=gu.DEV)   # stale bytes
    sw.swattn_workspace_init(ws, ws.numel(), torch.cuda.current_stream().cuda_stream)   # counters only
    first = {}
    for S, merge in ((2, sw.SWATTN_MERGE_FUSED), (5, sw.SWATTN_MERGE_KERNEL), (3, sw.SWATTN_MERGE_FUSED),
                     (5, sw.SWATTN_MERGE_FUSED), (2, sw.SWATTN_MERGE_KERNEL), (2, sw.SWATTN_MERGE_FUSED)):
        out, plan = sw.verify(t["q"], t["k"], t["v"], t["bt"], t["ctx"], w.n_q, w.window, w.scale, 4096,
                              out_dtype=sw.SWATTN_F32, num_splits=S, workspace=ws, merge=merge)
        torch.cuda.synchronize()
        assert plan.num_splits == S and plan.fused_merge == (merge == sw.SWATTN_MERGE_FUSED)
        got = out.cpu().numpy().astype(np.float64)
        gu.check(got, ref, w.kv_dtype, True, label=f"reuse S={S} merge={merge}")
        if S in first:   # the fused tail and the merge kernel combine with the same code
            assert np.array_equal(first[S], got), f"S={S} not reproducible"
        first[S] = got
    # every call left the arrival counters at zero
    assert int(ws[:sw.SWATTN_WORKSPACE_COUNTER_BYTES].count_nonzero()) == 0


# ---------------------------------------------------------------------------
# HIP graph capture and replay
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("merge", [sw.SWATTN_MERGE_KERNEL, sw.SWATTN_MERGE_FUSED])
def test_graph_capture_replay(merge):
    w, ref = gu.named("verify")
    t = gu.upload(w)
    desc = sw.make_desc(t["q"], t["k"], t["bt"], 4096, num_splits=2, merge=merge)
    plan = sw.swattn_plan(desc, w.n_q, w.window)
    out = torch.empty(t["q"].shape, dtype=torch.bfloat16, device=gu.DEV)
    assert plan.fused_merge == (merge == sw.SWATTN_MERGE_FUSED)
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device=gu.DEV)
    sw.swattn_workspace_init(ws, ws.numel(), torch.cuda.current_stream().cuda_stream)
    sw.verify(t["q"], t["k"], t["v"], t["bt"], t["ctx"], w.n_q, w.window, w.scale, 4096,
              out=out, num_splits=2, workspace=ws, merge=merge)
    torch.cuda.synchronize()
    eager = out.clone()
    out.zero_()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sw.verify(t["q"], t["k"], t["v"], t["bt"], t["ctx"], w.n_q, w.window, w.scale, 4096,
                  out=out, num_splits=2, workspace=ws, merge=merge)
    for rep in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from eager"
    gu.check(eager.float().cpu().numpy().astype(np.float64), ref, w.kv_dtype, False, label="graph")


# ---------------------------------------------------------------------------
# every e4m3 code decodes exactly: window 1 returns the query's own V row
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("variant", [sw.SWATTN_VARIANT_MFMA, sw.SWATTN_VARIANT_VALU])
def test_e4m3_every_code_through_window_one(variant):
    from oracle.formats import e4m3_value_table
    w = synth.make_workload("codes", B=1, H=4, Hkv=1, D=256, n_q=2, window=1, ctx=[37], bs=16, seed=11,
                            kv_dtype="e4m3")
    pos = int(w.ctx_len[0]) - 1                       # the last query's own position
    blk = w.block_table[0, pos // w.bs]
    w.v_cache[blk, 0, pos % w.bs, :] = np.arange(256, dtype=np.uint8)
    w.v_scale[:] = 1.0
    got, _ = gu.run(w, out_f32=True, variant=variant)
    table = e4m3_value_table()
    for h in range(w.H):
        row = got[0, 1, h]
        assert np.array_equal(np.isnan(row), np.isnan(table))
        assert np.array_equal(row[~np.isnan(table)], table[~np.isnan(table)])


# ---------------------------------------------------------------------------
# the API's largest step: 64 queries (and a 512-position prefill chunk) with a window
# covering the whole 4096-position context, so the key range needs the most splits
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n_q,prefill", [(64, False), (512, True)])
def test_largest_queries_full_window(n_q, prefill):
    w = synth.make_workload(f"largest{n_q}", B=1, H=8, Hkv=2, D=256, n_q=n_q, window=4096, ctx=[4096], bs=16,
                            seed=110 + n_q % 7, max_blocks=256)
    ref = gu.reference(w)
    gu.log(f"[largest] n_q {n_q} window 4096 ctx 4096")
    got, plan = gu.run(w, out_f32=True, max_ctx=4096, prefill=prefill)
    gu.log(f"  plan {plan.as_dict()}")
    assert plan.num_splits >= 8                      # 4096 + n_q - 1 keys, at most 512 per workgroup
    gu.check(got, ref, w.kv_dtype, True, label=f"largest n_q={n_q}")


def test_column_splits_do_not_change_the_bits():
    # the same sequences in launches that split a 16-row chunk's columns four ways (1
    # problem), two ways (24 problems) and not at all (48 problems): identical output bits
    w = synth.make_workload("colsplit", B=48, H=8, Hkv=2, D=256, n_q=8, window=188, ctx=None, bs=16, seed=120,
                            ctx_range=(8, 3000), max_blocks=256)
    t = gu.upload(w)
    outs, splits = {}, {}
    for nb in (48, 24, 1):
        # one split throughout (a lone problem would otherwise split its keys per tile)
        desc = sw.make_desc(t["q"][:nb], t["k"], t["bt"][:nb], int(w.ctx_len.max()), out_dtype=sw.SWATTN_F32,
                            num_splits=1)
        plan = sw.swattn_plan(desc, w.n_q, w.window)
        assert plan.rows_per_chunk == 16 and plan.num_splits == 1, plan.as_dict()
        splits[nb] = plan.grid // (nb * w.Hkv * plan.row_chunks)
        out = torch.empty(t["q"][:nb].shape, dtype=torch.float32, device=gu.DEV)
        sw.swattn_verify(desc, t["q"][:nb], t["k"], t["v"], t["bt"][:nb], t["ctx"][:nb], w.n_q, w.window, w.scale,
                         out, None, 0, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        outs[nb] = out
    assert splits == {48: 1, 24: 2, 1: 4}, splits
    assert torch.equal(outs[48][:24].view(torch.int32), outs[24].view(torch.int32))
    assert torch.equal(outs[48][:1].view(torch.int32), outs[1].view(torch.int32))
    gu.check(outs[48].cpu().numpy().astype(np.float64), gu.reference(w), w.kv_dtype, True, label="colsplit")


# ---------------------------------------------------------------------------
# NaN in pool blocks that no table references: a read outside the referenced
# blocks would turn outputs into NaN
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("key", ["verify", "decode", "batched_fp8", "batched_bf16"])
def test_nan_in_unreferenced_blocks(key):
    gu.log(f"[nan blocks] {key}")
    w = synth.named_workload(key, extra_blocks=384)
    ref = gu.reference(w)
    got, plan = gu.run(w)
    gu.log(f"  plan {plan.as_dict()}")
    gu.check(got, ref, w.kv_dtype, False, label=f"{key} + NaN blocks")
    got32, _ = gu.run(w, out_f32=True)
    gu.check(got32, ref, w.kv_dtype, True, label=f"{key} + NaN blocks f32")


@pytest.mark.parametrize("case", fuzz_cases()[:16], ids=lambda c: f"nanfz{c['idx']}")
def test_fuzz_nan_in_unreferenced_blocks(case):
    c = case
    w = synth.make_workload(f"nanfz{c['idx']}", B=c["B"], H=c["G"] * c["Hkv"], Hkv=c["Hkv"], D=c["D"],
                            n_q=c["n_q"], window=c["window"], ctx=c["ctx"], bs=c["bs"],
                            seed=300 + c["idx"], q_dtype=c["qd"], kv_dtype=c["kd"], extra_blocks=7,
                            recent=(c["window"] + c["n_q"] - 1) if c["sentinels"] else None)
    ref = gu.reference(w)
    got, plan = gu.run(w, out_f32=True, num_splits=c["S"])
    gu.log(f"[nan fuzz] {c} plan {plan.as_dict()}")
    gu.check(got, ref, w.kv_dtype, True, label=f"nanfz{c['idx']}")


# ---------------------------------------------------------------------------
# normalisation: V = 1 on every window position gives out = 1 (sentinels V = 100
# stay on the older positions, NaN past the context)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("variant,kv", [(sw.SWATTN_VARIANT_MFMA, "bf16"), (sw.SWATTN_VARIANT_MFMA, "e4m3"),
                                        (sw.SWATTN_VARIANT_VALU, "bf16"), (sw.SWATTN_VARIANT_VALU, "e4m3")])
def test_all_ones_values_give_one(variant, kv):
    w = synth.make_workload("ones", B=4, H=8, Hkv=2, D=256, n_q=8, window=188, ctx=[4096, 300, 195, 9], bs=16,
                            seed=31, recent=195, max_blocks=256, kv_dtype=kv)
    lo, hi = oracle.window_bounds(w.ctx_len, w.n_q, w.window)
    one = synth.to_bf16_bits(np.float32([1.0]))[0] if kv == "bf16" else np.uint8(0x38)   # E4M3 0.0111.000 = 1
    for b in range(w.B):
        for j in range(int(lo[b, 0]), int(hi[b, -1]) + 1):
            w.v_cache[w.block_table[b, j // w.bs], :, j % w.bs, :] = one
    if kv == "e4m3":
        w.v_scale[:] = 1.0
    for out_f32 in (True, False):
        got, plan = gu.run(w, out_f32=out_f32, variant=variant)
        gu.log(f"[ones] variant {variant} kv {kv} f32 {out_f32}: max |out-1| {np.abs(got - 1).max():.3e}")
        # within bfloat16 rounding: one bf16 step below 1 is 2^-8
        assert np.isfinite(got).all() and np.abs(got - 1.0).max() <= 2.0 ** -8


# ---------------------------------------------------------------------------
# E4M3 plain decode on 16-row chunks split four ways by columns, with splits
# combined by the fused tail (each (row chunk, column split) group merges its own
# columns) and by the merge kernel: identical bits, oracle parity, counters reset
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B", [1, 8])
def test_e4m3_decode_column_quarters_fused_merge(B):
    w = synth.make_workload(f"e4m3dec{B}", B=B, H=8, Hkv=2, D=256, n_q=1, window=188, ctx=None, bs=16, seed=130 + B,
                            kv_dtype="e4m3", recent=188, ctx_range=(1, 4096), max_blocks=256)
    ref = gu.reference(w)
    t = gu.upload(w)
    auto, aplan = gu.run(w, t, out_f32=True, max_ctx=4096)
    gu.log(f"[e4m3 decode] B={B} auto plan {aplan.as_dict()}")
    gu.check(auto, ref, w.kv_dtype, True, label=f"e4m3 decode B={B} auto")
    for S in (2, 3):
        outs = {}
        for merge in (sw.SWATTN_MERGE_KERNEL, sw.SWATTN_MERGE_FUSED):
            desc = sw.make_desc(t["q"], t["k"], t["bt"], 4096, out_dtype=sw.SWATTN_F32, k_scale=t["ks"],
                                v_scale=t["vs"], num_splits=S, merge=merge, rows_per_chunk=16, col_splits=4)
            plan = sw.swattn_plan(desc, w.n_q, w.window)
            assert plan.col_splits == 4 and plan.rows_per_chunk == 16 and plan.num_splits == S
            assert plan.fused_merge == (merge == sw.SWATTN_MERGE_FUSED)
            ws = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device=gu.DEV)
            for rep in range(3):
                out = torch.empty(t["q"].shape, dtype=torch.float32, device=gu.DEV)
                sw.swattn_verify(desc, t["q"], t["k"], t["v"], t["bt"], t["ctx"], w.n_q, w.window, w.scale, out, ws,
                                 plan.workspace_bytes, torch.cuda.current_stream().cuda_stream)
                torch.cuda.synchronize()
                got = out.cpu().numpy().astype(np.float64)
                if merge in outs:
                    assert np.array_equal(got, outs[merge]), f"S={S} merge={merge} rep {rep} not reproducible"
                outs[merge] = got
            assert int(ws[:sw.SWATTN_WORKSPACE_COUNTER_BYTES].count_nonzero()) == 0
            gu.check(outs[merge], ref, w.kv_dtype, True, label=f"e4m3 decode B={B} S={S} merge={merge}")
        assert np.array_equal(outs[sw.SWATTN_MERGE_KERNEL], outs[sw.SWATTN_MERGE_FUSED])


# ---------------------------------------------------------------------------
# the measurement aid: the verify call's data movement without arithmetic
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("key,parts", [("batched_fp8", 1), ("batched_fp8", 3), ("verify", 1), ("verify", 4),
                                       ("tiny_decode", 1), ("tiny_decode", 2)])
def test_window_gather_moves_the_data_and_writes_zeros(key, parts):
    # every output row is written (zeros) whatever the number of workgroups per unit,
    # including slices that split rows unevenly; out-of-range part counts are refused
    w, _ = gu.named(key)
    t = gu.upload(w)
    out = torch.full(t["q"].shape, 7.0, dtype=torch.float32 if w.q_dtype == "f32" else torch.bfloat16, device=gu.DEV)
    desc = sw.make_desc(t["q"], t["k"], t["bt"], int(w.ctx_len.max()), k_scale=t["ks"], v_scale=t["vs"])
    stream = torch.cuda.current_stream().cuda_stream
    sw.swattn_window_gather(desc, t["q"], t["k"], t["v"], t["bt"], t["ctx"], w.n_q, w.window, parts, out, stream)
    torch.cuda.synchronize()
    assert int(out.count_nonzero()) == 0
    for bad in (0, 17):
        st = sw.swattn_window_gather(desc, t["q"], t["k"], t["v"], t["bt"], t["ctx"], w.n_q, w.window, bad, out,
                                     stream, check=False)
        assert sw.STATUS[st] == "SWATTN_ERR_ARG"


@pytest.mark.parametrize("n16,grid", [(0, 1), (1, 1), (1, 3), (1023, 1), (1025, 2), (3 * 1024 + 5, 1),
                                      (4 * 2 * 1024 + 7, 2), (655_361, 512), (655_361, 37)])
def test_stream_read_xor_per_workgroup(n16, grid):
    # every 16-byte chunk i is read once, by workgroup (i mod 1024*grid) div 1024: each
    # workgroup's xor matches the host's over exactly those chunks (zeros where none)
    gu.log(f"[stream read] n16={n16} grid={grid}")
    rng = np.random.default_rng(n16 * 7 + grid)
    host = rng.integers(0, 1 << 32, size=(n16, 4), dtype=np.uint32)
    x = torch.from_numpy(host.reshape(-1).view(np.int32)).to(gu.DEV) if n16 else torch.zeros(4, dtype=torch.int32,
                                                                                              device=gu.DEV)
    xors = torch.full((grid * 4,), -1, dtype=torch.int32, device=gu.DEV)
    sw.swattn_stream_read(x, n16 * 16, grid, xors, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = xors.cpu().numpy().view(np.uint32).reshape(grid, 4)
    want = np.zeros((grid, 4), dtype=np.uint32)
    owner = (np.arange(n16) % (grid * 1024)) // 1024
    for wg in np.unique(owner):
        want[wg] = np.bitwise_xor.reduce(host[owner == wg], axis=0)
    assert np.array_equal(got, want)


def test_stream_read_rejects_bad_arguments():
    x = torch.zeros(64, dtype=torch.int32, device=gu.DEV)
    xors = torch.zeros(16, dtype=torch.int32, device=gu.DEV)
    s = torch.cuda.current_stream().cuda_stream
    for args, want in [((x, 24, 1, xors), "SWATTN_ERR_ARG"), ((x, -16, 1, xors), "SWATTN_ERR_ARG"),
                       ((x, 64, 0, xors), "SWATTN_ERR_ARG"), ((x, 64, 65537, xors), "SWATTN_ERR_ARG"),
                       ((x.data_ptr() + 4, 64, 1, xors), "SWATTN_ERR_ALIGN"),
                       ((x, 64, 1, xors.data_ptr() + 2), "SWATTN_ERR_ALIGN"),
                       ((None, 64, 1, xors), "SWATTN_ERR_NULL")]:
        assert sw.STATUS[sw.swattn_stream_read(*args, s, check=False)] == want, args[1:3]
    torch.cuda.synchronize()
    assert int(xors.count_nonzero()) == 0


def test_stream_read_without_xor_buffer():
    # the timing form (no xor buffer) is accepted at any grid; the same call with the
    # buffer still gives the host's xor afterwards
    host = np.random.default_rng(5).integers(0, 1 << 32, size=(70_000, 4), dtype=np.uint32)
    x = torch.from_numpy(host.reshape(-1).view(np.int32)).to(gu.DEV)
    s = torch.cuda.current_stream().cuda_stream
    for grid in (1, 5, 512):
        assert sw.swattn_stream_read(x, host.size * 4, grid, None, s) == 0
    xors = torch.zeros(8, dtype=torch.int32, device=gu.DEV)
    sw.swattn_stream_read(x, host.size * 4, 2, xors, s)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(xors.cpu().numpy().view(np.uint32).reshape(2, 4), axis=0)
    assert np.array_equal(got, np.bitwise_xor.reduce(host, axis=0))
