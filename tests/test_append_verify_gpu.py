"""GPU parity of swattn_append_verify (through the C ABI).

One call must leave exactly what swattn_append_kv followed by swattn_verify leaves:
the same output bits and the same cache bytes.  Bfloat16 rows into a bfloat16 cache
take the one-launch form (the matrix-core kernel reads the new positions' keys from
the new rows and writes them into the cache); the other formats and the vector-ALU
variant take the two-launch form.  The output is also checked against the oracle's
append followed by its attention, at the verify tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import speculative_verify_kv_amd as sw
import synth
import gpu_util as gu

pytestmark = pytest.mark.gpu

FMT = {"bf16": sw.SWATTN_BF16, "f32": sw.SWATTN_F32}

CASES = [
    # one layer of the verify step: 16-row chunks, each over four workgroups (column quarters)
    dict(id="one_layer", B=1, n_q=8, ctx=[4096]),
    # the verify workload's 24 layers
    dict(id="layers", B=24, n_q=8, ctx=[4096] * 24),
    # splits, combined by the last workgroup and by the merge kernel
    dict(id="split_fused", B=1, n_q=8, ctx=[3000], S=4, merge=sw.SWATTN_MERGE_FUSED),
    dict(id="split_kernel", B=3, n_q=8, ctx=[3000, 200, 8], S=2, merge=sw.SWATTN_MERGE_KERNEL),
    # more units than CUs: 32-row chunks with 32-key tiles; plain decode; the widest step
    dict(id="many", B=160, n_q=8, ctx_range=(8, 1200), max_blocks=80),
    dict(id="decode", B=6, n_q=1, ctx=[300, 188, 1, 4096, 189, 2000]),
    dict(id="wide", B=2, n_q=64, ctx=[4096, 700]),
    # 64-row chunks (their 16-row grid would not fit the CUs): 64-key tiles while the grid
    # fits the CUs (12 x 2 x 4 chunks), 32-key tiles with Q^T in registers beyond them
    # (130 x 2 chunks)
    dict(id="tall", B=12, n_q=64, ctx_range=(64, 800), max_blocks=50),
    dict(id="tall_many", B=130, n_q=16, ctx_range=(16, 600), max_blocks=40),
    # the two-launch form: an E4M3 cache, float32 new rows, the vector-ALU kernel
    dict(id="e4m3_cache", B=3, n_q=8, ctx=[4096, 500, 9], kv="e4m3"),
    dict(id="f32_rows", B=3, n_q=8, ctx=[4096, 500, 9], new="f32"),
    dict(id="valu", B=3, n_q=8, ctx=[4096, 500, 9], variant=sw.SWATTN_VARIANT_VALU),
    # other head sizes, group sizes and block sizes through the one-launch form (the
    # in-kernel copy follows each row size and block arithmetic)
    dict(id="d64_mha", B=3, n_q=3, ctx=[700, 40, 3], D=64, H=4, Hkv=4),
    dict(id="d128_g8", B=2, n_q=5, ctx=[2000, 190], D=128, H=16, Hkv=2),
    dict(id="bs1", B=2, n_q=8, ctx=[400, 9], bs=1, max_blocks=512),
    dict(id="bs300", B=2, n_q=8, ctx=[600, 301], bs=300, max_blocks=2, window=100),
    # full attention past 4096 keys: more than eight splits per chunk
    dict(id="long_full", B=1, n_q=8, ctx=[8192], window=10 ** 6, max_blocks=512),
    dict(id="long_decode_d64", B=1, n_q=1, ctx=[9000], window=10 ** 6, max_blocks=563, D=64),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sw.lib()


def _inputs(c, seed):
    kv = c.get("kv", "bf16")
    window = c.get("window", 188)
    kw = dict(B=c["B"], H=c.get("H", 8), Hkv=c.get("Hkv", 2), D=c.get("D", 256), n_q=c["n_q"], window=window,
              bs=c.get("bs", 16), seed=seed, kv_dtype=synth.workloads.E4M3 if kv == "e4m3" else synth.workloads.BF16,
              recent=window + c["n_q"] - 1)
    if "ctx_range" in c:
        w = synth.make_workload(c["id"], ctx=None, ctx_range=c["ctx_range"], max_blocks=c["max_blocks"], **kw)
    else:
        w = synth.make_workload(c["id"], ctx=c["ctx"], max_blocks=c.get("max_blocks", 256), **kw)
    rng = np.random.default_rng(seed + 100)
    shape = (w.B, w.n_q, w.Hkv, w.D)
    kn = rng.standard_normal(shape).astype(np.float32)
    vn = rng.standard_normal(shape).astype(np.float32)
    new = c.get("new", "bf16")
    if new == "bf16":
        kn, vn = oracle.f32_to_bf16_rne(kn), oracle.f32_to_bf16_rne(vn)
    return w, kn, vn, new


def _dev_rows(a, new):
    a = np.ascontiguousarray(a)
    if new == "bf16":
        return torch.from_numpy(a.view(np.int16)).to(gu.DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(gu.DEV)


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.mark.parametrize("c", CASES, ids=lambda c: c["id"])
def test_append_verify_equals_append_then_verify(c):
    w, kn, vn, new = _inputs(c, seed=30 + CASES.index(c))
    gu.log(f"[append_verify] {c['id']} kv {w.kv_format} new {new}")
    t = gu.upload(w)
    knd, vnd = _dev_rows(kn, new), _dev_rows(vn, new)
    mc = int(w.ctx_len.max())
    desc = sw.make_desc(t["q"], t["k"], t["bt"], mc, out_dtype=sw.SWATTN_F32, k_scale=t["ks"], v_scale=t["vs"],
                        num_splits=c.get("S", 0), variant=c.get("variant", 0), merge=c.get("merge", 0))
    plan = sw.swattn_plan(desc, w.n_q, w.window)
    gu.log(f"  plan {plan.as_dict()}")
    if c["id"] in ("tall", "tall_many"):
        assert plan.rows_per_chunk == 64 and plan.tile_keys == (64 if c["id"] == "tall" else 32), plan.as_dict()
    if c["id"].startswith("long"):
        assert plan.num_splits > 8, plan.as_dict()
    stream = torch.cuda.current_stream().cuda_stream
    outs, caches = [], []
    for fused in (True, False):
        k, v = t["k"].clone(), t["v"].clone()
        out = torch.empty(t["q"].shape, dtype=torch.float32, device=gu.DEV)
        ws = torch.zeros(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=gu.DEV)
        if fused:
            sw.swattn_append_verify(desc, t["q"], knd, vnd, FMT[new], k, v, t["bt"], t["ctx"], w.n_q, w.window,
                                    w.scale, out, ws, ws.numel(), stream)
        else:
            sw.swattn_append_kv(desc, knd, vnd, FMT[new], t["bt"], t["ctx"], w.n_q, k, v, stream)
            sw.swattn_verify(desc, t["q"], k, v, t["bt"], t["ctx"], w.n_q, w.window, w.scale, out, ws, ws.numel(),
                             stream)
        torch.cuda.synchronize()
        outs.append(out)
        caches.append((k, v))
    assert torch.equal(_bits(outs[0]), _bits(outs[1])), "output differs from append + verify"
    assert torch.equal(caches[0][0].view(torch.uint8), caches[1][0].view(torch.uint8)), "K cache differs"
    assert torch.equal(caches[0][1].view(torch.uint8), caches[1][1].view(torch.uint8)), "V cache differs"
    kc, vc = oracle.append_kv(w.k_cache, w.v_cache, w.block_table, w.ctx_len, kn, vn, w.n_q, new_format=new,
                              kv_format=w.kv_format, k_scale=w.k_scale, v_scale=w.v_scale, max_ctx=mc)
    ref = oracle.attend(w.q, kc, vc, w.block_table, w.ctx_len, w.n_q, w.window, w.scale, q_format=w.q_format,
                        kv_format=w.kv_format, k_scale=w.k_scale, v_scale=w.v_scale)
    gu.check(outs[0].cpu().numpy().astype(np.float64), ref, w.kv_dtype, True, label=c["id"])


def test_append_verify_bad_inputs_match_the_two_calls():
    # a sequence shorter than n_q (not appended, NaN output) and a bad block id among the
    # new positions (that row not written; its key reads as NaN): same bits both ways
    c = dict(id="bad", B=4, n_q=8, ctx=[4096, 5, 300, 1000])
    w, kn, vn, new = _inputs(c, seed=50)
    bt = w.block_table.copy()
    bt[3, (int(w.ctx_len[3]) - 2) // 16] = -7
    t = gu.upload(w)
    t["bt"] = torch.from_numpy(bt).to(gu.DEV)
    knd, vnd = _dev_rows(kn, new), _dev_rows(vn, new)
    desc = sw.make_desc(t["q"], t["k"], t["bt"], 4096, out_dtype=sw.SWATTN_F32)
    plan = sw.swattn_plan(desc, 8, w.window)
    stream = torch.cuda.current_stream().cuda_stream
    outs, caches = [], []
    for fused in (True, False):
        k, v = t["k"].clone(), t["v"].clone()
        out = torch.empty(t["q"].shape, dtype=torch.float32, device=gu.DEV)
        ws = torch.zeros(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=gu.DEV)
        if fused:
            sw.swattn_append_verify(desc, t["q"], knd, vnd, sw.SWATTN_BF16, k, v, t["bt"], t["ctx"], 8, w.window,
                                    w.scale, out, ws, plan.workspace_bytes, stream)
        else:
            sw.swattn_append_kv(desc, knd, vnd, sw.SWATTN_BF16, t["bt"], t["ctx"], 8, k, v, stream)
            sw.swattn_verify(desc, t["q"], k, v, t["bt"], t["ctx"], 8, w.window, w.scale, out, ws,
                             plan.workspace_bytes, stream)
        torch.cuda.synchronize()
        outs.append(out)
        caches.append((k, v))
    assert torch.equal(_bits(outs[0]), _bits(outs[1]))
    assert torch.equal(caches[0][0].view(torch.uint8), caches[1][0].view(torch.uint8))
    assert torch.equal(caches[0][1].view(torch.uint8), caches[1][1].view(torch.uint8))
    o = outs[0].cpu().numpy()
    assert np.isnan(o[1]).all() and np.isfinite(o[0]).all() and np.isfinite(o[2]).all()
    assert np.isnan(o[3]).any()


def test_append_verify_graph_replay():
    # captured once, replayed with the program's own work in between: every replay equals
    # the eager call (the append is idempotent for a fixed ctx_len)
    c = dict(id="graph", B=2, n_q=8, ctx=[4096, 1000])
    w, kn, vn, new = _inputs(c, seed=60)
    t = gu.upload(w)
    knd, vnd = _dev_rows(kn, new), _dev_rows(vn, new)
    desc = sw.make_desc(t["q"], t["k"], t["bt"], 4096, out_dtype=sw.SWATTN_F32)
    plan = sw.swattn_plan(desc, 8, w.window)
    ws = torch.zeros(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=gu.DEV)
    k, v = t["k"].clone(), t["v"].clone()
    eager = torch.empty(t["q"].shape, dtype=torch.float32, device=gu.DEV)
    sw.swattn_append_verify(desc, t["q"], knd, vnd, sw.SWATTN_BF16, k, v, t["bt"], t["ctx"], 8, w.window, w.scale,
                            eager, ws, ws.numel(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sw.swattn_append_verify(desc, t["q"], knd, vnd, sw.SWATTN_BF16, k, v, t["bt"], t["ctx"], 8, w.window,
                                w.scale, out, ws, ws.numel(), torch.cuda.current_stream().cuda_stream)
    for rep in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(eager)), f"replay {rep}"


def test_append_verify_host_errors_enqueue_nothing():
    # an error of either half returns before the append runs: the cache is untouched
    c = dict(id="err", B=2, n_q=8, ctx=[4096, 1000], kv="e4m3")
    w, kn, vn, new = _inputs(c, seed=70)
    t = gu.upload(w)
    knd, vnd = _dev_rows(kn, new), _dev_rows(vn, new)
    desc = sw.make_desc(t["q"], t["k"], t["bt"], 4096, out_dtype=sw.SWATTN_F32, k_scale=t["ks"], v_scale=t["vs"])
    k0, v0 = t["k"].clone(), t["v"].clone()
    out = torch.empty(t["q"].shape, dtype=torch.float32, device=gu.DEV)
    stream = torch.cuda.current_stream().cuda_stream

    def call(**kw):
        a = dict(q=t["q"], new_dtype=sw.SWATTN_BF16, n_q=8, window=w.window, out=out, ws=None, ws_bytes=0)
        a.update(kw)
        st = sw.swattn_append_verify(desc, a["q"], knd, vnd, a["new_dtype"], t["k"], t["v"], t["bt"], t["ctx"],
                                     a["n_q"], a["window"], w.scale, a["out"], a["ws"], a["ws_bytes"], stream,
                                     check=False)
        torch.cuda.synchronize()
        return sw.STATUS[st]

    assert call(window=0) == "SWATTN_ERR_WINDOW"             # the verify half
    assert call(n_q=65) == "SWATTN_ERR_NQ"                   # past the verify cap, within the append's
    assert call(new_dtype=sw.SWATTN_FP8_E4M3) == "SWATTN_ERR_DTYPE"   # the append half
    assert call(q=None) == "SWATTN_ERR_NULL"
    assert call(out=t["q"]) == "SWATTN_ERR_ARG"              # output overlapping q
    split = sw.make_desc(t["q"], t["k"], t["bt"], 4096, out_dtype=sw.SWATTN_F32, k_scale=t["ks"],
                         v_scale=t["vs"], num_splits=3)
    st = sw.swattn_append_verify(split, t["q"], knd, vnd, sw.SWATTN_BF16, t["k"], t["v"], t["bt"], t["ctx"], 8,
                                 w.window, w.scale, out, None, 0, stream, check=False)
    assert sw.STATUS[st] == "SWATTN_ERR_WORKSPACE"
    torch.cuda.synchronize()
    assert torch.equal(t["k"], k0) and torch.equal(t["v"], v0)
