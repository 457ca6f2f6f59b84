"""GPU test of swattn_verify_noalloc: the verify call that allocates nothing, whose split
plans use the library's static per-GPU scratch instead of a caller's workspace.

Two calls in a row, the second with a smaller input, each compared bit for bit with
swattn_verify (the same plan and kernels, with a caller-provided workspace) and with
the float64 oracle at the verify tolerance; then the fused and the kernel merge on
the shared scratch; a plan beyond the scratch's size is refused before anything is
enqueued; and the call captured in a HIP graph replays the eager result.
"""
import numpy as np
import pytest
import torch

import speculative_verify_kv_amd as sw
import synth
import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sw.lib()


def _both(w, t, S, merge, out_f32=True):
    """(noalloc output, swattn_verify output, plan) for one forced plan."""
    mc = int(w.ctx_len.max())
    desc = sw.make_desc(t["q"], t["k"], t["bt"], mc, out_dtype=sw.SWATTN_F32 if out_f32 else sw.SWATTN_BF16,
                        k_scale=t["ks"], v_scale=t["vs"], num_splits=S, merge=merge)
    plan = sw.swattn_plan(desc, w.n_q, w.window)
    tdt = torch.float32 if out_f32 else torch.bfloat16
    stream = torch.cuda.current_stream().cuda_stream
    out_na = torch.full(t["q"].shape, float("nan"), dtype=tdt, device=gu.DEV)
    sw.swattn_verify_noalloc(desc, t["q"], t["k"], t["v"], t["bt"], t["ctx"], w.n_q, w.window, w.scale, out_na,
                             stream)
    ws = torch.zeros(max(plan.workspace_bytes, 16), dtype=torch.uint8, device=gu.DEV)
    out_ref = torch.empty(t["q"].shape, dtype=tdt, device=gu.DEV)
    sw.swattn_verify(desc, t["q"], t["k"], t["v"], t["bt"], t["ctx"], w.n_q, w.window, w.scale, out_ref, ws,
                     plan.workspace_bytes, stream)
    torch.cuda.synchronize()
    return out_na, out_ref, plan


def test_noalloc_two_calls_second_smaller():
    big = synth.make_workload("na_big", B=8, H=8, Hkv=2, D=256, n_q=1, window=188, ctx=None, bs=16, seed=140,
                              recent=188, ctx_range=(1, 4096), max_blocks=256)
    small = synth.make_workload("na_small", B=2, H=8, Hkv=2, D=256, n_q=8, window=188, ctx=[700, 200], bs=16,
                                seed=141, recent=195)
    for w, S in ((big, 4), (small, 2)):
        t = gu.upload(w)
        ref = gu.reference(w)
        for merge in (sw.SWATTN_MERGE_FUSED, sw.SWATTN_MERGE_KERNEL):
            gu.log(f"[noalloc] {w.name} S={S} merge={merge}")
            got, exp, plan = _both(w, t, S, merge)
            assert plan.num_splits == S and plan.workspace_bytes > 0
            assert plan.fused_merge == (merge == sw.SWATTN_MERGE_FUSED)
            assert torch.equal(got.view(torch.int32), exp.view(torch.int32)), f"{w.name} S={S} merge={merge}"
            gu.check(got.cpu().numpy().astype(np.float64), ref, w.kv_dtype, True, label=f"noalloc {w.name} S={S}")


def test_noalloc_e4m3_and_default_plan():
    w = synth.make_workload("na_e4m3", B=3, H=8, Hkv=2, D=256, n_q=8, window=188, ctx=[4096, 300, 195], bs=16,
                            seed=142, recent=195, kv_dtype="e4m3", max_blocks=256)
    t = gu.upload(w)
    ref = gu.reference(w)
    for S in (0, 3):
        got, exp, plan = _both(w, t, S, sw.SWATTN_MERGE_AUTO, out_f32=False)
        gu.log(f"[noalloc e4m3] S={S} plan {plan.as_dict()}")
        assert torch.equal(got.view(torch.int16), exp.view(torch.int16))
        gu.check(got.float().cpu().numpy().astype(np.float64), ref, w.kv_dtype, False, label=f"noalloc e4m3 S={S}")


def test_noalloc_refuses_plans_beyond_the_scratch():
    w = synth.make_workload("na_tiny", B=1, H=8, Hkv=2, D=256, n_q=8, window=188, ctx=[300], bs=16, seed=143)
    t = gu.upload(w)
    # 512 problems at 64 queries and 16 splits: far more workspace than the scratch holds
    desc = sw.make_desc(t["q"], t["k"], t["bt"], 4096, out_dtype=sw.SWATTN_F32, num_splits=16,
                        merge=sw.SWATTN_MERGE_KERNEL)
    desc.batch = 512
    desc.max_blocks_per_seq = 256
    plan = sw.swattn_plan(desc, 64, 4096)
    assert plan.workspace_bytes > sw.SWATTN_STATIC_SCRATCH_BYTES
    out = torch.empty(4, dtype=torch.float32, device=gu.DEV)
    st = sw.swattn_verify_noalloc(desc, t["q"], t["k"], t["v"], t["bt"], t["ctx"], 64, 4096, w.scale, out,
                                  torch.cuda.current_stream().cuda_stream, check=False)
    assert sw.STATUS[st] == "SWATTN_ERR_SCRATCH"
    assert "static scratch" in sw.swattn_status_str(st)


def test_noalloc_under_graph_capture():
    w = synth.make_workload("na_graph", B=4, H=8, Hkv=2, D=256, n_q=1, window=188, ctx=[4096, 1000, 188, 50],
                            bs=16, seed=144, recent=188, max_blocks=256)
    t = gu.upload(w)
    mc = int(w.ctx_len.max())
    desc = sw.make_desc(t["q"], t["k"], t["bt"], mc, out_dtype=sw.SWATTN_F32, num_splits=3,
                        merge=sw.SWATTN_MERGE_FUSED)
    out = torch.empty(t["q"].shape, dtype=torch.float32, device=gu.DEV)
    sw.swattn_verify_noalloc(desc, t["q"], t["k"], t["v"], t["bt"], t["ctx"], w.n_q, w.window, w.scale, out,
                             torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sw.swattn_verify_noalloc(desc, t["q"], t["k"], t["v"], t["bt"], t["ctx"], w.n_q, w.window, w.scale, out,
                                 torch.cuda.current_stream().cuda_stream)
    for rep in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
    gu.check(eager.cpu().numpy().astype(np.float64), gu.reference(w), w.kv_dtype, True, label="noalloc graph")
