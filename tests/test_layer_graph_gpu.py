"""GPU parity of the graph-captured decode loop against the oracle.

One decode step of the verify workload's 24 layers is captured as a HIP graph per
buffer slot (3 slots), exactly as ``bench.py --op layer_graph`` builds it
(``speculative_verify_kv_amd.step_graph.LayerStep``): per layer the step's 8 new K/V
rows are appended and the layer's verify attention runs, then greedy acceptance on
the step's logits.  The graphs are replayed several times, round-robin and in other
orders, with eager work and synchronisations between replays; after every replay the
slot's outputs are compared with ``oracle.append_kv`` followed by ``oracle.attend``
(layer by layer, at the verify tolerance), its acceptance with
``oracle.greedy_accept`` (exactly), and the caches with the oracle's appended caches
(byte for byte).  Source of the loop: "The Fast Gemma Challenge: our verified-SOTA
recipe, in full", manifest ONEGRAPH, LOOPGRAPH_REQUIRE_CAPTURE=1,
LOOPGRAPH_PINGPONG_SLOTS=3, LOOPGRAPH_WARMUP_CALLS=20.
"""
import numpy as np
import pytest
import torch

import bench
import speculative_verify_kv_amd as sw
import synth
import gpu_util as gu

pytestmark = pytest.mark.gpu

N_SLOTS = 3
VOCAB = 262144


@pytest.fixture(scope="module")
def loop_setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sw.lib()
    w = synth.named_workload("verify")
    dev = torch.device(gu.DEV)
    t = gu.upload(w)
    slots = bench.layer_graph_inputs(w, N_SLOTS, VOCAB, 8, np, torch, dev)
    expected = [bench.layer_graph_expected(w, host, np) for host, _ in slots]
    return w, t, slots, expected


def _cache_bits(x):
    return x.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("form", ["fused", "separate", "stacked"])
def test_layer_graph_replays_match_oracle(loop_setup, form):
    from speculative_verify_kv_amd.step_graph import LayerStep
    w, t, slots, expected = loop_setup
    gu.log(f"[layer graph] form {form}")
    step = LayerStep(t["k"], t["v"], t["bt"], t["ctx"], w.n_q, w.window, w.scale, w.H, VOCAB, form=form)
    gu.log(f"  plan per layer {step.plan_layer.as_dict()} stacked {step.plan_all.as_dict()}")
    outs = [step.new_outputs() for _ in range(N_SLOTS)]
    graphs = [step.capture(dev_in, outs[i]) for i, (_, dev_in) in enumerate(slots)]
    for _ in range(20):                       # the manifest's warm-up replays
        for g in graphs:
            g.replay()
    torch.cuda.synchronize()
    order = [0, 1, 2, 2, 0, 1, 1, 0, 2]
    for n, i in enumerate(order):
        outs[i]["out"].fill_(float("nan"))
        outs[i]["tgt"].fill_(-1)
        outs[i]["acc"].fill_(-1)
        outs[i]["nxt"].fill_(-1)
        torch.cuda.synchronize()
        graphs[i].replay()
        torch.cuda.synchronize()
        exp = expected[i]
        excess, ids_ok = bench.layer_graph_errors(outs[i], exp, np)
        gu.log(f"  replay {n} slot {i}: worst excess {excess:.3e} ids {ids_ok}")
        assert excess <= 0.0, f"slot {i} replay {n}: outputs outside 2e-3 + 1e-2|ref| ({excess})"
        assert ids_ok, f"slot {i} replay {n}: acceptance differs from the oracle"
        got = outs[i]["out"].float().cpu().numpy().astype(np.float64)
        gu.check(got, exp["out"], w.kv_dtype, False, label=f"{form} slot {i} replay {n}")
        if n in (0, 4, len(order) - 1):
            assert np.array_equal(_cache_bits(t["k"]), exp["k"]), f"slot {i}: K cache bytes differ"
            assert np.array_equal(_cache_bits(t["v"]), exp["v"]), f"slot {i}: V cache bytes differ"


def test_layer_graph_fused_equals_separate_bitwise(loop_setup):
    """The one-launch append + verify per layer gives the bits of the two separate calls."""
    from speculative_verify_kv_amd.step_graph import LayerStep
    w, t, slots, _ = loop_setup
    res = {}
    for form in ("fused", "separate"):
        step = LayerStep(t["k"], t["v"], t["bt"], t["ctx"], w.n_q, w.window, w.scale, w.H, VOCAB, form=form)
        outs = [step.new_outputs() for _ in range(N_SLOTS)]
        graphs = [step.capture(dev_in, outs[i]) for i, (_, dev_in) in enumerate(slots)]
        for _ in range(3):
            for g in graphs:
                g.replay()
        torch.cuda.synchronize()
        res[form] = outs
    for i in range(N_SLOTS):
        for key in ("out", "tgt", "acc", "nxt"):
            assert torch.equal(res["fused"][i][key], res["separate"][i][key]), f"slot {i} {key}"
