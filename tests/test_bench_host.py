"""CPU tests of bench.py's host logic: the one-GPU contract, workload naming and the
committed traffic summaries' code hash."""
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_every_workload_is_named():
    for key in synth.NAMED:
        w = synth.named_workload(key)
        name = bench.DESCRIPTIONS.get(key, w.name)
        assert isinstance(name, str) and name
        assert "model" not in name.lower()


def test_code_hash_ignores_comments_and_blank_lines():
    code = "int a = 1;  // one\n\n/* block\n comment */int b = 2;\n"
    assert bench._code_only(code) == "int a = 1;\nint b = 2;"
    assert bench._code_only(code) == bench._code_only("int a = 1;\n// only a comment\nint b = 2;   \n")
    assert bench._code_only("x = 1;") != bench._code_only("x = 2;")


def test_traffic_summary_of_other_sources_is_ignored(tmp_path, monkeypatch):
    lines = ["# a summary", "kernel: k", "hbm_bytes_per_call: 12345", "source_hash: {}"]
    good = tmp_path / "good.txt"
    good.write_text("\n".join(lines).format(bench.source_hash()) + "\n")
    stale = tmp_path / "stale.txt"
    stale.write_text("\n".join(lines).format("0123456789abcdef") + "\n")
    monkeypatch.setitem(bench.TRAFFIC_SUMMARIES, "good", str(good))
    monkeypatch.setitem(bench.TRAFFIC_SUMMARIES, "stale", str(stale))
    assert bench.read_traffic("good") == 12345.0
    assert bench.read_traffic("stale") is None
    assert bench.read_traffic("no such workload") is None


def test_window_and_block_order_overrides():
    # --window: the window-188 workloads take another window, their recent rows follow it,
    # and the algorithmic bytes count the new union window; --unshuffled: each sequence's
    # blocks in order, the same blocks referenced; both refused where they do not apply
    import types
    import numpy as np
    base = synth.named_workload("verify")
    args = types.SimpleNamespace(unshuffled=False, window=185)
    w = bench.workload_of("verify", args, synth)
    assert (base.window, w.window) == (188, 185) and w.meta["recent"] == 185 + 8 - 1
    assert base.name.endswith("_w188_nq8") and w.name.endswith("_w185_nq8")
    per_key = base.Hkv * base.D * 2 * 2
    assert bench.algorithmic_bytes(base) - bench.algorithmic_bytes(w) == base.B * 3 * per_key
    same = bench.workload_of("verify", types.SimpleNamespace(unshuffled=False, window=0), synth)
    assert np.array_equal(same.block_table, base.block_table) and np.array_equal(same.q, base.q)
    flat = bench.workload_of("verify", types.SimpleNamespace(unshuffled=True, window=0), synth)
    nb = (base.ctx_len + base.bs - 1) // base.bs
    for b in range(base.B):
        assert np.array_equal(flat.block_table[b, :nb[b]], np.arange(nb[:b].sum(), nb[:b + 1].sum()))
    assert sorted(flat.block_table[flat.block_table >= 0]) == sorted(base.block_table[base.block_table >= 0])
    for key in ("tiny_decode", "fullctx_1024"):
        try:
            bench.workload_of(key, types.SimpleNamespace(unshuffled=False, window=100), synth)
        except SystemExit as e:
            assert "--window" in str(e)
        else:
            raise AssertionError(f"--window accepted for {key}")
