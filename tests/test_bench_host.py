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
