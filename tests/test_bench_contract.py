"""bench.py's command-line contract that needs no GPU: one GPU only."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_source_fingerprint_ignores_comments_only(tmp_path):
    """Counter traffic stays valid across comment edits and is dropped when the
    code changes."""
    sys.path.insert(0, ROOT)
    import bench
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("// header\nint f(int x) {\n  return x + 1;  // one\n}\n")
    b.write_text("/* another\n   header */\n\nint f(int x) {\n  return x + 1;\n}\n")
    c.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.source_fingerprint(str(a)) == bench.source_fingerprint(str(b))
    assert bench.source_fingerprint(str(a)) != bench.source_fingerprint(str(c))


def test_workload_description_follows_the_workload():
    sys.path.insert(0, ROOT)
    import bench
    import synth
    d = bench.workload_desc(synth.get_workload("ws1m"))
    assert d.startswith("1M-token workspace: 32768 blocks x 32 tokens, 64 layers")
    assert "512 query tokens, budget 4096 blocks (sink 1, recent 64)" in d
    d64 = bench.workload_desc(synth.get_workload("ctx64k"))
    assert d64.startswith("64K-token history: 2048 blocks") and "256 query tokens" in d64
