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


def test_traffic_lookups_name_profiled_kernels():
    """Every kernel the bench line attaches counter traffic to names an entry of
    the committed counter summary, and its template arguments name a kernel the
    library launches (a renamed instantiation would silently report null)."""
    sys.path.insert(0, ROOT)
    import bench
    per = json.load(open(os.path.join(ROOT, "profiles", "ws1m_traffic.json")))["per_dispatch"]
    looks = [("score_pass1_mfma", bench.SCORE_KERNEL_TAIL),
             ("score_pass2_mfma", bench.SCORE_KERNEL_TAIL),
             bench.REMAT_VIEW_KERNEL, bench.REMAT_DELTA_KERNEL]
    for short, tail in looks:
        hits = [n for n in per if n.split("<")[0].endswith(short) and n.endswith(tail)]
        assert len(hits) == 1, (short, tail)
    # the 10M- and 64K-token lines read their own counter files
    for name, (short, tail) in (("ws10m", ("score_stored_pass1_mfma", bench.STORED_KERNEL_TAIL)),
                                ("ctx64k", bench.REMAT_VIEW_KERNEL)):
        per_w = json.load(open(os.path.join(ROOT, "profiles", f"{name}_traffic.json")))
        hits = [n for n in per_w["per_dispatch"]
                if n.split("<")[0].endswith(short) and n.endswith(tail)]
        assert len(hits) == 1, (name, short, tail)
    src = open(os.path.join(ROOT, "attention_space_block_amd", "csrc", "remat.hip")).read()
    for _, tail in (bench.REMAT_VIEW_KERNEL, bench.REMAT_DELTA_KERNEL):
        delta, copy_v = tail.strip("<>").split(", ")[3:]
        assert f"remat_kernel<T, D, LAY, {delta}, {copy_v}>" in src


def test_every_kernel_maps_to_the_file_that_defines_it():
    """Counter traffic is tied to the source file of its kernel: every
    __global__ kernel of the library maps to the file it is defined in, and
    kernels the library does not define (the calibration copy) map to none."""
    import glob
    import re
    sys.path.insert(0, ROOT)
    import bench
    pat = re.compile(r"__global__\s+(?:__launch_bounds__\([^)]*\)\s+)?void\s+(\w+)\s*\(")
    seen = 0
    for path in glob.glob(os.path.join(ROOT, "attention_space_block_amd", "csrc", "*.hip")):
        rel = os.path.relpath(path, ROOT)
        for name in pat.findall(open(path).read()):
            assert bench._source_of(f"kvm::{name}<int>") == rel, name
            seen += 1
    assert seen >= 20
    assert bench._source_of("at::native::vectorized_elementwise_kernel<4>") is None
