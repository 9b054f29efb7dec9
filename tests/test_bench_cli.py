"""bench.py's contract checks that need no GPU: more than one GPU is refused
with a message, and the roofline's traffic figure is taken only from a
profile of the same code (comments and whitespace do not count)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr


def test_source_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    csrc = tmp_path / "mixed_precision_gemm_amd" / "csrc"
    inc = tmp_path / "include"
    csrc.mkdir(parents=True)
    inc.mkdir()
    (inc / "a.h").write_text("int f(void);\n")
    src = csrc / "k.hip"
    src.write_text("int g() { return 1; }  // one\n/* block */\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h1 = bench.kernel_source_hash()
    src.write_text("int g() {\n    return 1;\n}  // another comment\n")
    assert bench.kernel_source_hash() == h1
    src.write_text("int g() { return 2; }\n")
    assert bench.kernel_source_hash() != h1


def test_traffic_only_for_the_profiled_workload():
    assert bench.profiled_traffic("square nn 4096x4096x4096 f16") is None
    assert bench.profiled_traffic("square tt 8192x8192x8192 f16") is None
    args = bench.parse(["--workload", "linear", "--case", "16,11008"])
    assert bench.bench_key(args) == "linear 16,11008 f16"
    assert bench.bench_key(bench.parse([])) == "square nn 8192x8192x8192 f16"


def test_committed_profiles_name_their_run():
    """Every committed summary carries the key of the bench run it profiled,
    the hash of the code it profiled and the commands that made it."""
    import glob
    paths = glob.glob(os.path.join(ROOT, "profiles", "*.md"))
    assert paths
    for p in paths:
        f = bench.profile_fields(p)
        assert "kernel_source_hash" in f, p
        assert "rocprofv3" in open(p).read(), p
