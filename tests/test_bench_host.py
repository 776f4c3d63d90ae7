"""Host-side logic of bench.py (no GPU): the oracle baseline split over
threads does the same work as the single-thread pass."""

import bench
from workloads import gen


def test_threaded_oracle_baseline_copies_the_same_rows():
    cfg = gen.DSV32.with_(B=6, ctx=4096, H=512, K=256)
    one = bench.cpu_baseline(cfg, 1, 3, 0.0, threads=1)
    many = bench.cpu_baseline(cfg, 1, 3, 0.0, threads=4)
    assert one[0] == many[0] > 0
    assert one[2] == many[2] == 1


def test_host_threads_is_bounded():
    n = bench.host_threads()
    assert 1 <= n <= 16


def _run_bench(*args):
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    return subprocess.run([sys.executable, os.path.join(root, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr


def test_unknown_legs_are_refused():
    r = _run_bench("--only", "headline,nonsense")
    assert r.returncode == 2 and "nonsense" in r.stderr


def test_traffic_is_reported_only_for_the_sources_it_was_measured_on():
    import json
    import os
    path = os.path.join(bench.ROOT, "profiles", "swap_copy_traffic.json")
    entries = json.load(open(path))["workloads"]
    for name, w in entries.items():
        want = w["bytes_per_launch"] if w["kernel_sources_sha256_16"] == bench.sources_hash(
            w["kernel_sources"]) else None
        assert bench.measured_traffic(name) == want


def test_source_hash_ignores_comments_and_layout_but_not_code(tmp_path, monkeypatch):
    src = 'int f(int x) {  // doubles x\n  /* note */ return 2 * x; }\nconst char* s = "a // b";\n'
    (tmp_path / "a.hip").write_text(src)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.sources_hash(["a.hip"])
    (tmp_path / "a.hip").write_text(src.replace("doubles x", "twice x").replace("  /* note */", ""))
    assert bench.sources_hash(["a.hip"]) == h0
    (tmp_path / "a.hip").write_text(src.replace('"a // b"', '"a // c"'))
    assert bench.sources_hash(["a.hip"]) != h0      # text inside a literal is code
    (tmp_path / "a.hip").write_text(src.replace("2 * x", "3 * x"))
    assert bench.sources_hash(["a.hip"]) != h0
