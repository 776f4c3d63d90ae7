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
