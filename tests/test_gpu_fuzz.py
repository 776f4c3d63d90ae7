"""Seeded random sweep of the swap-in against the oracle.

Each case draws its own sizes and options from a fixed seed: batch, hot size
(from 1 to past 4096, many off the 64-slot and 1024-lane grids), top-k, a
context short enough for a direct table or past 65 536 positions (hashed
plans), row size (4 bytes to 1152), pool kind, and either a workload trace
(uniform or Zipf new ids, random retention) or random calls with invalid ids,
padding rows, permuted state rows and, in some cases, slot-row and pool-row
tables. Every call is compared with the oracle on outputs, counts, state, the
running counters and the whole hot buffer (gpu_harness.ParityRun).
"""

import os

import numpy as np
import pytest

from workloads import gen

pytestmark = pytest.mark.gpu

N_CASES = int(os.environ.get("HS_FUZZ_CASES", 64))   # more seeds of the same draw on request
H_CHOICES = [1, 2, 3, 7, 31, 63, 64, 65, 100, 255, 256, 1000, 1023, 1024, 2047, 4096, 4100, 5000]
RB_CHOICES = [4, 8, 16, 48, 132, 656, 1152]
POOL_CAP = 48 << 20   # bytes of pool per case


def draw_case(i: int) -> dict:
    rng = np.random.default_rng(7_000 + i)
    H = int(rng.choice(H_CHOICES))
    K = int(rng.integers(1, min(H, 4096) + 1))
    big = bool(rng.random() < 0.25)                     # positions past 65 536: hashed plans
    ctx = int(rng.integers(65_537, 90_000)) if big else int(rng.integers(K + 4, min(65_536, 4 * K + 4_096) + 1))
    B = int(rng.integers(1, 4 if big else 10))
    rb = int(rng.choice(RB_CHOICES))
    while B * ctx * rb > POOL_CAP and rb > 4:
        rb = max(r for r in RB_CHOICES if r < rb)
    mode = str(rng.choice(["trace", "random"]))
    return dict(i=i, H=H, K=K, ctx=ctx, B=B, row_bytes=rb,
                kind=str(rng.choice(["host", "device"])), mode=mode,
                dist=str(rng.choice(["uniform", "zipf"])), rho=float(rng.random()),
                tables=mode == "random" and bool(rng.random() < 0.4),
                extra_rows=int(rng.integers(0, 4)), seed=int(rng.integers(1, 2**31)))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case_matches_oracle(i):
    import gpu_harness as h
    c = draw_case(i)
    h.log(f"  fuzz case {c}")
    steps = 3
    cfg = gen.SwapConfig(f"fuzz{i}", B=c["B"], H=c["H"], K=c["K"], ctx=c["ctx"],
                         row_bytes=c["row_bytes"], steps=steps, rho=c["rho"], dist=c["dist"],
                         pool_kind=c["kind"], seed=c["seed"])
    check = cfg.K * cfg.B <= 4096
    if c["mode"] == "trace":
        run = h.ParityRun(cfg)
        for t, topk in enumerate(gen.topk_trace(cfg, steps)):
            _, cnt = run.step(topk, gen.seq_lens(cfg, t), check_invariants=check)
            h.log(f"  fuzz{i} step {t}: misses {int(cnt.sum())} ok")
        return
    rng = np.random.default_rng(c["seed"])
    R = cfg.B + c["extra_rows"]
    kw = {}
    if c["tables"]:
        S_r = cfg.S_r
        hot_nrows = R * S_r + int(rng.integers(0, 9))
        kw["slot_rows"] = rng.permutation(hot_nrows)[:R * S_r].astype(np.int32).reshape(R, S_r)
        kw["pool_rows"] = rng.permutation(R * cfg.ctx).astype(np.int64).reshape(R, cfg.ctx)
        kw["hot_nrows"] = hot_nrows
        kw["pool_nrows"] = R * cfg.ctx - int(rng.integers(0, 20))   # the last rows have no pool row
    run = h.ParityRun(cfg, R=R, req_rows=rng.permutation(R)[:cfg.B].astype(np.int64), **kw)
    for t in range(steps):
        rows, seq, topk = gen.random_case(rng, B=cfg.B, R=R, H=cfg.H, K=cfg.K, ctx=cfg.ctx,
                                          n_invalid=int(rng.integers(0, 3)))
        run.req_rows = rows
        num_real = int(rng.integers(0, cfg.B + 1)) if t == 2 else -1
        _, cnt = run.step(topk, seq, num_real=num_real, check_invariants=check)
        h.log(f"  fuzz{i} step {t}: misses {int(cnt.sum())} ok")


def test_the_sweep_reaches_every_plan_and_option():
    """The drawn cases cover what the sweep is for (checked on the CPU side of
    the draw, so a change of seeds cannot quietly narrow it)."""
    cases = [draw_case(i) for i in range(N_CASES)]
    assert any(c["ctx"] > 65_536 for c in cases) and any(c["ctx"] <= 65_536 for c in cases)
    assert {c["kind"] for c in cases} == {"host", "device"}
    assert {c["mode"] for c in cases} == {"trace", "random"}
    assert any(c["tables"] for c in cases)
    assert any(c["row_bytes"] % 16 for c in cases) and any(c["row_bytes"] % 16 == 0 for c in cases)
    assert any(c["H"] % 64 for c in cases) and any(c["K"] > 2048 for c in cases)
