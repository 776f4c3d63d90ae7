"""Pin the oracle's plan outputs and its plan replay.

The plan is what index-sharing layers reuse (vLLM hisparse_kernels.cu,
hisparse_gather_plan_kernel and hisparse_gather_compact_kernel): a mask of the
entries that missed and the compact list of (pool row, hot row) copies in miss
order. Pins, none of which retypes the oracle:

* the hand-derived replay in ``tests/golden/plan_replay_worked_example.json``
  (count clamping, skipped entries, a zero-filled row whose source is past
  the end of the pool);
* replaying a call's list on the hot buffer as it was before the call gives
  the hot buffer the call produced, on every step of the small workload traces;
* the list is the dense plan read in top-k order: for each masked entry, the
  pool row of its id and the hot row it was given (out_rows);
* replay on several layers equals numpy fancy indexing layer by layer;
* the mask against the model is covered by ``test_oracle_model``.
"""

import json
import os

import numpy as np
import pytest

import oracle
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_replay_worked_example():
    fx = json.load(open(os.path.join(GOLDEN, "plan_replay_worked_example.json")))
    L, rb = fx["layers"], fx["row_bytes"]
    pools = [np.array([[(100 * l + 10 * p + j) for j in range(rb)] for p in range(fx["pool_nrows"])],
                      dtype=np.uint8) for l in range(L)]
    hots = [np.full((fx["hot_nrows"], rb), fx["hot_fill"][l], dtype=np.uint8) for l in range(L)]
    z = oracle.gather_compact_layers(np.asarray(fx["count"], np.int32), np.asarray(fx["src"], np.int64),
                                     np.asarray(fx["dst"], np.int32), pools, hots)
    assert z == fx["expect_zeroed"]
    for l in range(L):
        assert hots[l].tolist() == fx["expect_hot"][l]


def _pool_of(cfg_ctx, r, t, pool_rows):
    return int(pool_rows[r, t]) if pool_rows is not None else r * cfg_ctx + t


@pytest.mark.parametrize("name", ["tiny", "adversarial_small"])
def test_replay_reproduces_each_call(name):
    if name == "tiny":
        cfg = gen.TINY
    else:
        cfg = gen.ADVERSARIAL.with_(name="adv_small", B=3, H=64, K=32, ctx=512, row_bytes=12,
                                    steps=5, collide_window=16, collide_table=128)
    pool = gen.fill_pool(cfg.seed, np.empty((cfg.pool_nrows, cfg.row_bytes), np.uint8))
    tok, lru = gen.initial_state(cfg)
    hot = np.zeros((cfg.R * cfg.S_r, cfg.row_bytes), np.uint8)
    rows = np.arange(cfg.B, dtype=np.int64)
    for t, topk in enumerate(gen.topk_trace(cfg, cfg.steps)):
        before = hot.copy()
        seq = gen.seq_lens(cfg, t)
        out, cnt, plan = oracle.swap_in(topk=topk, req_rows=rows, seq_lens=seq, slot_tokens=tok,
                                        lru=lru, pool=pool, hot=hot, ctx_stride=cfg.ctx, plan=True)
        assert plan["count"].tolist() == cnt.tolist()
        assert (plan["miss_mask"].sum(axis=1) == cnt).all()
        z = oracle.gather_compact_layers(plan["count"], plan["src"], plan["dst"], [pool], [before])
        assert z == 0
        assert np.array_equal(before, hot), f"step {t}: replay differs from the call"
        # the list is the dense plan (mask, out_rows, each id's pool row) in top-k order
        for b in range(cfg.B):
            idx = np.nonzero(plan["miss_mask"][b])[0]
            dense = [(_pool_of(cfg.ctx, b, int(topk[b, i]), None), int(out[b, i])) for i in idx]
            n = int(cnt[b])
            assert dense == list(zip(plan["src"][b, :n].tolist(), plan["dst"][b, :n].tolist()))


@pytest.mark.parametrize("seed", range(4))
def test_replay_layers_matches_numpy(seed):
    rng = np.random.default_rng(seed)
    B, K, L, rb, P, Hn = 4, 9, 3, 12, 40, 30
    count = rng.integers(-2, K + 3, size=B).astype(np.int32)
    src = rng.integers(-3, P + 4, size=(B, K)).astype(np.int64)
    # destinations are distinct across the whole plan (a plan's hot rows are)
    flat = rng.permutation(Hn + 6)[:B * K].reshape(B, K) - 3
    dst = flat.astype(np.int32)
    pools = [rng.integers(0, 256, size=(P, rb), dtype=np.uint8) for _ in range(L)]
    hots = [rng.integers(0, 256, size=(Hn, rb), dtype=np.uint8) for _ in range(L)]
    want = [h.copy() for h in hots]
    zeroed = 0
    for l in range(L):
        for b in range(B):
            n = min(max(int(count[b]), 0), K)
            d, s = dst[b, :n].astype(np.int64), src[b, :n]
            ok = (s >= 0) & (d >= 0) & (d < Hn)
            has = ok & (s < P)
            want[l][d[has]] = pools[l][s[has]]
            want[l][d[ok & ~has]] = 0
            zeroed += int((ok & ~has).sum())
    z = oracle.gather_compact_layers(count, src, dst, pools, hots)
    assert z == zeroed
    for l in range(L):
        assert np.array_equal(hots[l], want[l])


def test_replay_empty_and_no_layers():
    c = np.zeros(2, np.int32)
    s = np.zeros((2, 3), np.int64)
    d = np.zeros((2, 3), np.int32)
    hot = np.full((4, 8), 9, np.uint8)
    assert oracle.gather_compact_layers(c, s, d, [np.zeros((4, 8), np.uint8)], [hot]) == 0
    assert (hot == 9).all()
