"""Run the workload traces through the oracle and check every invariant after
every step. Full size for the tiny workload; the larger ones with fewer rows
and steps so the CPU suite stays short (same H, K, distributions and ratios)."""

import numpy as np
import pytest

import oracle
from invariants import check_swap_step
from workloads import gen


def _trace(cfg, steps, check_every=1):
    st, lru = gen.initial_state(cfg)
    pool = gen.fill_pool(cfg.seed, np.empty((cfg.pool_nrows, cfg.row_bytes), np.uint8))
    pool_copy = pool.copy()
    hot = np.zeros((cfg.R * cfg.S_r, cfg.row_bytes), np.uint8)
    rows = np.arange(cfg.B, dtype=np.int64)
    counts_seen = []
    for t, topk in enumerate(gen.topk_trace(cfg, steps)):
        seq = gen.seq_lens(cfg, t)
        # the harness writes the newest token's row into slot H before the call
        loc = rows * cfg.S_r + cfg.H
        oracle.store_kv_scatter(pool[rows * cfg.ctx + seq - 1], hot, loc)
        before = (st.copy(), lru.copy(), hot.copy())
        out, cnt = oracle.swap_in(topk=topk, req_rows=rows, seq_lens=seq, slot_tokens=st, lru=lru,
                                  pool=pool, hot=hot, ctx_stride=cfg.ctx)
        counts_seen.append(cnt.copy())
        if t % check_every == 0:
            check_swap_step(topk=topk, req_rows=rows, seq_lens=seq, num_real=-1,
                            ctx_stride=cfg.ctx, pool=pool, tokens_before=before[0],
                            lru_before=before[1], hot_before=before[2], tokens_after=st,
                            lru_after=lru, hot_after=hot, out=out, counts=cnt)
    assert np.array_equal(pool, pool_copy)          # I10
    return np.asarray(counts_seen)


def test_tiny_trace_invariants():
    counts = _trace(gen.TINY, gen.TINY.steps)
    assert (counts[0] == gen.TINY.K).all()               # cold start: all misses


def test_dsv32_like_reduced():
    cfg = gen.DSV32.with_(B=2)
    counts = _trace(cfg, 6, check_every=5)
    assert (counts[0] <= cfg.K).all() and (counts[1:] < cfg.K * (1 - cfg.rho) + 1).all()


def test_device_pool_reduced():
    cfg = gen.DEVPOOL.with_(B=2)
    counts = _trace(cfg, 4, check_every=3)
    # 60% retention, uniform new ids over 16k: at most 40% of K can miss
    assert (counts[1:] <= int(round(0.4 * cfg.K))).all()


@pytest.mark.parametrize("rb", [1152, 132])
def test_adversarial_reduced(rb):
    cfg = gen.ADVERSARIAL.with_(B=2, row_bytes=rb)
    counts = _trace(cfg, 3, check_every=2)
    assert (counts[0] == cfg.K).all()


def test_adversarial_kernel_hash_reduced():
    cfg = gen.ADVERSARIAL_KERNEL_HASH.with_(B=2)
    counts = _trace(cfg, 3, check_every=2)
    assert (counts[0] == cfg.K).all()
