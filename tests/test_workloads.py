"""The synthetic traces have the shapes and statistics the workloads name."""

import numpy as np
import pytest

from workloads import gen


def test_pool_rows_are_counter_based():
    full = gen.fill_pool(7, np.empty((gen.POOL_CHUNK_ROWS * 2 + 100, 36), np.uint8))
    part = gen.pool_rows_bytes(7, 4000, 300, 36)
    assert np.array_equal(full[4000:4300], part)
    assert not np.array_equal(full[0], full[1])


def _check_trace(cfg, steps):
    prev = None
    for t, tk in enumerate(gen.topk_trace(cfg, steps)):
        L = cfg.seq_len(t)
        assert tk.shape == (cfg.B, cfg.K) and tk.dtype == np.int32
        for b in range(cfg.B):
            row = tk[b]
            assert len(np.unique(row)) == cfg.K, "ids must be distinct"
            assert row.min() >= 0 and row.max() < L
            if prev is not None:
                kept = len(set(row.tolist()) & set(prev[b].tolist()))
                assert kept >= int(round(cfg.rho * cfg.K))
        prev = tk
    return prev


def test_tiny_trace():
    cfg = gen.TINY
    last = None
    for t, tk in enumerate(gen.topk_trace(cfg)):
        if t % 2 == 1:
            assert cfg.seq_len(t) - 1 in tk[0].tolist()
        last = tk
    _check_trace(cfg, cfg.steps)
    assert cfg.seq_len(cfg.steps - 1) == cfg.ctx


def test_zipf_favours_recent():
    cfg = gen.DSV32.with_(B=2)
    tk = next(iter(gen.topk_trace(cfg, 1)))
    L = cfg.seq_len(0)
    ranks = L - tk.astype(np.int64)
    assert np.median(ranks) < L / 8


def test_collide_ids_share_low_bit_buckets():
    cfg = gen.ADVERSARIAL.with_(B=2)
    tk = _check_trace(cfg, 2)
    for b in range(cfg.B):
        ids = tk[b].astype(np.uint64)
        bucket = ((ids * np.uint64(gen.KNUTH_A)) & np.uint64(0xFFFFFFFF)) % np.uint64(cfg.collide_table)
        span = np.unique(bucket)
        assert len(span) <= cfg.collide_window


def test_kernel_hash_ids_share_high_bit_buckets():
    cfg = gen.ADVERSARIAL_KERNEL_HASH.with_(B=2)
    tk = _check_trace(cfg, 2)
    for b in range(cfg.B):
        ids = tk[b].astype(np.uint64)
        bucket = ((ids * np.uint64(gen.KNUTH_A)) & np.uint64(0xFFFFFFFF)) >> np.uint64(32 - 11)
        assert len(np.unique(bucket)) <= cfg.collide_window
        # one window: every id's bucket within 128 of some start (wrapping)
        starts = np.unique(bucket.astype(np.int64))
        assert any(((bucket.astype(np.int64) - s0) % 2048 < 128).all() for s0 in starts)


@pytest.mark.parametrize("cfg", [gen.DEVPOOL.with_(B=2), gen.DSV32.with_(B=2)])
def test_retention(cfg):
    _check_trace(cfg, 3)


def test_transfer_indices():
    s, d = gen.transfer_indices(gen.ALL_LAYER)
    assert len(np.unique(d)) == gen.ALL_LAYER.n_pairs and s.dtype == np.int64
    assert s.max() < gen.ALL_LAYER.rows_per_layer
