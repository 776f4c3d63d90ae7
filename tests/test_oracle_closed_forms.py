"""Pin the oracle to closed forms that follow from the pages' rules alone."""

import numpy as np
import pytest

import oracle
from workloads import gen


def _setup(R, H, S_r, ctx, rb=16, seed=0):
    st, lru = gen.initial_state(R, H, S_r)
    pool = np.random.default_rng(seed).integers(0, 256, size=(R * ctx, rb), dtype=np.uint8)
    hot = np.zeros((R * S_r, rb), dtype=np.uint8)
    return st, lru, pool, hot


@pytest.mark.parametrize("H,K", [(8, 8), (64, 16), (4096, 2048)])
def test_cold_start(H, K):
    """Empty state: miss j (j-th valid non-newest id in top-k order) takes slot j,
    lru becomes [M..H) ++ [0..M), every valid id is a miss."""
    rng = np.random.default_rng(H)
    R, ctx = 3, 4 * H
    st, lru, pool, hot = _setup(R, H, H + 1, ctx)
    rows, seq, topk = gen.random_case(rng, B=R, R=R, H=H, K=K, ctx=ctx, n_invalid=2)
    out, cnt = oracle.swap_in(topk=topk, req_rows=rows, seq_lens=seq, slot_tokens=st, lru=lru,
                              pool=pool, hot=hot, ctx_stride=ctx)
    for b in range(R):
        r, L = int(rows[b]), int(seq[b])
        j = 0
        for i in range(K):
            t = int(topk[b, i])
            if t < 0 or t >= L:
                assert out[b, i] == -1
            elif t == L - 1:
                assert out[b, i] == r * (H + 1) + H
            else:
                assert out[b, i] == r * (H + 1) + j
                assert st[r, j] == t
                assert np.array_equal(hot[r * (H + 1) + j], pool[r * ctx + t])
                j += 1
        assert cnt[b] == j
        assert lru[r].tolist() == list(range(j, H)) + list(range(j))


@pytest.mark.parametrize("seed", range(4))
def test_repeat_step_is_all_hits(seed):
    """The same top-k twice: no misses and the LRU is unchanged the second time."""
    rng = np.random.default_rng(seed)
    R, H, K, ctx = 4, 32, 12, 200
    st, lru, pool, hot = _setup(R, H, H + 1, ctx, seed=seed)
    for _ in range(3):  # some history first
        rows, seq, topk = gen.random_case(rng, B=R, R=R, H=H, K=K, ctx=ctx)
        oracle.swap_in(topk=topk, req_rows=rows, seq_lens=seq, slot_tokens=st, lru=lru, pool=pool,
                       hot=hot, ctx_stride=ctx)
    out1, _ = oracle.swap_in(topk=topk, req_rows=rows, seq_lens=seq, slot_tokens=st, lru=lru,
                             pool=pool, hot=hot, ctx_stride=ctx)
    st2, lru2, hot2 = st.copy(), lru.copy(), hot.copy()
    out2, cnt2 = oracle.swap_in(topk=topk, req_rows=rows, seq_lens=seq, slot_tokens=st, lru=lru,
                                pool=pool, hot=hot, ctx_stride=ctx)
    assert (cnt2 == 0).all()
    assert np.array_equal(out1, out2)
    assert np.array_equal(lru, lru2) and np.array_equal(st, st2) and np.array_equal(hot, hot2)


@pytest.mark.parametrize("seed", range(4))
def test_disjoint_step_evicts_oldest(seed):
    """No id of the new step is resident: the victims are the M oldest slots in
    LRU order and the LRU rotates by M."""
    rng = np.random.default_rng(50 + seed)
    H, K, ctx = 40, 10, 1000
    st, lru, pool, hot = _setup(1, H, H + 1, ctx, seed=seed)
    req = np.zeros(1, dtype=np.int64)
    sl = np.full(1, ctx, dtype=np.int64)
    ids = rng.permutation(ctx - 1)
    used = 0
    for _ in range(6):
        topk = ids[used:used + K].astype(np.int32)[None]
        used += K
        old = lru[0].tolist()
        out, cnt = oracle.swap_in(topk=topk, req_rows=req, seq_lens=sl, slot_tokens=st, lru=lru,
                                  pool=pool, hot=hot, ctx_stride=ctx)
        assert cnt[0] == K
        assert out[0].tolist() == old[:K]
        assert lru[0].tolist() == old[K:] + old[:K]


def test_all_newest_or_invalid_touches_nothing():
    H, K, ctx = 8, 4, 30
    st, lru, pool, hot = _setup(1, H, H + 1, ctx)
    lru[0] = np.asarray([3, 1, 4, 0, 5, 7, 2, 6], dtype=np.int16)
    st[0, :H] = np.arange(10, 10 + H)
    before = (st.copy(), lru.copy(), hot.copy())
    out, cnt = oracle.swap_in(topk=np.asarray([[29, -5, 30, 29]], dtype=np.int32),
                              req_rows=np.zeros(1, dtype=np.int64),
                              seq_lens=np.full(1, 30, dtype=np.int64), slot_tokens=st, lru=lru,
                              pool=pool, hot=hot, ctx_stride=ctx)
    assert out.tolist() == [[H, -1, -1, H]]
    assert cnt.tolist() == [0]
    # every slot was evictable and nothing missed: the LRU is unchanged
    assert np.array_equal(st, before[0]) and np.array_equal(lru, before[1])
    assert np.array_equal(hot, before[2])
