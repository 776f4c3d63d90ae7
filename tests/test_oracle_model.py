"""Pin the oracle's swap-in to independent models.

* Exhaustive: every top-k sequence over a tiny id universe, three calls deep,
  compared with the OrderedDict model in ``tests/model.py`` (a different
  formulation: a textbook LRU cache over the non-hit slots, hits appended).
* Textbook special case: with top_k = 1 and no newest or invalid ids the swap-in
  is an LRU cache of capacity H; hits/misses and the resident set must match
  ``TextbookLRU``.
* The two pages' LRU write-back formulas (different index algebra on the
  same compacted array) give the oracle's order.
* Every comparison with the model also covers the plan the oracle publishes
  for index-sharing layers: the miss mask and the compact copy list in miss
  order, and the running hit / miss counters against their definition (a
  pending id is a hit when its token sits in one of the row's LRU slots before
  the call).
"""

import itertools

import numpy as np
import pytest

import oracle
from model import TextbookLRU, lru_model_swap_in
from workloads import gen


def _pool(n, rb):
    rng = np.random.default_rng(n * 7 + rb)
    return rng.integers(0, 256, size=(n, rb), dtype=np.uint8)


def _expected_stats(c, st, *, R, H, ctx_stride, pool_rows, pool_nrows):
    """(hits, misses) of one call from the definition, on the state before it:
    over the real rows, a pending id (valid, not the newest token) is a hit when
    its token sits in one of the row's H LRU slots, else a miss."""
    hits = misses = 0
    nreal = c.get("num_real", -1)
    for b, r in enumerate(c["req_rows"].tolist()):
        if (nreal >= 0 and b >= nreal) or not 0 <= r < R:
            continue
        L = int(c["seq_lens"][b])
        resident = set(st[r, :H].tolist()) - {-1}
        for t in set(c["topk"][b].tolist()):
            if t < 0 or t >= L or t >= ctx_stride or t == L - 1:
                continue
            pr = int(pool_rows[r, t]) if pool_rows is not None else r * ctx_stride + t
            if not 0 <= pr < pool_nrows:
                continue
            if t in resident:
                hits += 1
            else:
                misses += 1
    return hits, misses


def _run_both(calls, *, R, H, S_r, ctx_stride, rb=8, slot_rows=None, pool_rows=None,
              hot_nrows=None, pool_nrows=None, kv=False):
    # The pool is a view past four spare rows, so a negative pool row that
    # were let through would read bytes (and differ from the model) instead
    # of leaving the array.
    n = pool_nrows or R * ctx_stride
    pool = _pool(n + 4, rb)[4:]
    hot_nrows = hot_nrows or R * S_r
    st_o, lru_o = gen.initial_state(R, H, S_r)
    st_m, lru_m = st_o.copy(), lru_o.copy()
    hot_o = np.zeros((hot_nrows, rb), dtype=np.uint8)
    hot_m = hot_o.copy()
    pool_v = (255 - pool) if kv else None
    hv_o = np.zeros_like(hot_o) if kv else None
    hv_m = np.zeros_like(hot_o) if kv else None
    stats = np.zeros(2, np.uint64)
    want = np.zeros(2, np.int64)
    for c in calls:
        kw = dict(topk=c["topk"], req_rows=c["req_rows"], seq_lens=c["seq_lens"],
                  ctx_stride=ctx_stride, num_real=c.get("num_real", -1), slot_rows=slot_rows,
                  pool_rows=pool_rows, pool=pool)
        want += _expected_stats(c, st_o, R=R, H=H, ctx_stride=ctx_stride, pool_rows=pool_rows,
                                pool_nrows=pool.shape[0])
        out_o, cnt_o, plan_o = oracle.swap_in(slot_tokens=st_o, lru=lru_o, hot=hot_o, plan=True,
                                              pool_v=pool_v, hot_v=hv_o, stats=stats, **kw)
        # running counters: hits and misses from the definition, accumulated
        assert stats.tolist() == want.tolist()
        out_m, cnt_m, plan_m = lru_model_swap_in(slot_tokens=st_m, lru=lru_m, hot=hot_m, plan=True,
                                                 pool_v=pool_v, hot_v=hv_m, **kw)
        if kv:
            assert np.array_equal(hv_o, hv_m)
        # the plan: which entries missed, and the copies in the order made
        assert plan_o["miss_mask"].tolist() == plan_m["miss_mask"].tolist()
        assert plan_o["count"].tolist() == cnt_m.tolist()
        for b, cp in enumerate(plan_m["copies"]):
            n = len(cp)
            assert list(zip(plan_o["src"][b, :n].tolist(), plan_o["dst"][b, :n].tolist())) == cp
        assert out_o.tolist() == out_m.tolist()
        assert cnt_o.tolist() == cnt_m.tolist()
        assert st_o.tolist() == st_m.tolist()
        assert lru_o.tolist() == lru_m.tolist()
        assert np.array_equal(hot_o, hot_m)


def test_exhaustive_tiny_universe():
    """H=3, K=2, seq_len 5 (ids 0..4 valid, 4 newest, -1 and 5 invalid), 3 calls,
    every ordered pair of distinct ids per call: 42^3 = 74088 sequences is too many
    for a unit test, so every pair at call 1 and 2, and a fixed set at call 3."""
    H, K, S_r, L = 3, 2, 4, 5
    ids = [-1, 0, 1, 2, 3, 4, 5]
    pairs = [p for p in itertools.permutations(ids, 2) if not (p[0] == p[1])]
    third = [(0, 1), (3, 2), (4, 1), (5, -1), (2, 0)]
    req = np.zeros(1, dtype=np.int64)
    sl = np.full(1, L, dtype=np.int64)
    n = 0
    for p1 in pairs:
        for p2 in pairs:
            for p3 in third:
                calls = [dict(topk=np.asarray([p], dtype=np.int32), req_rows=req, seq_lens=sl)
                         for p in (p1, p2, p3)]
                _run_both(calls, R=1, H=H, S_r=S_r, ctx_stride=8)
                n += 1
    assert n == len(pairs) ** 2 * len(third)


def test_exhaustive_k3_h4_growing_seq():
    """Every 3-subset order of ids 0..6 at call 1 (seq_len 7), then every 3-subset
    of 0..7 at call 2 (seq_len 8): newest moves from 6 to 7 between calls."""
    H, K, S_r = 4, 3, 5
    req = np.zeros(1, dtype=np.int64)
    c1 = list(itertools.permutations(range(7), 3))[::7]
    c2 = list(itertools.combinations(range(8), 3))
    for a in c1:
        for b in c2:
            calls = [dict(topk=np.asarray([a], dtype=np.int32), req_rows=req,
                          seq_lens=np.full(1, 7, dtype=np.int64)),
                     dict(topk=np.asarray([b], dtype=np.int32), req_rows=req,
                          seq_lens=np.full(1, 8, dtype=np.int64))]
            _run_both(calls, R=1, H=H, S_r=S_r, ctx_stride=8)


@pytest.mark.parametrize("seed", range(6))
def test_random_multirow_with_tables(seed, kv=False):
    """Random calls over permuted state rows, padding, invalid ids, slot-row and
    pool-row tables. About a tenth of the pool-row entries are negative (-1 to
    -3): those ids have no pool row and are invalid."""
    rng = np.random.default_rng(seed)
    R, B, H, K, ctx = 5, 3, 12, 6, 40
    S_r = H + 2
    slot_rows = rng.permutation(R * S_r + 7)[:R * S_r].astype(np.int32).reshape(R, S_r)
    pool_rows = rng.permutation(R * ctx + 9)[:R * ctx].astype(np.int64).reshape(R, ctx)
    neg = rng.random(pool_rows.shape) < 0.1
    pool_rows[neg] = -rng.integers(1, 4, int(neg.sum()))
    calls = []
    for _ in range(12):
        rows, seq, topk = gen.random_case(rng, B=B, R=R, H=H, K=K, ctx=ctx, n_invalid=int(rng.integers(0, 3)))
        calls.append(dict(topk=topk, req_rows=rows, seq_lens=seq,
                          num_real=int(rng.integers(1, B + 1)) if rng.random() < 0.3 else -1))
    _run_both(calls, R=R, H=H, S_r=S_r, ctx_stride=ctx, slot_rows=slot_rows, pool_rows=pool_rows,
              hot_nrows=R * S_r + 7, pool_nrows=R * ctx + 9, kv=kv)


@pytest.mark.parametrize("seed", range(3))
def test_random_multirow_kv(seed):
    """The same random calls with a V pool: V rows follow the K rows."""
    test_random_multirow_with_tables(100 + seed, kv=True)


def test_tiny_workload_trace_matches_model():
    cfg = gen.TINY
    calls = [dict(topk=tk, req_rows=np.arange(cfg.B, dtype=np.int64), seq_lens=gen.seq_lens(cfg, t))
             for t, tk in enumerate(gen.topk_trace(cfg))]
    _run_both(calls, R=cfg.R, H=cfg.H, S_r=cfg.S_r, ctx_stride=cfg.ctx, rb=cfg.row_bytes)


@pytest.mark.parametrize("H,universe,seed", [(1, 4, 0), (4, 9, 1), (16, 40, 2), (64, 100, 3)])
def test_topk1_is_textbook_lru(H, universe, seed):
    """K=1: each call is one access to an LRU cache of capacity H."""
    rng = np.random.default_rng(seed)
    L = universe + 1                          # newest = universe, never drawn
    st, lru = gen.initial_state(1, H, H + 1)
    pool = _pool(universe + 1, 4)
    hot = np.zeros((H + 1, 4), dtype=np.uint8)
    ref = TextbookLRU(H)
    for _ in range(2000):
        t = int(rng.integers(0, universe))
        out, cnt = oracle.swap_in(topk=np.asarray([[t]], dtype=np.int32),
                                  req_rows=np.zeros(1, dtype=np.int64),
                                  seq_lens=np.full(1, L, dtype=np.int64), slot_tokens=st,
                                  lru=lru, pool=pool, hot=hot, ctx_stride=L)
        was_hit = ref.access(t)
        assert int(cnt[0]) == (0 if was_hit else 1)
        resident = [int(st[0, s]) for s in lru[0] if st[0, s] >= 0]
        assert resident == ref.resident()     # same tokens, LRU first
        assert np.array_equal(hot[out[0, 0]], pool[t])


def _p1_writeback(lru_out, H, hits, misses):
    """SGLang page's write-back index algebra on the compacted array
    [hits forward | evictables backward]."""
    E = H - hits
    new = [None] * H
    for i in range(H):
        if i < misses:
            new[E - misses + i] = lru_out[H - 1 - i]
        elif i < E:
            new[i - misses] = lru_out[H - 1 - i]
        else:
            new[i] = lru_out[i - E]
    return new


def _p2_writeback(lru_out, H, hits, misses):
    """vLLM page's write-back index algebra on the same compacted array."""
    rem = (H - hits) - misses
    new = [None] * H
    for i in range(H):
        if i < rem:
            new[i] = lru_out[H - 1 - misses - i]
        elif i < rem + misses:
            new[i] = lru_out[H - 1 - (i - rem)]
        else:
            new[i] = lru_out[i - rem - misses]
    return new


@pytest.mark.parametrize("seed", range(20))
def test_both_pages_writeback_match_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    H, K = int(rng.integers(2, 30)), None
    K = int(rng.integers(1, H + 1))
    L = 3 * H + 2
    st, lru = gen.initial_state(1, H, H + 1)
    pool = _pool(L, 4)
    hot = np.zeros((H + 1, 4), dtype=np.uint8)
    req = np.zeros(1, dtype=np.int64)
    seql = np.full(1, L, dtype=np.int64)
    for _ in range(5):
        ids = rng.choice(L - 1, size=K, replace=False).astype(np.int32)[None]
        old_lru = lru[0].tolist()
        old_tok = st[0].copy()
        before = {int(old_tok[s]) for s in range(H) if old_tok[s] >= 0}
        out, cnt = oracle.swap_in(topk=ids, req_rows=req, seq_lens=seql, slot_tokens=st, lru=lru,
                                  pool=pool, hot=hot, ctx_stride=L)
        want = set(ids[0].tolist())
        hit_slots = [s for s in old_lru if old_tok[s] in want]
        evict = [s for s in old_lru if old_tok[s] not in want or old_tok[s] < 0]
        compact = hit_slots + [None] * 0 + evict[::-1]          # [hits fwd | evict bwd]
        M = int(cnt[0])
        assert M == len(want - before)
        assert _p1_writeback(compact, H, len(hit_slots), M) == lru[0].tolist()
        assert _p2_writeback(compact, H, len(hit_slots), M) == lru[0].tolist()
