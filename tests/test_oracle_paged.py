"""Pin the oracle's vLLM-style paged addressing and write invalidation.

* ``tests/golden/swap_in_paged_worked_example.json``: three calls and an
  invalidation derived by hand (vLLM hisparse_kernels.cu:
  hisparse_resolve_residency_kernel, get_physical_hot_row, store_hot_index,
  hisparse_invalidate_written_slots_kernel) -- outputs, counts, slot keys,
  LRU rows, attention indices and hot rows after every step.
* The OrderedDict model (``tests/model.py``) with its own block-table
  translation, on random multi-row calls with random hot, source and resident
  tables, null blocks, padding and invalidations in between.
* Reduction: with a one-row-per-block hot table that reproduces the flat
  layout and a source table that reproduces a pool-row table, paged keying
  gives the position-keyed swap-in's outputs, LRU and hot buffer, and its
  slot keys are the pool rows of the position-keyed slots' tokens.
* Invalidation against a numpy mask.
"""

import json
import os

import numpy as np
import pytest

import oracle
from model import lru_model_swap_in
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _paged_dict(fx_paged, B, K):
    d = {k: (np.asarray(v, np.int32) if k.endswith("table") else v) for k, v in fx_paged.items()}
    d["attention_indices"] = np.full((B, K), 7777, np.int32)
    return d


def test_paged_worked_example():
    fx = json.load(open(os.path.join(GOLDEN, "swap_in_paged_worked_example.json")))
    H, S_r, R, K, rb = fx["H"], fx["S_r"], fx["R"], fx["K"], fx["row_bytes"]
    pool = np.array([[(p + j) % 256 for j in range(rb)] for p in range(fx["pool_nrows"])], np.uint8)
    hot = np.zeros((fx["hot_nrows"], rb), np.uint8)
    keys = np.full((R, S_r), -1, np.int32)
    lru = np.tile(np.arange(H, dtype=np.int16), (R, 1))
    for step in fx["steps"]:
        e = step["expect"]
        if "invalidate" in step:
            inv = step["invalidate"]
            n = oracle.invalidate_written(keys, np.asarray(inv["rows"], np.int64),
                                          np.asarray(inv["written"], np.int64))
            assert n == e["cleared"]
        else:
            c = step["call"]
            B = len(c["req_rows"])
            pg = _paged_dict(fx["paged"], B, K)
            out, cnt = oracle.swap_in(topk=np.asarray(c["topk"], np.int32),
                                      req_rows=np.asarray(c["req_rows"], np.int64), seq_lens=None,
                                      slot_tokens=keys, lru=lru, pool=pool, hot=hot, ctx_stride=0,
                                      num_real=c["num_real"], paged=pg)
            assert out.tolist() == e["out"]
            assert cnt.tolist() == e["miss_counts"]
            assert pg["attention_indices"].tolist() == e["attention"]
            want = np.zeros_like(hot)
            for row, p in e["hot_from_pool"].items():
                want[int(row)] = pool[p]
            assert np.array_equal(hot, want)
        assert keys.tolist() == e["slot_tokens"]
        assert lru.tolist() == e["lru"]


def _random_tables(rng, R, H, ctx, hb=None):
    hb = int(rng.choice([1, 2, 4, 8])) if hb is None else hb
    nhb = -(-H // hb)
    extra = 3
    hot_blocks = rng.permutation(R * nhb + extra)[:R * nhb].reshape(R, nhb).astype(np.int32)
    hot_nrows = (R * nhb + extra) * hb
    sb = int(rng.choice([4, 16]))
    nsb = -(-ctx // sb) + 1
    phys = rng.permutation(np.arange(1, R * nsb + 4))[:R * nsb].reshape(R, nsb).astype(np.int32)
    nulls = rng.random((R, nsb)) < 0.1
    phys[nulls] = rng.choice([0, -1], size=int(nulls.sum()))
    pool_nrows = (R * nsb + 4) * sb - sb // 2           # the last block is cut: some ids have no row
    # Resident table inside the vLLM page's domain (its host checks): block
    # size equal to the hot block size and a non-negative null block. Most
    # blocks hold the null block, some a negative block, some a real one;
    # the null block is drawn so that it is often 0 and sometimes a block id
    # that real entries could also hold.
    rbs = hb
    nrb = -(-ctx // rbs)
    null = int(rng.choice([0, 0, 3, 17]))
    res = np.full((R, nrb), null, np.int32)
    neg = rng.random((R, nrb)) < 0.1
    res[neg] = -1
    hit = rng.random((R, nrb)) < 0.15
    res[hit] = rng.integers(0, 50, int(hit.sum()))
    paged = {"hot_block_table": hot_blocks, "hot_block_size": hb, "src_block_table": phys,
             "src_block_size": sb, "resident_block_table": res, "resident_block_size": rbs,
             "resident_null_block": null}
    return paged, hot_nrows, pool_nrows


@pytest.mark.parametrize("seed", range(6))
def test_paged_matches_model(seed):
    rng = np.random.default_rng(1000 + seed)
    R, B, H, K, ctx, rb = 5, 3, 16, 8, 120, 4
    S_r = H + 1
    paged, hot_nrows, pool_nrows = _random_tables(rng, R, H, ctx)
    if seed % 2:
        paged = {k: v for k, v in paged.items() if not k.startswith("resident")}
    pool = rng.integers(0, 256, (pool_nrows, rb), dtype=np.uint8)
    st_o, lru_o = gen.initial_state(R, H, S_r)
    st_m, lru_m = st_o.copy(), lru_o.copy()
    hot_o = np.zeros((hot_nrows, rb), np.uint8)
    hot_m = hot_o.copy()
    for call in range(14):
        if call % 5 == 4:
            # invalidate a few global rows that some slots hold
            rows = rng.integers(-1, R + 1, 6).astype(np.int64)
            written = np.array([st_o[r % R, rng.integers(0, H)] for r in rows], np.int64)
            n_o = oracle.invalidate_written(st_o, rows, written)
            for r, g in zip(rows, written):
                if 0 <= r < R and g >= 0:
                    st_m[r][st_m[r] == g] = -1
            assert np.array_equal(st_o, st_m) and n_o >= 0
            continue
        req = rng.permutation(R)[:B].astype(np.int64)
        topk = np.stack([rng.permutation(np.arange(-3, ctx + 5))[:K] for _ in range(B)]).astype(np.int32)
        nreal = int(rng.integers(1, B + 1)) if rng.random() < 0.3 else -1
        kw = dict(topk=topk, req_rows=req, seq_lens=None, pool=pool, ctx_stride=0, num_real=nreal,
                  paged=paged)
        stats = np.zeros(2, np.uint64)
        out_o, cnt_o, plan_o = oracle.swap_in(slot_tokens=st_o, lru=lru_o, hot=hot_o, plan=True,
                                              stats=stats, **kw)
        out_m, cnt_m, plan_m = lru_model_swap_in(slot_tokens=st_m, lru=lru_m, hot=hot_m, plan=True, **kw)
        assert int(stats[1]) == int(cnt_m.sum())   # misses, from the model's counts
        assert out_o.tolist() == out_m.tolist(), call
        assert cnt_o.tolist() == cnt_m.tolist()
        assert st_o.tolist() == st_m.tolist()
        assert lru_o.tolist() == lru_m.tolist()
        assert np.array_equal(hot_o, hot_m)
        assert plan_o["miss_mask"].tolist() == plan_m["miss_mask"].tolist()
        for b, cp in enumerate(plan_m["copies"]):
            n = len(cp)
            assert list(zip(plan_o["src"][b, :n].tolist(), plan_o["dst"][b, :n].tolist())) == cp


@pytest.mark.parametrize("seed", range(3))
def test_paged_reduces_to_position_keying(seed):
    rng = np.random.default_rng(2000 + seed)
    R, B, H, K, ctx, rb = 4, 3, 24, 10, 200, 8
    S_r = H + 1
    # hot table with one row per block: Row(r, s) = r * S_r + s, the flat layout
    hot_table = np.array([[r * S_r + s for s in range(H)] for r in range(R)], np.int32)
    # source table with one block per request: g = (r + 1) * ctx + t
    src_table = np.array([[r + 1] for r in range(R)], np.int32)
    pool_rows = np.array([[(r + 1) * ctx + t for t in range(ctx)] for r in range(R)], np.int64)
    paged = {"hot_block_table": hot_table, "hot_block_size": 1, "src_block_table": src_table,
             "src_block_size": ctx}
    pool = rng.integers(0, 256, ((R + 1) * ctx, rb), dtype=np.uint8)
    st_p, lru_p = gen.initial_state(R, H, S_r)
    st_q, lru_q = st_p.copy(), lru_p.copy()
    hot_p = np.zeros((R * S_r, rb), np.uint8)
    hot_q = hot_p.copy()
    for _ in range(10):
        req = rng.permutation(R)[:B].astype(np.int64)
        # positions below ctx - 1: no newest-token binding on the position side
        topk = np.stack([rng.permutation(ctx - 1)[:K] for _ in range(B)]).astype(np.int32)
        out_p, cnt_p = oracle.swap_in(topk=topk, req_rows=req, seq_lens=None, slot_tokens=st_p,
                                      lru=lru_p, pool=pool, hot=hot_p, ctx_stride=0, paged=paged)
        out_q, cnt_q = oracle.swap_in(topk=topk, req_rows=req, seq_lens=np.full(B, ctx, np.int64),
                                      slot_tokens=st_q, lru=lru_q, pool=pool, hot=hot_q,
                                      ctx_stride=ctx, pool_rows=pool_rows)
        assert out_p.tolist() == out_q.tolist()
        assert cnt_p.tolist() == cnt_q.tolist()
        assert lru_p.tolist() == lru_q.tolist()
        assert np.array_equal(hot_p, hot_q)
        keys_from_q = np.where(st_q[:, :H] >= 0,
                               np.take_along_axis(pool_rows, np.maximum(st_q[:, :H], 0).astype(np.int64), 1),
                               -1)
        assert st_p[:, :H].tolist() == keys_from_q.tolist()


@pytest.mark.parametrize("change", ["no_source_table", "block_sizes_differ", "negative_null"])
def test_paged_rejects_resident_tables_the_page_rejects(change):
    """vLLM hisparse_kernels.cu, host checks of hisparse_resolve_residency: a
    resident lookup needs the source block table, the resident and hot block
    sizes must match, and the resident null block must be non-negative."""
    R, H, K, ctx, rb = 2, 4, 2, 16, 4
    hb = 2
    paged = {"hot_block_table": np.array([[0, 1], [2, 3]], np.int32), "hot_block_size": hb,
             "src_block_table": np.array([[1, 2, 3, 4], [5, 6, 7, 8]], np.int32),
             "src_block_size": 4,
             "resident_block_table": np.zeros((2, ctx // hb), np.int32),
             "resident_block_size": hb, "resident_null_block": 0}
    st, lru = gen.initial_state(R, H, H + 1)
    kw = dict(topk=np.array([[1, 2], [3, 4]], np.int32), req_rows=np.arange(2, dtype=np.int64),
              seq_lens=None, slot_tokens=st, lru=lru, pool=np.zeros((40, rb), np.uint8),
              hot=np.zeros((8, rb), np.uint8), ctx_stride=0)
    oracle.swap_in(**kw, paged=paged)              # inside the page's domain: accepted
    if change == "no_source_table":
        paged = {k: v for k, v in paged.items() if not k.startswith("src")}
    elif change == "block_sizes_differ":
        paged = dict(paged, resident_block_size=4, resident_block_table=np.zeros((2, 4), np.int32))
    else:
        paged = dict(paged, resident_null_block=-1)
    with pytest.raises(oracle.OracleError) as e:
        oracle.swap_in(**kw, paged=paged)
    assert e.value.code == -1


def _run_calls(paged, R, H, K, ctx, rb, pool_nrows, hot_nrows, seed, calls=4):
    rng = np.random.default_rng(seed)
    st, lru = gen.initial_state(R, H, H + 1)
    pool = rng.integers(0, 256, (pool_nrows, rb), dtype=np.uint8)
    hot = np.zeros((hot_nrows, rb), np.uint8)
    seen = []
    for _ in range(calls):
        topk = np.stack([rng.permutation(np.arange(-2, ctx + 2))[:K] for _ in range(R)]).astype(np.int32)
        att = np.zeros((R, K), np.int32)
        out, cnt = oracle.swap_in(topk=topk, req_rows=np.arange(R, dtype=np.int64), seq_lens=None,
                                  slot_tokens=st, lru=lru, pool=pool, hot=hot, ctx_stride=0,
                                  paged=dict(paged, attention_indices=att, attention_block_stride=9))
        seen.append((topk, out.copy(), cnt.copy(), att, st.copy(), lru.copy(), hot.copy()))
    return seen


def test_resident_row_past_int32_is_not_resident():
    """A resident row that no int32 output can hold counts as no resident row:
    every call gives exactly what it gives with the null block in those table
    entries. A row of exactly INT32_MAX (one-row blocks) is still served."""
    R, H, K, ctx, rb = 3, 16, 8, 120, 4
    rng = np.random.default_rng(31)
    paged, hot_nrows, pool_nrows = _random_tables(rng, R, H, ctx, hb=2)
    res = paged["resident_block_table"]
    huge = np.zeros_like(res, dtype=bool)
    huge[:, ::3] = True                                  # every third block of each row
    big = dict(paged, resident_block_table=np.where(huge, np.int32(2**30), res))   # rows >= 2^31
    null = dict(paged, resident_block_table=np.where(huge, np.int32(paged["resident_null_block"]), res))
    a = _run_calls(big, R, H, K, ctx, rb, pool_nrows, hot_nrows, seed=3)
    b = _run_calls(null, R, H, K, ctx, rb, pool_nrows, hot_nrows, seed=3)
    hit_huge = 0
    for x, y in zip(a, b):
        for u, v in zip(x[1:], y[1:]):
            assert np.array_equal(u, v)
        t = x[0]
        hit_huge += int(sum(huge[r, t[r][(t[r] >= 0) & (t[r] < ctx)] // 2].sum() for r in range(R)))
    assert hit_huge > 0                                  # the calls did name those blocks

    # One-row blocks: block INT32_MAX is row INT32_MAX, an int32 output.
    paged1, hot_nrows1, pool_nrows1 = _random_tables(np.random.default_rng(32), R, H, ctx, hb=1)
    tab = paged1["resident_block_table"].copy()
    tab[0, 5] = 2**31 - 1
    st, lru = gen.initial_state(R, H, H + 1)
    topk = np.tile(np.arange(5, 5 + K, dtype=np.int32), (R, 1))
    out, _ = oracle.swap_in(topk=topk, req_rows=np.arange(R, dtype=np.int64), seq_lens=None,
                            slot_tokens=st, lru=lru, pool=np.zeros((pool_nrows1, rb), np.uint8),
                            hot=np.zeros((hot_nrows1, rb), np.uint8), ctx_stride=0,
                            paged=dict(paged1, resident_block_table=tab))
    assert out[0, 0] == 2**31 - 1


def test_invalidate_matches_numpy():
    rng = np.random.default_rng(7)
    R, S_r, n = 6, 20, 40
    keys = rng.integers(-1, 30, (R, S_r)).astype(np.int32)
    rows = rng.integers(-2, R + 2, n).astype(np.int64)
    written = rng.integers(-3, 30, n).astype(np.int64)
    want = keys.copy()
    cleared = 0
    for r, g in zip(rows, written):
        if 0 <= r < R and g >= 0:
            m = want[r] == g
            cleared += int(m.sum())
            want[r][m] = -1
    assert oracle.invalidate_written(keys, rows, written) == cleared
    assert np.array_equal(keys, want)
