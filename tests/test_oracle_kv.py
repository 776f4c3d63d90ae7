"""Pin the oracle's non-MLA (K+V) variants.

* ``tests/golden/kv_copies_worked_example.json``: the K+V all-layer transfer and
  the K+V scatter derived by hand (tokenspeed kvcache/triton.py,
  _kv_transfer_all_layer_kernel and _store_kv_cache_kernel).
* The swap-in with a V pool: on the hand-derived swap-in examples every V hot
  row must hold the V pool row that the fixture says its K row came from
  (SGLang hisparse.cuh, the !IsMLA branch of the miss copy), and the K side
  must be unchanged by the presence of V.
* The OrderedDict model copies V rows too (``tests/test_oracle_model.py``).
* numpy fancy indexing for both K+V copies on random inputs.
"""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _strided(rows, rb, stride, fill):
    back = np.zeros(rows * stride, np.uint8)
    view = np.lib.stride_tricks.as_strided(back, shape=(rows, rb), strides=(stride, 1))
    for j, v in enumerate(fill):
        view[j] = v
    return back, view


def test_kv_copies_worked_example():
    fx = json.load(open(os.path.join(GOLDEN, "kv_copies_worked_example.json")))
    t = fx["transfer"]
    L, rows, rb = t["layers"], t["rows"], t["row_bytes"]
    ks = [np.array([[10 * l + p] * rb for p in range(rows)], np.uint8) for l in range(L)]
    vs = [np.array([[50 + 10 * l + p] * rb for p in range(rows)], np.uint8) for l in range(L)]
    kd = [np.full((rows, rb), 238, np.uint8) for _ in range(L)]
    vd = [np.full((rows, rb), 238, np.uint8) for _ in range(L)]
    skipped = oracle.transfer_kv_all_layer(ks, vs, kd, vd, np.asarray(t["src_idx"], np.int64),
                                           np.asarray(t["dst_idx"], np.int64))
    assert skipped == t["expect_skipped"]
    assert [x.tolist() for x in kd] == t["expect_k"]
    assert [x.tolist() for x in vd] == t["expect_v"]

    c = fx["scatter"]
    n, rb = c["n"], c["row_bytes"]
    _, ksrc = _strided(n, rb, c["k_src_stride"], [[j + 1] * rb for j in range(n)])
    _, vsrc = _strided(n, rb, c["v_src_stride"], [[j + 21] * rb for j in range(n)])
    _, kdst = _strided(c["dst_rows"], rb, c["k_dst_stride"], [])
    _, vdst = _strided(c["dst_rows"], rb, c["v_dst_stride"], [])
    skipped = oracle.store_kv_cache(ksrc, vsrc, kdst, vdst, np.asarray(c["loc"], np.int64))
    assert skipped == c["expect_skipped"]
    assert kdst.tolist() == c["expect_k"]
    assert vdst.tolist() == c["expect_v"]


@pytest.mark.parametrize("name", ["swap_in_worked_example_1.json", "swap_in_worked_example_2.json"])
def test_swap_in_v_rows_follow_k_rows(name):
    fx = json.load(open(os.path.join(GOLDEN, name)))
    H, S_r, R, rb = fx["H"], fx["S_r"], fx["R"], fx["row_bytes"]
    n = fx["pool_nrows"]
    pool = np.array([[(p + j) % 256 for j in range(rb)] for p in range(n)], np.uint8)
    pool_v = np.array([[(p + j + 100) % 256 for j in range(rb)] for p in range(n)], np.uint8)
    hot_nrows = fx.get("hot_nrows", R * S_r)
    hot = np.zeros((hot_nrows, rb), np.uint8)
    hot_v = np.zeros_like(hot)
    hot_k_only = np.zeros_like(hot)
    tokens = np.full((R, S_r), -1, np.int32)
    lru = np.tile(np.arange(H, dtype=np.int16), (R, 1))
    tokens2, lru2 = tokens.copy(), lru.copy()
    slot_rows = np.asarray(fx["slot_rows"], np.int32) if "slot_rows" in fx else None
    pool_rows = np.asarray(fx["pool_rows"], np.int64) if "pool_rows" in fx else None
    for call in fx["calls"]:
        kw = dict(topk=np.asarray(call["topk"], np.int32), req_rows=np.asarray(call["req_rows"], np.int64),
                  seq_lens=np.asarray(call["seq_lens"], np.int64), pool=pool, ctx_stride=fx["ctx_stride"],
                  num_real=call["num_real"], slot_rows=slot_rows, pool_rows=pool_rows)
        out, cnt = oracle.swap_in(slot_tokens=tokens, lru=lru, hot=hot, pool_v=pool_v, hot_v=hot_v, **kw)
        out2, cnt2 = oracle.swap_in(slot_tokens=tokens2, lru=lru2, hot=hot_k_only, **kw)
        assert out.tolist() == out2.tolist() == call["expect"]["out"]
        assert cnt.tolist() == cnt2.tolist()
        assert np.array_equal(hot, hot_k_only)
        want_v = np.zeros_like(hot_v)
        for row, p in call["expect"]["hot_from_pool"].items():
            want_v[int(row)] = pool_v[p]
        assert np.array_equal(hot_v, want_v)


@pytest.mark.parametrize("seed", range(4))
def test_kv_copies_match_numpy(seed):
    rng = np.random.default_rng(seed)
    L, S, D, rb, n = 3, 40, 30, 12, 25
    ks = [rng.integers(0, 256, (S, rb), dtype=np.uint8) for _ in range(L)]
    vs = [rng.integers(0, 256, (S, rb), dtype=np.uint8) for _ in range(L)]
    kd = [rng.integers(0, 256, (D, rb), dtype=np.uint8) for _ in range(L)]
    vd = [rng.integers(0, 256, (D, rb), dtype=np.uint8) for _ in range(L)]
    si = rng.integers(-2, S + 3, n).astype(np.int64)
    di = (rng.permutation(D + 4)[:n] - 2).astype(np.int64)
    wk, wv = [x.copy() for x in kd], [x.copy() for x in vd]
    ok = (si >= 0) & (si < S) & (di >= 0) & (di < D)
    for l in range(L):
        wk[l][di[ok]] = ks[l][si[ok]]
        wv[l][di[ok]] = vs[l][si[ok]]
    assert oracle.transfer_kv_all_layer(ks, vs, kd, vd, si, di) == int((~ok).sum())
    for l in range(L):
        assert np.array_equal(kd[l], wk[l]) and np.array_equal(vd[l], wv[l])

    m = 17
    ksrc = rng.integers(0, 256, (m, rb + 4), dtype=np.uint8)[:, :rb]
    vsrc = rng.integers(0, 256, (m, rb + 8), dtype=np.uint8)[:, :rb]
    kdst = rng.integers(0, 256, (D, rb), dtype=np.uint8)
    vdst = rng.integers(0, 256, (D, rb + 4), dtype=np.uint8)[:, :rb]
    vdst_back = vdst.base
    loc = (rng.permutation(D + 6)[:m] - 3).astype(np.int64)
    good = (loc >= 0) & (loc < D)
    wk, wv = kdst.copy(), vdst.copy()
    wk[loc[good]] = ksrc[good]
    wv[loc[good]] = vsrc[good]
    assert oracle.store_kv_cache(ksrc, vsrc, kdst, vdst, loc) == int((~good).sum())
    assert np.array_equal(kdst, wk) and np.array_equal(vdst, wv)
    assert vdst_back is not None
