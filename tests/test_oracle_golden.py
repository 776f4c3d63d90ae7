"""Pin the oracle to hand-derived worked examples (tests/golden/*.json).

The pages print no worked example, so each fixture was derived by hand from the
rules the pages' kernels implement; the fixture's ``citation`` and
``derivation`` fields say which rule gives each expected value.
"""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pool(n, rb):
    return np.array([[(p + j) % 256 for j in range(rb)] for p in range(n)], dtype=np.uint8)


@pytest.mark.parametrize("name", ["swap_in_worked_example_1.json", "swap_in_worked_example_2.json"])
def test_swap_in_worked_examples(name):
    fx = json.load(open(os.path.join(GOLDEN, name)))
    H, S_r, R, rb = fx["H"], fx["S_r"], fx["R"], fx["row_bytes"]
    pool = _pool(fx["pool_nrows"], rb)
    hot_nrows = fx.get("hot_nrows", R * S_r)
    hot = np.zeros((hot_nrows, rb), dtype=np.uint8)
    tokens = np.full((R, S_r), -1, dtype=np.int32)
    lru = np.tile(np.arange(H, dtype=np.int16), (R, 1))
    slot_rows = np.asarray(fx["slot_rows"], dtype=np.int32) if "slot_rows" in fx else None
    pool_rows = np.asarray(fx["pool_rows"], dtype=np.int64) if "pool_rows" in fx else None
    for call in fx["calls"]:
        out, counts, plan = oracle.swap_in(
            topk=np.asarray(call["topk"], dtype=np.int32),
            req_rows=np.asarray(call["req_rows"], dtype=np.int64),
            seq_lens=np.asarray(call["seq_lens"], dtype=np.int64),
            slot_tokens=tokens, lru=lru, pool=pool, hot=hot, ctx_stride=fx["ctx_stride"],
            num_real=call["num_real"], slot_rows=slot_rows, pool_rows=pool_rows, plan=True)
        e = call["expect"]
        assert out.tolist() == e["out"]
        assert counts.tolist() == e["miss_counts"]
        assert plan["miss_mask"].tolist() == e["miss_mask"]
        assert plan["count"].tolist() == e["miss_counts"]
        for b, lst in enumerate(e["miss_list"]):
            n = len(lst)
            got = list(zip(plan["src"][b, :n].tolist(), plan["dst"][b, :n].tolist()))
            assert got == [tuple(x) for x in lst], (b, got, lst)
        assert tokens.tolist() == e["slot_tokens"]
        assert lru.tolist() == e["lru"]
        want = np.zeros_like(hot)
        for row, p in e["hot_from_pool"].items():
            want[int(row)] = pool[p]
        assert np.array_equal(hot, want)


def test_copies_worked_example():
    fx = json.load(open(os.path.join(GOLDEN, "copies_worked_example.json")))
    t = fx["transfer"]
    src = [np.full((t["rows"], t["row_bytes"]), 0, dtype=np.uint8) for _ in range(t["layers"])]
    for l in range(t["layers"]):
        for p in range(t["rows"]):
            src[l][p] = 10 * l + p
    dst = [np.full((t["rows"], t["row_bytes"]), 0xEE, dtype=np.uint8) for _ in range(t["layers"])]
    skipped = oracle.transfer_rows_all_layer(src, dst, np.asarray(t["src_idx"], dtype=np.int64),
                                             np.asarray(t["dst_idx"], dtype=np.int64))
    assert skipped == 0
    assert [d.tolist() for d in dst] == t["expect_dst"]

    s = fx["scatter"]
    backing = np.zeros((s["n"], s["src_row_stride"]), dtype=np.uint8)
    for j in range(s["n"]):
        backing[j, :s["row_bytes"]] = j + 1
        backing[j, s["row_bytes"]:] = 0x77        # bytes past the row must not move
    src_view = backing[:, :s["row_bytes"]]
    dst = np.zeros((s["dst_rows"], s["row_bytes"]), dtype=np.uint8)
    skipped = oracle.store_kv_scatter(src_view, dst, np.asarray(s["loc"], dtype=np.int64))
    assert skipped == 1
    assert dst.tolist() == s["expect_dst"]
