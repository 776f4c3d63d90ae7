"""Pin the oracle's row copies to numpy fancy indexing, and check that it
rejects inputs that break the pages' stated preconditions."""

import numpy as np
import pytest

import oracle
from workloads import gen


@pytest.mark.parametrize("L,rows,rb,n", [(1, 10, 4, 3), (3, 50, 656, 20), (5, 64, 132, 64)])
def test_transfer_matches_numpy(L, rows, rb, n):
    rng = np.random.default_rng(L * 100 + n)
    src = [rng.integers(0, 256, size=(rows, rb), dtype=np.uint8) for _ in range(L)]
    dst = [rng.integers(0, 256, size=(rows, rb), dtype=np.uint8) for _ in range(L)]
    si = rng.permutation(rows)[:n].astype(np.int64)
    di = rng.permutation(rows)[:n].astype(np.int64)
    want = [d.copy() for d in dst]
    for l in range(L):
        want[l][di] = src[l][si]
    assert oracle.transfer_rows_all_layer(src, dst, si, di) == 0
    for l in range(L):
        assert np.array_equal(dst[l], want[l])


def test_transfer_skips_out_of_range_pairs():
    src = [np.arange(40, dtype=np.uint8).reshape(10, 4)]
    dst = [np.zeros((6, 4), dtype=np.uint8)]
    si = np.asarray([1, 10, -1, 2], dtype=np.int64)
    di = np.asarray([0, 1, 2, 6], dtype=np.int64)
    assert oracle.transfer_rows_all_layer(src, dst, si, di) == 3
    want = np.zeros((6, 4), dtype=np.uint8)
    want[0] = src[0][1]
    assert np.array_equal(dst[0], want)


@pytest.mark.parametrize("n,rb,stride", [(1, 4, 4), (17, 656, 700), (33, 132, 132)])
def test_scatter_matches_numpy(n, rb, stride):
    rng = np.random.default_rng(n)
    backing = rng.integers(0, 256, size=(n, stride), dtype=np.uint8)
    src = backing[:, :rb]
    dst = rng.integers(0, 256, size=(3 * n, rb), dtype=np.uint8)
    loc = rng.permutation(3 * n)[:n].astype(np.int64)
    want = dst.copy()
    want[loc] = src
    assert oracle.store_kv_scatter(src, dst, loc) == 0
    assert np.array_equal(dst, want)


def test_state_reset():
    st = np.full((4, 6), 7, dtype=np.int32)
    lru = np.full((4, 5), 3, dtype=np.int16)
    oracle.state_reset(st, lru, [1, 3])
    assert st[1].tolist() == [-1] * 6 and st[3].tolist() == [-1] * 6
    assert st[0].tolist() == [7] * 6 and lru[2].tolist() == [3] * 5
    assert lru[1].tolist() == list(range(5)) and lru[3].tolist() == list(range(5))


def _base():
    R, H, K, ctx, rb = 2, 4, 2, 10, 4
    st, lru = gen.initial_state(R, H, H + 1)
    pool = np.zeros((R * ctx, rb), dtype=np.uint8)
    hot = np.zeros((R * (H + 1), rb), dtype=np.uint8)
    kw = dict(topk=np.asarray([[1, 2], [3, 4]], dtype=np.int32),
              req_rows=np.asarray([0, 1], dtype=np.int64),
              seq_lens=np.asarray([10, 10], dtype=np.int64), slot_tokens=st, lru=lru, pool=pool,
              hot=hot, ctx_stride=ctx)
    return kw


def test_rejects_duplicate_ids():
    kw = _base()
    kw["topk"] = np.asarray([[2, 2], [3, 4]], dtype=np.int32)
    with pytest.raises(oracle.OracleError) as e:
        oracle.swap_in(**kw)
    assert e.value.code == -2


def test_duplicate_invalid_or_newest_ids_are_fine():
    kw = _base()
    kw["topk"] = np.asarray([[9, 9], [-1, -1]], dtype=np.int32)
    out, cnt = oracle.swap_in(**kw)
    assert out.tolist() == [[4, 4], [-1, -1]] and cnt.tolist() == [0, 0]


def test_rejects_non_permutation_lru():
    kw = _base()
    kw["lru"][1] = np.asarray([0, 1, 1, 3], dtype=np.int16)
    with pytest.raises(oracle.OracleError) as e:
        oracle.swap_in(**kw)
    assert e.value.code == -3


def test_rejects_shared_state_row_among_real_rows():
    kw = _base()
    kw["req_rows"] = np.asarray([1, 1], dtype=np.int64)
    with pytest.raises(oracle.OracleError) as e:
        oracle.swap_in(**kw)
    assert e.value.code == -4
    # ... unless the second one is padding
    out, cnt = oracle.swap_in(**kw, num_real=1)
    assert out[1].tolist() == [-1, -1] and cnt[1] == 0


def test_rejects_duplicate_resident_token():
    kw = _base()
    kw["slot_tokens"][0, :2] = 1
    with pytest.raises(oracle.OracleError) as e:
        oracle.swap_in(**kw)
    assert e.value.code == -6


def test_rejects_hot_row_outside_buffer():
    kw = _base()
    kw["hot"] = kw["hot"][:6]
    with pytest.raises(oracle.OracleError) as e:
        oracle.swap_in(**kw)
    assert e.value.code == -5


def test_rejects_top_k_above_hot_size():
    kw = _base()
    kw["topk"] = np.zeros((2, 5), dtype=np.int32)
    with pytest.raises(oracle.OracleError) as e:
        oracle.swap_in(**kw)
    assert e.value.code == -1


def test_state_row_out_of_range_is_padding():
    kw = _base()
    kw["req_rows"] = np.asarray([0, 5], dtype=np.int64)
    out, cnt = oracle.swap_in(**kw)
    assert out[1].tolist() == [-1, -1] and cnt[1] == 0 and cnt[0] == 2


def test_state_row_past_R_is_padding_with_otherwise_valid_ids():
    """req_rows names state row R (one past the last). The pool and the hot
    buffer have rows for it and the state arrays are views of arrays with a
    spare row, so its ids would be valid and its slots addressable: only the
    state-row bound makes the row padding. The spare row and the hot rows
    past R*S_r stay untouched."""
    R, H, K, ctx, rb = 2, 4, 2, 10, 4
    S_r = H + 1
    st_big, lru_big = gen.initial_state(R + 1, H, S_r)
    pool = np.arange((R + 1) * ctx * rb, dtype=np.uint32).astype(np.uint8).reshape((R + 1) * ctx, rb)
    hot = np.zeros(((R + 1) * S_r, rb), dtype=np.uint8)
    out, cnt = oracle.swap_in(topk=np.asarray([[1, 2], [3, 4]], dtype=np.int32),
                              req_rows=np.asarray([0, R], dtype=np.int64),
                              seq_lens=np.asarray([10, 10], dtype=np.int64),
                              slot_tokens=st_big[:R], lru=lru_big[:R], pool=pool, hot=hot,
                              ctx_stride=ctx)
    assert out[1].tolist() == [-1, -1] and cnt.tolist() == [2, 0]
    assert out[0].tolist() == [0, 1]
    assert st_big[R].tolist() == [-1] * S_r and lru_big[R].tolist() == list(range(H))
    assert not hot[R * S_r:].any()


def test_ids_past_ctx_stride_or_pool_are_invalid():
    kw = _base()
    kw["seq_lens"] = np.asarray([30, 10], dtype=np.int64)
    kw["topk"] = np.asarray([[12, 3], [3, 4]], dtype=np.int32)   # 12 >= ctx_stride 10
    out, cnt = oracle.swap_in(**kw)
    assert out[0, 0] == -1 and cnt[0] == 1
    kw2 = _base()
    kw2["pool"] = kw2["pool"][:13]                                # row 1's ids 3,4 -> pool 13,14
    out, cnt = oracle.swap_in(**kw2)
    assert out[1].tolist() == [-1, -1] and cnt[1] == 0
