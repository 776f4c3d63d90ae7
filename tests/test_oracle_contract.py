"""Pin the oracle's entry conditions and its edge rules, one case per rule.

Each entry point rejects what it must (negative sizes, missing buffers,
geometry the pages rule out) with its error code and accepts the boundary
just inside; empty calls write nothing; the state checks look at every real
row (row 0 and the first LRU position included) and at no padding row; and a
few results at the edges of the rules: an id equal to the row stride, paged
global id 0, a resident block 0 that is not the null block, attention rows
wider than top-k. The swap-in is called through its C struct so that each
argument can be set on its own."""

import ctypes

import numpy as np
import pytest

import oracle
from workloads import gen

EARG, EDUP, ELRU, EROWS, EHOT = -1, -2, -3, -4, -5


def _p(a):
    return None if a is None else a.ctypes.data


class Call:
    """A valid flat swap-in (R 2, H 4, K 2, 10-token contexts) whose struct
    fields can be changed one at a time before the call."""

    def __init__(self, paged=None):
        R, H, K, ctx, rb = 2, 4, 2, 10, 4
        self.st, self.lru = gen.initial_state(R, H, H + 1)
        self.pool = np.arange(R * ctx * rb, dtype=np.uint8).reshape(R * ctx, rb)
        self.hot = np.zeros((R * (H + 1), rb), np.uint8)
        self.topk = np.asarray([[1, 2], [3, 4]], np.int32)
        self.rows = np.asarray([0, 1], np.int64)
        self.seq = np.asarray([ctx, ctx], np.int64)
        self.out = np.full((2, K), 7777, np.int32)
        self.cnt = np.full(2, 7777, np.int32)
        self.keep = []
        self.a = oracle._SwapArgs(
            B=2, K=K, H=H, S_r=H + 1, R=R, topk=_p(self.topk), topk_stride=K,
            req_rows=_p(self.rows), seq_lens=_p(self.seq), num_real=-1,
            slot_tokens=_p(self.st), lru=_p(self.lru), slot_rows=None, pool_rows=None,
            ctx_stride=ctx, pool=_p(self.pool), pool_nrows=R * ctx, hot=_p(self.hot),
            hot_nrows=R * (H + 1), row_bytes=rb, out_rows=_p(self.out), miss_counts=_p(self.cnt),
            miss_mask=None, list_count=None, list_src=None, list_dst=None, pool_v=None,
            hot_v=None, paged=None, stats=None)
        if paged is not None:
            self.set_paged(**paged)

    def set_paged(self, **kw):
        hbt = np.asarray([[0, 1], [2, 3]], np.int32)          # hot blocks of 2 slots
        self.keep.append(hbt)
        self.pg = oracle._Paged(hot_block_table=_p(hbt), hot_table_stride=2, hot_block_size=2,
                                src_block_table=None, src_table_stride=0, src_num_blocks=0,
                                src_block_size=1, resident_block_table=None,
                                resident_table_stride=0, resident_num_blocks=0,
                                resident_block_size=1, resident_null_block=0,
                                attention_indices=None, attention_row_stride=0,
                                attention_block_stride=0)
        for k, v in kw.items():
            if isinstance(v, np.ndarray):
                self.keep.append(v)
                v = _p(v)
            setattr(self.pg, k, v)
        self.a.paged = ctypes.pointer(self.pg)
        self.a.hot_nrows = 8

    def __call__(self, **kw):
        for k, v in kw.items():
            if isinstance(v, np.ndarray):
                self.keep.append(v)
                v = _p(v)
            setattr(self.a, k, v)
        return oracle._load().oracle_swap_in(ctypes.byref(self.a))


def test_the_base_call_is_valid():
    c = Call()
    assert c() == 0
    assert c.out.tolist() == [[0, 1], [5, 6]] and c.cnt.tolist() == [2, 2]   # the oldest slots


@pytest.mark.parametrize("field,value", [
    ("B", -1), ("K", -1), ("H", -1), ("R", -1),
    ("topk", None), ("req_rows", None), ("seq_lens", None), ("slot_tokens", None), ("lru", None),
    ("pool", None), ("hot", None), ("out_rows", None),
    ("H", 1),                      # H < K
    ("S_r", 4),                    # no newest slot after the H LRU slots
    ("topk_stride", 1),            # rows overlap
    ("row_bytes", 0), ("ctx_stride", 0),
])
def test_swap_in_rejects_each_bad_argument(field, value):
    c = Call()
    assert c(**{field: value}) == EARG
    assert c.out.tolist() == [[7777] * 2] * 2 and c.cnt.tolist() == [7777] * 2


def test_swap_in_accepts_the_boundaries():
    assert Call()(H=2, S_r=5, lru=np.tile(np.arange(2, dtype=np.int16), (2, 1))) == 0   # H == K
    assert Call()(row_bytes=1, ctx_stride=1, seq_lens=np.asarray([1, 1], np.int64)) == 0
    c = Call()
    assert c(topk_stride=3, topk=np.asarray([[1, 2, 0], [3, 4, 0]], np.int32)) == 0
    assert c.out.tolist() == [[0, 1], [5, 6]]


@pytest.mark.parametrize("field", ["B", "K"])
def test_empty_swap_in_writes_nothing(field):
    c = Call()
    assert c(**{field: 0}) == 0
    assert c.out.tolist() == [[7777] * 2] * 2 and c.cnt.tolist() == [7777] * 2
    assert c.lru.tolist() == [[0, 1, 2, 3]] * 2 and (c.st == -1).all()


def test_empty_swap_in_reads_nothing():
    assert Call()(B=0, topk=None, req_rows=None, seq_lens=None, out_rows=None) == 0
    assert Call()(K=0, H=0, S_r=1, topk=None, pool=None, hot=None) == 0


def test_no_state_rows_makes_every_row_padding():
    c = Call()
    assert c(R=0) == 0
    assert c.out.tolist() == [[-1, -1], [-1, -1]] and c.cnt.tolist() == [0, 0]


@pytest.mark.parametrize("broken", ["lru", "rows", "hot"])
def test_a_rejected_call_writes_nothing(broken):
    c = Call()
    if broken == "lru":
        c.lru[1] = [0, 0, 1, 2]
        want = ELRU
    elif broken == "rows":
        c.rows[:] = 1
        want = EROWS
    else:
        c.a.hot_nrows = 9            # slot H of state row 1 is row 9
        want = EHOT
    assert c() == want
    assert c.out.tolist() == [[7777] * 2] * 2 and c.cnt.tolist() == [7777] * 2
    assert (c.st == -1).all() and not c.hot.any()


def test_plan_and_v_buffers_come_in_pairs():
    c = Call()
    cnt = np.zeros(2, np.int32)
    src = np.zeros((2, 2), np.int64)
    dst = np.zeros((2, 2), np.int32)
    assert c(list_count=cnt, list_src=None, list_dst=dst) == EARG
    assert Call()(list_count=cnt, list_src=src, list_dst=None) == EARG
    assert Call()(list_count=cnt, list_src=src, list_dst=dst) == 0
    assert Call()(pool_v=np.zeros((20, 4), np.uint8)) == EARG
    assert Call()(hot_v=np.zeros((10, 4), np.uint8)) == EARG


@pytest.mark.parametrize("field,value", [
    ("hot_block_table", None), ("hot_block_size", 0), ("hot_table_stride", 1),
    ("src_block_size", 0), ("src_num_blocks", -1),
    ("resident_block_size", 0), ("resident_num_blocks", -1),
])
def test_paged_rejects_each_bad_table(field, value):
    src = np.asarray([np.arange(1, 11), np.arange(10, 20)], np.int32)
    res = np.zeros((2, 5), np.int32)
    kw = dict(src_block_table=src, src_table_stride=10, src_num_blocks=10, src_block_size=1,
              resident_block_table=res, resident_table_stride=5, resident_num_blocks=5,
              resident_block_size=2, resident_null_block=0)
    c = Call(paged=kw)
    assert c() == 0
    kw[field] = value
    if field == "resident_block_size":
        kw["hot_block_size"] = 0 if value == 0 else 2
    assert Call(paged=kw)() == EARG


def test_paged_boundaries_accepted_and_pool_rows_beyond_int32_rejected():
    # a hot table of exactly H slots; zero source blocks (every position has no row)
    c = Call(paged=dict(src_block_table=np.ones((2, 1), np.int32), src_table_stride=1,
                        src_num_blocks=0, src_block_size=1))
    assert c() == 0 and c.out.tolist() == [[-1, -1], [-1, -1]]
    assert Call(paged={})(pool_nrows=2**31) == EARG
    c = Call(paged={})
    assert c(pool_nrows=2**31 - 1) == 0 and c.cnt.tolist() == [2, 2]
    # a resident table of zero blocks: no position is resident
    c = Call(paged=dict(src_block_table=np.asarray([np.arange(1, 11), np.arange(10, 20)], np.int32),
                        src_table_stride=10, src_num_blocks=10, src_block_size=1,
                        resident_block_table=np.zeros((2, 1), np.int32), resident_table_stride=1,
                        resident_num_blocks=0, resident_block_size=2, resident_null_block=5))
    assert c() == 0 and c.cnt.tolist() == [2, 2]


def test_state_checks_cover_row_zero_and_the_first_lru_position():
    c = Call()
    c.lru[0] = [3, 1, 2, 3]            # row 0, position 0 repeats position 3
    assert c() == ELRU
    for bad in ([-1, 1, 2, 3], [4, 1, 2, 3], [0, 1, 2, 4]):   # -1 and H are not slot ids
        c = Call()
        c.lru[1] = bad
        assert c() == ELRU


def test_padding_rows_are_not_checked():
    """A padding row may name a real row's state row, and a state row at R
    (padding) is never read: its LRU row here is not a permutation."""
    st, lru = gen.initial_state(3, 4, 5)
    lru[2] = [0, 0, 0, 0]
    c = Call()
    c.st, c.lru = st[:2], lru[:2]
    assert c(slot_tokens=st, lru=lru, req_rows=np.asarray([0, 2], np.int64)) == 0
    assert c.out[1].tolist() == [-1, -1] and c.cnt.tolist() == [2, 0]
    c = Call()
    assert c(req_rows=np.asarray([0, 0], np.int64), num_real=1) == 0
    assert c.cnt.tolist() == [2, 0]
    c = Call()
    c.lru[1] = [0, 0, 0, 0]          # the padding row's own state row
    assert c(num_real=1) == 0 and c.cnt.tolist() == [2, 0]


@pytest.mark.parametrize("slot,row", [(0, 10), (4, 10), (4, -1), (3, 10)])
def test_every_slot_row_must_lie_in_the_hot_buffer(slot, row):
    """Slot rows from a table: the first slot, the newest slot (H) and the
    last LRU slot are all checked, and row == hot_nrows is already outside."""
    rows = np.arange(10, dtype=np.int32).reshape(2, 5)
    c = Call()
    assert c(slot_rows=rows) == 0
    rows = rows.copy()
    rows[1, slot] = row
    assert Call()(slot_rows=rows) == EHOT


def test_num_real_zero_makes_every_row_padding():
    c = Call()
    assert c(num_real=0) == 0
    assert c.out.tolist() == [[-1, -1], [-1, -1]] and c.cnt.tolist() == [0, 0]
    c = Call()
    assert c(num_real=2) == 0 and c.cnt.tolist() == [2, 2]


def test_an_id_equal_to_the_row_stride_is_invalid():
    """seq_len past ctx_stride: ids at or past the stride have no pool row of
    this request (r * ctx_stride + ctx_stride is the next request's row 0)."""
    c = Call()
    assert c(seq_lens=np.asarray([15, 15], np.int64), topk=np.asarray([[10, 9], [11, 0]], np.int32)) == 0
    assert c.out.tolist() == [[-1, 0], [-1, 5]] and c.cnt.tolist() == [1, 1]
    assert np.array_equal(c.hot[0], c.pool[9]) and np.array_equal(c.hot[5], c.pool[10])


def test_paged_global_id_zero_is_a_row():
    """No source table: a position is its global id, and id 0 is pool row 0."""
    c = Call(paged={})
    assert c(topk=np.asarray([[0, 1], [0, 5]], np.int32)) == 0
    assert c.cnt.tolist() == [2, 2] and c.out.tolist() == [[0, 1], [4, 5]]
    assert c.st.tolist() == [[0, 1, -1, -1, -1], [0, 5, -1, -1, -1]]


def test_paged_resident_block_zero_is_real_when_it_is_not_the_null_block():
    src = np.asarray([np.arange(1, 11), np.arange(10, 20)], np.int32)
    res = np.full((2, 5), 3, np.int32)      # null block 3 ...
    res[0, 0] = 0                          # ... and block 0 resident: positions 0, 1 -> rows 0, 1
    c = Call(paged=dict(src_block_table=src, src_table_stride=10, src_num_blocks=10,
                        src_block_size=1, resident_block_table=res, resident_table_stride=5,
                        resident_num_blocks=5, resident_block_size=2, resident_null_block=3))
    assert c(topk=np.asarray([[1, 0], [1, 2]], np.int32)) == 0
    assert c.out[0].tolist() == [1, 0] and c.cnt.tolist() == [0, 2]


def test_attention_rows_wider_than_top_k_keep_their_tail():
    att = np.full((2, 5), 7777, np.int32)
    c = Call(paged=dict(attention_indices=att, attention_row_stride=5, attention_block_stride=10))
    assert c() == 0
    assert att[:, 2:].tolist() == [[7777] * 3] * 2
    assert att[:, :2].tolist() == [[0, 1], [20, 21]]    # rows 0, 1 | 4, 5 in blocks of 2


# ---- the copy entry points -------------------------------------------------

def _lib():
    return oracle._load()


def test_copies_reject_bad_sizes_and_missing_buffers():
    L = _lib()
    one = (ctypes.c_void_p * 1)(1)
    idx = np.zeros(1, np.int64)
    buf = np.zeros((1, 4), np.uint8)
    for args in [(one, one, 1, 1, _p(idx), _p(idx), -1, 1, 4), (one, one, 1, 1, _p(idx), _p(idx), 1, -1, 4),
                 (one, one, 1, 1, _p(idx), _p(idx), 1, 1, 0), (None, one, 1, 1, _p(idx), _p(idx), 1, 1, 4),
                 (one, None, 1, 1, _p(idx), _p(idx), 1, 1, 4), (one, one, 1, 1, None, _p(idx), 1, 1, 4),
                 (one, one, 1, 1, _p(idx), None, 1, 1, 4)]:
        assert L.oracle_transfer_rows_all_layer(*args) == EARG
    for args in [(one, one, one, one, 1, 1, _p(idx), _p(idx), -1, 1, 4),
                 (one, one, one, one, 1, 1, _p(idx), _p(idx), 1, -1, 4),
                 (one, one, one, one, 1, 1, _p(idx), _p(idx), 1, 1, 0)] + \
                [tuple(None if k == j else x for k, x in enumerate((one, one, one, one, 1, 1, _p(idx), _p(idx), 1, 1, 4)))
                 for j in (0, 1, 2, 3, 6, 7)]:
        assert L.oracle_transfer_kv_all_layer(*args) == EARG
    p = _p(buf)
    for args in [(p, 4, p, 4, p, 4, p, 4, 1, _p(idx), -1, 4), (p, 4, p, 4, p, 4, p, 4, 1, _p(idx), 1, 0)] + \
                [tuple(None if k == j else x for k, x in enumerate((p, 4, p, 4, p, 4, p, 4, 1, _p(idx), 1, 4)))
                 for j in (0, 2, 4, 6, 9)]:
        assert L.oracle_store_kv_cache(*args) == EARG
    for args in [(p, 4, p, 4, 1, _p(idx), -1, 4), (p, 4, p, 4, 1, _p(idx), 1, 0),
                 (None, 4, p, 4, 1, _p(idx), 1, 4), (p, 4, None, 4, 1, _p(idx), 1, 4),
                 (p, 4, p, 4, 1, None, 1, 4)]:
        assert L.oracle_store_kv_scatter(*args) == EARG
    cnt = np.ones(1, np.int32)
    s = np.zeros((1, 1), np.int64)
    d = np.zeros((1, 1), np.int32)
    base = (_p(cnt), _p(s), _p(d), 1, 1, one, 1, one, 1, 1, 4)
    for j, v in [(3, -1), (4, -1), (9, -1), (10, 0), (0, None), (1, None), (2, None), (5, None), (7, None)]:
        assert L.oracle_gather_compact_layers(*[v if k == j else x for k, x in enumerate(base)]) == EARG


def test_empty_copies_touch_nothing():
    """Zero pairs, zero layers or zero rows: nothing is read (missing buffers
    included) and nothing is skipped."""
    L = _lib()
    one = (ctypes.c_void_p * 1)(1)
    assert L.oracle_transfer_rows_all_layer(None, None, 1, 1, None, None, 0, 1, 4) == 0
    assert L.oracle_transfer_rows_all_layer(None, None, 1, 1, None, None, 5, 0, 4) == 0
    assert L.oracle_transfer_kv_all_layer(None, None, None, None, 1, 1, None, None, 0, 1, 4) == 0
    assert L.oracle_transfer_kv_all_layer(None, None, None, None, 1, 1, None, None, 3, 0, 4) == 0
    assert L.oracle_store_kv_cache(None, 4, None, 4, None, 4, None, 4, 1, None, 0, 4) == 0
    assert L.oracle_store_kv_scatter(None, 4, None, 4, 1, None, 0, 4) == 0
    assert L.oracle_gather_compact_layers(None, None, None, 0, 1, one, 1, one, 1, 1, 4) == 0
    assert L.oracle_gather_compact_layers(None, None, None, 1, 0, one, 1, one, 1, 1, 4) == 0
    assert L.oracle_gather_compact_layers(None, None, None, 1, 1, None, 1, None, 1, 0, 4) == 0
    assert L.oracle_invalidate_written(None, 1, 1, None, None, 0) == 0


def test_a_row_at_the_destination_end_is_skipped():
    src = np.arange(8, dtype=np.uint8).reshape(2, 4)
    dst = np.zeros((3, 4), np.uint8)
    assert oracle.store_kv_scatter(src, dst, np.asarray([3, 1], np.int64)) == 1
    assert dst.tolist() == [[0] * 4, [4, 5, 6, 7], [0] * 4]
    k, v = np.zeros((3, 4), np.uint8), np.zeros((3, 4), np.uint8)
    assert oracle.store_kv_cache(src, src + 1, k, v, np.asarray([0, 3], np.int64)) == 1
    assert k.tolist() == [[0, 1, 2, 3], [0] * 4, [0] * 4] and v[0].tolist() == [1, 2, 3, 4]


def test_copies_of_one_byte_rows():
    """Any positive row size: one-byte rows are copied like any other."""
    src = [np.arange(5, dtype=np.uint8).reshape(5, 1)]
    dst = [np.zeros((5, 1), np.uint8)]
    idx = np.asarray([4, 1], np.int64)
    assert oracle.transfer_rows_all_layer(src, dst, idx, idx[::-1].copy()) == 0
    assert dst[0].ravel().tolist() == [0, 4, 0, 0, 1]
    kd, vd = [np.zeros((5, 1), np.uint8)], [np.zeros((5, 1), np.uint8)]
    assert oracle.transfer_kv_all_layer(src, [s + 1 for s in src], kd, vd, idx, idx) == 0
    assert kd[0].ravel().tolist() == [0, 1, 0, 0, 4] and vd[0].ravel().tolist() == [0, 2, 0, 0, 5]
    d = np.zeros((5, 1), np.uint8)
    assert oracle.store_kv_scatter(src[0][:2], d, idx) == 0 and d.ravel().tolist() == [0, 1, 0, 0, 0]
    k, v = np.zeros((5, 1), np.uint8), np.zeros((5, 1), np.uint8)
    assert oracle.store_kv_cache(src[0][:2], src[0][2:4], k, v, idx) == 0
    assert k.ravel().tolist() == [0, 1, 0, 0, 0] and v.ravel().tolist() == [0, 3, 0, 0, 2]
    hot = [np.zeros((5, 1), np.uint8)]
    assert oracle.gather_compact_layers(np.asarray([1], np.int32), np.asarray([[3]], np.int64),
                                        np.asarray([[2]], np.int32), src, hot) == 0   # K = 1
    assert hot[0].ravel().tolist() == [0, 0, 3, 0, 0]


def test_gather_clamps_the_count_to_top_k():
    pool = [np.arange(16, dtype=np.uint8).reshape(4, 4)]
    hot = [np.zeros((4, 4), np.uint8)]
    src = np.asarray([[1, 2]], np.int64)
    dst = np.asarray([[0, 3]], np.int32)
    assert oracle.gather_compact_layers(np.asarray([5], np.int32), src, dst, pool, hot) == 0
    assert hot[0][0].tolist() == [4, 5, 6, 7] and hot[0][3].tolist() == [8, 9, 10, 11]
    hot = [np.zeros((4, 4), np.uint8)]
    assert oracle.gather_compact_layers(np.asarray([-3], np.int32), src, dst, pool, hot) == 0
    assert not hot[0].any()


# ---- invalidation and reset --------------------------------------------------

def test_invalidate_edges():
    L = _lib()
    keys = np.asarray([[0, 5, 0], [7, 0, 9]], np.int32)
    assert oracle.invalidate_written(keys, np.asarray([0, 2, -1], np.int64), np.asarray([0, 9, 9], np.int64)) == 2
    assert keys.tolist() == [[-1, 5, -1], [7, 0, 9]]        # global row 0 is a row; state row 2 is past R
    # only the first n pairs count: the spare pair past n would clear key 7
    rows = np.asarray([1, 1], np.int64)
    written = np.asarray([9, 7], np.int64)
    assert L.oracle_invalidate_written(_p(keys), 2, 3, _p(rows), _p(written), 1) == 1
    assert keys.tolist() == [[-1, 5, -1], [7, 0, -1]]
    # state rows -1 and R exist in the backing array here and hold the keys:
    # they are outside [0, R) all the same; a negative written id clears nothing
    back = np.asarray([[5, 5, 5], [-1, 5, 6], [-1, 6, -1], [5, 5, 5]], np.int32)
    keys2 = back[1:3]
    rows2 = np.asarray([-1, 2, 0, 1], np.int64)
    written2 = np.asarray([5, 5, -1, -1], np.int64)
    assert L.oracle_invalidate_written(_p(keys2), 2, 3, _p(rows2), _p(written2), 4) == 0
    assert back.tolist() == [[5, 5, 5], [-1, 5, 6], [-1, 6, -1], [5, 5, 5]]
    assert L.oracle_invalidate_written(_p(keys2), 0, 3, _p(rows2), _p(written2), 4) == 0   # R = 0
    assert L.oracle_invalidate_written(_p(keys2), 2, 0, _p(rows2), _p(written2), 4) == 0   # S_r = 0
    for args in [(_p(keys), -1, 3, _p(rows), _p(written), 1), (_p(keys), 2, -1, _p(rows), _p(written), 1),
                 (_p(keys), 2, 3, _p(rows), _p(written), -1), (None, 2, 3, _p(rows), _p(written), 1),
                 (_p(keys), 2, 3, None, _p(written), 1), (_p(keys), 2, 3, _p(rows), None, 1)]:
        assert L.oracle_invalidate_written(*args) == EARG


def test_state_reset_edges():
    """Rows must be in [0, R) and a row needs its H LRU slots and the newest
    slot (S_r >= H + 1); a reset leaves the neighbouring rows alone."""
    L = _lib()
    st = np.full((3, 5), 7, np.int32)
    lru = np.full((3, 4), 3, np.int16)
    rows = np.asarray([1], np.int64)
    assert L.oracle_state_reset(_p(st), _p(lru), _p(rows), 1, 4, 5, 3) == 0
    assert st.tolist() == [[7] * 5, [-1] * 5, [7] * 5]
    assert lru.tolist() == [[3] * 4, [0, 1, 2, 3], [3] * 4]
    assert L.oracle_state_reset(_p(st), _p(lru), _p(rows), 0, 4, 5, 3) == 0
    row0 = np.asarray([0], np.int64)
    st0, lru0 = np.full((1, 1), 7, np.int32), np.zeros((1, 0), np.int16)
    assert L.oracle_state_reset(_p(st0), _p(lru0), _p(row0), 1, 0, 1, 1) == 0   # H = 0
    assert st0.tolist() == [[-1]]
    past, neg = np.asarray([3], np.int64), np.asarray([-1], np.int64)
    for args in [(_p(st), _p(lru), _p(past), 1, 4, 5, 3),
                 (_p(st), _p(lru), _p(neg), 1, 4, 5, 3),
                 (_p(st), _p(lru), _p(rows), -1, 4, 5, 3), (_p(st), _p(lru), _p(rows), 1, -1, 5, 3),
                 (_p(st), _p(lru), _p(rows), 1, 4, 4, 3), (None, _p(lru), _p(rows), 1, 4, 5, 3),
                 (_p(st), None, _p(rows), 1, 4, 5, 3), (_p(st), _p(lru), None, 1, 4, 5, 3)]:
        assert L.oracle_state_reset(*args) == EARG
    assert st.tolist() == [[7] * 5, [-1] * 5, [7] * 5]
    assert L.oracle_state_reset(_p(st), _p(lru), _p(row0), 1, 4, 5, 3) == 0     # row 0
    assert st.tolist() == [[-1] * 5, [-1] * 5, [7] * 5]
