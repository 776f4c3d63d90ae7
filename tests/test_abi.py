"""The C-ABI library loads, exports every function include/hisparse.h declares,
and rejects bad arguments on the host before touching the GPU (no compute
calls here: these run without a GPU)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hisparse.h")


@pytest.fixture(scope="module")
def lib():
    from sparse_attention_kv_hisparse_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from sparse_attention_kv_hisparse_amd.build import build
        build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w[\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_expected_calls():
    from sparse_attention_kv_hisparse_amd._lib import EXPORTS
    assert declared_functions() == sorted(EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def _args(**kw):
    from sparse_attention_kv_hisparse_amd._lib import SwapInArgs
    fake = 0x100000   # never dereferenced: validation fails first
    base = dict(B=2, K=4, H=8, S_r=9, R=2, topk_ids=fake, topk_stride=4, req_rows=fake,
                seq_lens=fake, num_real=None, slot_tokens=fake, lru=fake, slot_rows=None,
                pool_rows=None, ctx_stride=100, pool=fake, pool_nrows=200, hot=fake,
                hot_nrows=18, row_bytes=16, out_rows=fake, miss_counts=None)
    base.update(kw)
    return SwapInArgs(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), -1),
    (dict(H=3), -1),                      # H < K
    (dict(H=40000, K=4), -2),             # H above int16 slots
    (dict(S_r=8), -1),                    # no newest slot
    (dict(row_bytes=6), -1),
    (dict(row_bytes=0), -1),
    (dict(topk_stride=3), -1),
    (dict(ctx_stride=0), -1),
    (dict(pool=None), -1),
    (dict(out_rows=None), -1),
    (dict(hot_nrows=17), -1),             # flat regions need R*S_r rows
    (dict(pool=0x100002), -1),            # not 4-byte aligned
    (dict(row_bytes=1 << 21), -2),
    (dict(stats=0x100004), -1),           # counters not 8-byte aligned
])
def test_swap_in_rejects_bad_arguments(lib, kw, status):
    a = _args(**kw)
    rc = lib.hisparse_swap_in(ctypes.byref(a), ctypes.c_void_p(0x200000), 1 << 20, None)
    assert rc == status
    assert lib.hisparse_last_error()


def test_swap_in_rejects_small_workspace(lib):
    a = _args()
    need = lib.hs_swap_in_workspace_bytes(2, 4)
    assert lib.hisparse_swap_in(ctypes.byref(a), ctypes.c_void_p(0x200000), need - 1, None) == -5
    assert lib.hisparse_swap_in(ctypes.byref(a), ctypes.c_void_p(0x200010), need, None) == -5
    assert lib.hisparse_swap_in(ctypes.byref(a), None, need, None) == -5
    assert lib.hisparse_swap_in(None, None, 0, None) == -1


def test_swap_in_empty_is_ok(lib):
    assert lib.hisparse_swap_in(ctypes.byref(_args(B=0)), None, 0, None) == 0
    assert lib.hisparse_swap_in(ctypes.byref(_args(K=0)), None, 0, None) == 0


def test_workspace_size(lib):
    assert lib.hs_swap_in_workspace_bytes(0, 5) == 0
    b, k = 32, 2048
    size = lib.hs_swap_in_workspace_bytes(b, k)
    assert size >= b * 4 + b * k * 12 and size % 256 == 0


def test_workspace_layout(lib):
    c, s, d = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    b, k = 7, 300
    total = lib.hs_swap_in_workspace_layout(b, k, ctypes.byref(c), ctypes.byref(s), ctypes.byref(d))
    assert total == lib.hs_swap_in_workspace_bytes(b, k)
    # three disjoint, 256-byte aligned regions, in order, inside the total
    assert c.value == 0 and s.value >= 4 * b and d.value >= s.value + 8 * b * k
    assert d.value + 4 * b * k <= total
    assert s.value % 256 == 0 and d.value % 256 == 0
    assert lib.hs_swap_in_workspace_layout(0, 3, None, None, None) == 0


@pytest.mark.parametrize("name", ["hisparse_resolve", "hisparse_gather_compact"])
def test_split_calls_validate_like_swap_in(lib, name):
    fn = getattr(lib, name)
    assert fn(ctypes.byref(_args(H=3)), ctypes.c_void_p(0x200000), 1 << 20, None) == -1
    assert fn(ctypes.byref(_args(B=0)), None, 0, None) == 0
    assert fn(None, None, 0, None) == -1


def test_transfer_rejects(lib):
    f = 0x100000
    assert lib.transfer_rows_all_layer(f, f, f, f, -1, 3, 16, 10, 10, 0, None) == -1
    assert lib.transfer_rows_all_layer(f, f, f, f, 5, 3, 6, 10, 10, 0, None) == -1
    assert lib.transfer_rows_all_layer(None, f, f, f, 5, 3, 16, 10, 10, 0, None) == -1
    assert lib.transfer_rows_all_layer(f, f, f, f, 5, 3, 16, -1, 10, 0, None) == -1
    assert lib.transfer_rows_all_layer(None, None, None, None, 0, 3, 16, 10, 10, 0, None) == 0
    assert lib.transfer_rows_all_layer(None, None, None, None, 4, 0, 16, 10, 10, 0, None) == 0
    # flags: only HS_TRANSFER_HOST_LINK (1) is defined
    assert lib.transfer_rows_all_layer(None, None, None, None, 0, 3, 16, 10, 10, 1, None) == 0
    assert lib.transfer_rows_all_layer(f, f, f, f, 5, 3, 16, 10, 10, 2, None) == -1
    assert b"flags" in lib.hisparse_last_error()
    assert lib.transfer_rows_all_layer(None, None, None, None, 0, 3, 16, 10, 10, 0x80000000, None) == -1


def test_transfer_flags_for_rejects_null(lib):
    flags = ctypes.c_uint32(7)
    assert lib.hs_transfer_flags_for(None, ctypes.c_void_p(0x1000), ctypes.byref(flags)) == -1
    assert lib.hs_transfer_flags_for(ctypes.c_void_p(0x1000), None, ctypes.byref(flags)) == -1
    assert lib.hs_transfer_flags_for(ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1000), None) == -1
    assert flags.value == 7


def test_scatter_rejects(lib):
    f = 0x100000
    assert lib.store_kv_scatter(f, 8, f, 16, 10, f, 3, 16, None) == -1      # src stride < rb
    assert lib.store_kv_scatter(f, 16, f, 16, 10, f, 3, 10, None) == -1     # rb % 4
    assert lib.store_kv_scatter(f + 2, 16, f, 16, 10, f, 3, 16, None) == -1  # misaligned
    assert lib.store_kv_scatter(None, 16, f, 16, 10, f, 3, 16, None) == -1
    assert lib.store_kv_scatter(None, 16, None, 16, 10, None, 0, 16, None) == 0


def test_reset_rejects(lib):
    f = 0x100000
    assert lib.hisparse_state_reset(f, f, f, 3, 8, 8, 4, None) == -1        # S_r < H+1
    assert lib.hisparse_state_reset(f, f, f, 3, 40000, 40001, 4, None) == -2
    assert lib.hisparse_state_reset(None, None, None, 0, 8, 9, 4, None) == 0


def test_fastdiv_is_exact():
    """The copy kernels' division by a run-time constant: q = (n*m) >> s with
    s = 31 + ceil(log2 d), m = ceil(2^s/d), claimed exact for n < 2^31."""
    import random
    rnd = random.Random(5)
    divisors = list(range(1, 2100)) + [rnd.randrange(1, 1 << 31) for _ in range(300)] + [(1 << 31) - 1]
    for d in divisors:
        l = (d - 1).bit_length()
        s = 31 + l
        m = ((1 << s) + d - 1) // d
        assert m < (1 << 33)
        ns = [0, 1, d - 1, d, d + 1, (1 << 31) - 1, (1 << 31) - 2] + \
             [rnd.randrange(0, 1 << 31) for _ in range(40)] + \
             [k * d - 1 for k in (1, 2, 1000) if k * d - 1 < (1 << 31)]
        for n in ns:
            if 0 <= n < (1 << 31):
                assert ((n * m) & ((1 << 64) - 1)) >> s == n // d, (n, d)


def test_gather_layers_rejects(lib):
    f = ctypes.c_void_p(0x100000)
    ws = ctypes.c_void_p(0x200000)
    need = lib.hs_swap_in_workspace_bytes(2, 4)
    g = lib.hisparse_gather_compact_layers
    assert g(ws, need, 0, 4, f, 10, f, 10, 3, 16, None) == 0           # empty
    assert g(ws, need, 2, 4, f, 10, f, 10, 0, 16, None) == 0           # no layers
    assert g(ws, need, -1, 4, f, 10, f, 10, 3, 16, None) == -1
    assert g(ws, need, 2, 4, None, 10, f, 10, 3, 16, None) == -1
    assert g(ws, need, 2, 4, f, 10, f, 10, 3, 18, None) == -1          # row_bytes % 4
    assert g(ws, need, 2, 4, f, -1, f, 10, 3, 16, None) == -1
    assert g(ws, need, 2, 4, f, 10, f, 1 << 40, 3, 16, None) == -2     # hot rows beyond int32
    assert g(ws, need, 2, 4, f, 10, f, 10, 3, 1 << 21, None) == -2
    assert g(ws, need - 1, 2, 4, f, 10, f, 10, 3, 16, None) == -5
    assert g(None, need, 2, 4, f, 10, f, 10, 3, 16, None) == -5
    assert g(ctypes.c_void_p(0x200010), need, 2, 4, f, 10, f, 10, 3, 16, None) == -5
    assert g(ws, need, 2, 4, f, 10, f, 10, 1 << 20, 1 << 20, None) == -2   # items beyond 2^31
    assert lib.hisparse_last_error()


def test_kv_entries_reject(lib):
    f = 0x100000
    t = lib.transfer_kv_all_layer
    assert t(f, f, f, f, f, f, 0, 3, 16, 10, 10, 0, None) == 0            # empty
    assert t(f, f, f, f, f, f, 5, 0, 16, 10, 10, 1, None) == 0            # no layers
    assert t(f, None, f, f, f, f, 5, 3, 16, 10, 10, 0, None) == -1        # V arrays missing
    assert t(f, f, f, None, f, f, 5, 3, 16, 10, 10, 0, None) == -1
    assert t(f, f, f, f, f, f, 5, 3, 14, 10, 10, 0, None) == -1           # row_bytes % 4
    assert t(f, f, f, f, f, f, -1, 3, 16, 10, 10, 0, None) == -1
    assert t(f, f, f, f, f, f, 5, 3, 16, 10, 10, 4, None) == -1           # unknown flag
    s = lib.store_kv_cache
    assert s(None, 16, None, 16, None, 16, None, 16, 10, None, 0, 16, None) == 0
    assert s(f, 16, f, 8, f, 16, f, 16, 10, f, 3, 16, None) == -1         # v src stride < rb
    assert s(f, 16, f, 16, f, 16, f + 2, 16, 10, f, 3, 16, None) == -1    # misaligned v dst
    assert s(f, 16, None, 16, f, 16, f, 16, 10, f, 3, 16, None) == -1
    assert s(f, 16, f, 16, f, 16, f, 16, 10, f, 3, 10, None) == -1        # row_bytes % 4
    assert lib.hisparse_last_error()


def test_swap_in_rejects_half_kv(lib):
    a = _args()
    a.pool_v = 0x300000
    assert lib.hisparse_swap_in(ctypes.byref(a), ctypes.c_void_p(0x200000), 1 << 20, None) == -1
    a.pool_v = None
    a.hot_v = 0x300000
    assert lib.hisparse_swap_in(ctypes.byref(a), ctypes.c_void_p(0x200000), 1 << 20, None) == -1
    a.pool_v = 0x300002
    assert lib.hisparse_swap_in(ctypes.byref(a), ctypes.c_void_p(0x200000), 1 << 20, None) == -1


def test_paged_addressing_validation(lib):
    from sparse_attention_kv_hisparse_amd._lib import PagedAddressing
    f = 0x100000
    good = dict(hot_block_table=f, hot_table_stride=4, hot_block_size=2)

    def call(**kw):
        pg = PagedAddressing(**{**good, **kw})
        a = _args(seq_lens=None, ctx_stride=0)
        a.paged = ctypes.pointer(pg)
        return lib.hisparse_swap_in(ctypes.byref(a), ctypes.c_void_p(0x200000), 1 << 20, None)

    assert call(hot_block_table=None) == -1
    assert call(hot_block_size=0) == -1
    assert call(hot_table_stride=3) == -1                       # 3 blocks of 2 < H = 8
    assert call(src_block_table=f, src_block_size=0) == -1
    assert call(src_block_table=f, src_block_size=4, src_num_blocks=5, src_table_stride=4) == -1
    assert call(resident_block_table=f, resident_block_size=4, resident_num_blocks=2,
                resident_table_stride=1) == -1
    # The vLLM page's host checks of a resident table: it needs the source
    # table, block sizes equal to the hot block size, a non-negative null block.
    src = dict(src_block_table=f, src_block_size=4, src_num_blocks=4, src_table_stride=4)
    res = dict(resident_block_table=f, resident_block_size=2, resident_num_blocks=4,
               resident_table_stride=4, resident_null_block=0)
    assert call(**res) == -1                                      # no source table
    assert call(**src, **dict(res, resident_block_size=4)) == -1  # sizes differ
    assert call(**src, **dict(res, resident_null_block=-1)) == -1
    assert call(**src, **res) != -1                               # in the page's domain
    assert call(attention_indices=f, attention_row_stride=3) == -1   # < K = 4
    a = _args(seq_lens=None)
    assert lib.hisparse_swap_in(ctypes.byref(a), ctypes.c_void_p(0x200000), 1 << 20, None) == -1
    pg = PagedAddressing(**good)
    a = _args(slot_rows=f)
    a.paged = ctypes.pointer(pg)
    assert lib.hisparse_swap_in(ctypes.byref(a), ctypes.c_void_p(0x200000), 1 << 20, None) == -1


def test_invalidate_rejects(lib):
    f = 0x100000
    g = lib.hisparse_invalidate_written
    assert g(f, 4, 9, f, f, 0, None) == 0
    assert g(f, 4, 9, f, f, -1, None) == -1
    assert g(None, 4, 9, f, f, 3, None) == -1
    assert g(f, 4, 9, None, f, 3, None) == -1


def test_noalloc_rejects_before_touching_the_gpu(lib):
    """hisparse_swap_in_noalloc: empty calls are no-ops, NULL args and miss
    lists beyond the fixed array (HS_NOALLOC_SCRATCH_BYTES) are rejected on the
    host, before any HIP call."""
    from sparse_attention_kv_hisparse_amd._lib import HS_NOALLOC_SCRATCH_BYTES
    f = lib.hisparse_swap_in_noalloc
    assert f(None, None) == -1
    assert f(ctypes.byref(_args(B=0)), None) == 0
    assert f(ctypes.byref(_args(K=0)), None) == 0
    assert lib.hs_swap_in_workspace_bytes(256, 2048) > HS_NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(_args(B=256, K=2048, H=2048, topk_stride=2048)), None) == -2
    assert b"allocation-free" in lib.hisparse_last_error()
    assert lib.hs_swap_in_workspace_bytes(128, 2048) <= HS_NOALLOC_SCRATCH_BYTES
