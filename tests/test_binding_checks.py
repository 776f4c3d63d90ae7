"""Every argument check of the Python binding, one case each: the call is
well formed except for one tensor, and must raise ValueError naming that
tensor before anything reaches the library. The checks that come before the
device checks run on CPU tensors; the rest (dtype checks, outputs checked
after the device check, per-call arguments of a prepared call) take device
tensors and are marked gpu -- every one of them raises before a launch."""

import pytest
import torch

import sparse_attention_kv_hisparse_amd as hs

B, K, R, H, S_r, ctx, rb = 3, 4, 5, 8, 9, 20, 16
i32, i64, i16, u8 = torch.int32, torch.int64, torch.int16, torch.uint8


def _z(shape, dtype, dev="cpu"):
    return torch.zeros(shape, dtype=dtype, device=dev)


def swap_args(dev="cpu", **over):
    a = dict(topk=_z((B, K), i32, dev), req_rows=_z(B, i64, dev), seq_lens=_z(B, i64, dev),
             slot_tokens=_z((R, S_r), i32, dev), lru=_z((R, H), i16, dev),
             pool=_z((R * ctx, rb), u8, dev), hot=_z((R * S_r, rb), u8, dev),
             out_rows=_z((B, K), i32, dev), ctx_stride=ctx, workspace=_z(1 << 16, u8, dev))
    a.update(over)
    return a


def _paged(**kw):
    p = {"hot_block_table": _z((R, 4), i32), "hot_block_size": 2}
    p.update(kw)
    return p


def _strided(shape, dtype, dev="cpu"):
    """A tensor of `shape` whose columns are not contiguous."""
    return _z((shape[0], 2 * shape[1]), dtype, dev)[:, ::2]


SWAP_CPU = [
    (dict(pool_v=_z((R * ctx, rb), u8)), "go together"),
    (dict(hot_v=_z((R * S_r, rb), u8)), "go together"),
    (dict(pool_v=_z((R * ctx - 1, rb), u8), hot_v=_z((R * S_r, rb), u8)), "pool_v / hot_v"),
    (dict(pool_v=_z((R * ctx, rb), u8), hot_v=_z((R * S_r - 1, rb), u8)), "pool_v / hot_v"),
    (dict(pool_v=_z((R * ctx, rb), i32), hot_v=_z((R * S_r, rb), u8)), "pool_v / hot_v"),
    (dict(pool_v=_z((R * ctx, rb), u8), hot_v=_z((R * S_r, rb), i32)), "pool_v / hot_v"),
    (dict(pool_v=_z((rb, R * ctx), u8).t(), hot_v=_z((R * S_r, rb), u8)), "pool_v / hot_v"),
    (dict(pool_v=_z((R * ctx, rb), u8), hot_v=_z((rb, R * S_r), u8).t()), "pool_v / hot_v"),
    (dict(pool_v=_z((R * ctx, rb), u8), hot_v=_z((R * S_r, rb), u8)), "hot_v must be a device"),
    (dict(topk=_z((B, K, 1), i32)), "topk"),
    (dict(topk=_z((B + 1, K), i32)), "topk"),
    (dict(topk=_z((B, K - 1), i32)), "topk"),
    (dict(topk=_strided((B, K), i32)), "topk"),
    (dict(slot_tokens=_strided((R, S_r), i32)), "slot_tokens must be contiguous"),
    (dict(lru=_strided((R, H), i16)), "lru must be contiguous"),
    (dict(out_rows=_strided((B, K), i32), topk=_z((B, 2 * K), i32)), "out_rows must be contiguous"),
    (dict(pool=_z(R * ctx * rb, u8)), "pool and hot must be contiguous"),
    (dict(hot=_z(R * S_r * rb, u8)), "pool and hot must be contiguous"),
    (dict(pool=_z((R * ctx, rb + 4), u8)), "pool and hot must be contiguous"),
    (dict(pool=_z((rb, R * ctx), u8).t()), "pool and hot must be contiguous"),
    (dict(hot=_z((rb, R * S_r), u8).t()), "pool and hot must be contiguous"),
    (dict(pool=_z((R * ctx, rb), i32), hot=_z((R * S_r, rb), i32)), "uint8 byte rows"),
    (dict(hot=_z((R * S_r, rb), i32), pool=_z((R * ctx, rb), i32)), "uint8 byte rows"),
    (dict(pool=_z((R * ctx, rb), i32)), "uint8 byte rows"),
    (dict(slot_tokens=_z(R * S_r, i32)), "slot_tokens must be"),
    (dict(lru=_z(R * H, i16)), "slot_tokens must be"),
    (dict(paged=_paged(hot_block_table=_z(R * 4, i32))), "hot_block_table must be a contiguous"),
    (dict(paged=_paged(hot_block_table=_strided((R, 4), i32))), "hot_block_table must be a contiguous"),
    (dict(paged=_paged(src_block_table=_z(R * 4, i32))), "src_block_table must be a contiguous"),
    (dict(paged=_paged(resident_block_table=_z((R - 1, 4), i32))), "resident_block_table must have"),
    (dict(out_rows=_z(B * K, i32)), "out_rows must be"),
    (dict(slot_rows=_z(R * S_r, i32)), "slot_rows"),
]


@pytest.mark.parametrize("over,needle", SWAP_CPU, ids=[f"{i}" for i in range(len(SWAP_CPU))])
def test_swap_in_rejects_each_bad_tensor(over, needle):
    with pytest.raises(ValueError, match=needle):
        hs.hisparse_swap_in(**swap_args(**over))


def test_prepared_call_checks_its_out_rows_first():
    with pytest.raises(ValueError, match="out_rows must be"):
        hs.SwapInCall(**{k: v for k, v in swap_args(out_rows=_z(B * K, i32)).items()
                         if k not in ("topk", "req_rows", "seq_lens")})


def test_copy_entry_points_check_lengths_and_shapes():
    p3, p2 = _z(3, i64), _z(2, i64)
    cases = [
        (hs.hisparse_gather_compact_layers,
         dict(workspace=_z(64, u8), B=1, K=1, pool_layer_ptrs=p3, pool_nrows=1, hot_layer_ptrs=p2,
              hot_nrows=1, row_bytes=4), "equal lengths"),
        (hs.transfer_rows_all_layer,
         dict(src_layer_ptrs=p3, dst_layer_ptrs=p2, src_idx=p3, dst_idx=p3, row_bytes=4,
              src_nrows=1, dst_nrows=1), "equal lengths"),
        (hs.transfer_rows_all_layer,
         dict(src_layer_ptrs=p3, dst_layer_ptrs=p3, src_idx=p3, dst_idx=p2, row_bytes=4,
              src_nrows=1, dst_nrows=1), "equal lengths"),
        (hs.transfer_rows_all_layer,
         dict(src_layer_ptrs=p3, dst_layer_ptrs=p3, src_idx=_z((3, 1), i64), dst_idx=_z((3, 1), i64),
              row_bytes=4, src_nrows=1, dst_nrows=1), "src_idx"),
        (hs.transfer_kv_all_layer,
         dict(k_src_layer_ptrs=p3, v_src_layer_ptrs=p2, k_dst_layer_ptrs=p3, v_dst_layer_ptrs=p3,
              src_idx=p3, dst_idx=p3, row_bytes=4, src_nrows=1, dst_nrows=1), "layer pointer arrays"),
        (hs.transfer_kv_all_layer,
         dict(k_src_layer_ptrs=p3, v_src_layer_ptrs=p3, k_dst_layer_ptrs=p2, v_dst_layer_ptrs=p3,
              src_idx=p3, dst_idx=p3, row_bytes=4, src_nrows=1, dst_nrows=1), "layer pointer arrays"),
        (hs.transfer_kv_all_layer,
         dict(k_src_layer_ptrs=p3, v_src_layer_ptrs=p3, k_dst_layer_ptrs=p3, v_dst_layer_ptrs=p2,
              src_idx=p3, dst_idx=p3, row_bytes=4, src_nrows=1, dst_nrows=1), "layer pointer arrays"),
        (hs.transfer_kv_all_layer,
         dict(k_src_layer_ptrs=p3, v_src_layer_ptrs=p3, k_dst_layer_ptrs=p3, v_dst_layer_ptrs=p3,
              src_idx=p3, dst_idx=p2, row_bytes=4, src_nrows=1, dst_nrows=1), "index arrays"),
        (hs.store_kv_cache, dict(k_src=_z((3, 8), i32), v_src=_z((3, 8), u8), k_dst=_z((9, 8), u8),
                                 v_dst=_z((9, 8), u8), loc=p3), "k_src must be"),
        (hs.store_kv_cache, dict(k_src=_z((3, 8), u8), v_src=_z(24, u8), k_dst=_z((9, 8), u8),
                                 v_dst=_z((9, 8), u8), loc=p3), "v_src must be"),
        (hs.store_kv_cache, dict(k_src=_z((3, 8), u8), v_src=_z((3, 8), u8),
                                 k_dst=_z((8, 9), u8).t(), v_dst=_z((9, 8), u8), loc=p3), "k_dst must be"),
        (hs.store_kv_cache, dict(k_src=_z((3, 8), u8), v_src=_z((3, 8), u8), k_dst=_z((9, 8), u8),
                                 v_dst=_z((8, 8), u8), loc=p3), "matching row counts"),
        (hs.store_kv_cache, dict(k_src=_z((3, 8), u8), v_src=_z((2, 8), u8), k_dst=_z((9, 8), u8),
                                 v_dst=_z((9, 8), u8), loc=p2), "matching row counts"),
        (hs.store_kv_cache, dict(k_src=_z((2, 8), u8), v_src=_z((2, 8), u8), k_dst=_z((9, 8), u8),
                                 v_dst=_z((9, 8), u8), loc=p3), "loc has"),
        (hs.store_kv_cache, dict(k_src=_z((3, 8), u8), v_src=_z((3, 8), u8), k_dst=_z((9, 8), u8),
                                 v_dst=_z((9, 4), u8), loc=p3), "row_bytes exceeds"),
        (hs.store_kv_scatter, dict(src=_z((3, 8), i32), dst=_z((9, 8), u8), loc=p3), "2-D uint8"),
        (hs.store_kv_scatter, dict(src=_z((3, 8), u8), dst=_z((9, 8), i32), loc=p3), "2-D uint8"),
        (hs.store_kv_scatter, dict(src=_z(24, u8), dst=_z((9, 8), u8), loc=p3), "2-D uint8"),
        (hs.store_kv_scatter, dict(src=_z((3, 8), u8), dst=_z(72, u8), loc=p3), "2-D uint8"),
        (hs.store_kv_scatter, dict(src=_z((8, 3), u8).t(), dst=_z((9, 8), u8), loc=p3), "contiguous"),
        (hs.store_kv_scatter, dict(src=_z((3, 8), u8), dst=_z((8, 9), u8).t(), loc=p3), "contiguous"),
        (hs.store_kv_scatter, dict(src=_z((3, 8), u8), dst=_z((9, 8), u8), loc=p3, row_bytes=12),
         "row_bytes exceeds"),
        (hs.hisparse_invalidate_written, dict(slot_keys=_z(R * S_r, i32), rows=p3, written=p3),
         "slot_keys must be"),
        (hs.hisparse_invalidate_written, dict(slot_keys=_strided((R, S_r), i32), rows=p3, written=p3),
         "slot_keys must be"),
        (hs.hisparse_invalidate_written, dict(slot_keys=_z((R, S_r), i32), rows=p3, written=p2),
         "equal lengths"),
        (hs.hisparse_state_reset, dict(slot_tokens=_z(R * S_r, i32), lru=_z((R, H), i16), rows=p3),
         "slot_tokens"),
        (hs.hisparse_state_reset, dict(slot_tokens=_z((R, S_r), i32), lru=_z(R * H, i16), rows=p3),
         "slot_tokens"),
        (hs.hisparse_state_reset, dict(slot_tokens=_strided((R, S_r), i32), lru=_z((R, H), i16),
                                       rows=p3), "slot_tokens"),
        (hs.hisparse_state_reset, dict(slot_tokens=_z((R, S_r), i32), lru=_strided((R, H), i16),
                                       rows=p3), "slot_tokens"),
    ]
    for fn, kw, needle in cases:
        with pytest.raises(ValueError, match=needle):
            fn(**kw)


def test_boundaries_pass_the_checks_and_fail_only_on_the_device_check():
    """Rows exactly as wide as row_bytes, and well-formed state for a reset:
    every shape check passes, and CPU tensors then fail the device check."""
    p3 = _z(3, i64)
    with pytest.raises(ValueError, match="device tensor"):
        hs.store_kv_scatter(src=_z((3, 8), u8), dst=_z((9, 8), u8), loc=p3, row_bytes=8)
    with pytest.raises(ValueError, match="device tensor"):
        hs.store_kv_cache(k_src=_z((3, 8), u8), v_src=_z((3, 8), u8), k_dst=_z((9, 8), u8),
                          v_dst=_z((9, 8), u8), loc=p3, row_bytes=8)
    with pytest.raises(ValueError, match="device tensor"):
        hs.hisparse_state_reset(slot_tokens=_z((R, S_r), i32), lru=_z((R, H), i16), rows=p3)


# ---- checks that come after the device checks (device tensors) ------------

@pytest.mark.gpu
def test_device_checks_of_the_swap_in():
    d = "cuda"
    cases = [
        (dict(topk=_z((B, K), i64, d)), "topk must be torch.int32"),
        (dict(req_rows=_z(B, i32, d)), "req_rows must be torch.int64"),
        (dict(lru=_z((R, H), i32, d)), "lru must be torch.int16"),
        (dict(topk=_z((B, K), i32)), "topk must be a device tensor"),
        (dict(miss_mask=_z((B, K + 1), i32, d)), "miss_mask"),
        (dict(miss_mask=_strided((B, K), i32, d)), "miss_mask"),
        (dict(stats=_z(2, i32, d)), "stats"),
        (dict(stats=_z(3, i64, d)), "stats"),
        (dict(stats=_z((2, 2), i64, d)[:, 0]), "stats"),
        (dict(workspace=_z(64, i32, d)), "workspace must be torch.uint8"),
    ]
    for over, needle in cases:
        with pytest.raises(ValueError, match=needle):
            hs.hisparse_swap_in(**swap_args(d, **over))


@pytest.mark.gpu
def test_device_checks_of_paged_tables():
    d = "cuda"

    def paged(**kw):
        p = {"hot_block_table": _z((R, 4), i32, d), "hot_block_size": 2,
             "src_block_table": _z((R, 6), i32, d), "resident_block_table": _z((R, 6), i32, d)}
        p.update(kw)
        return p
    for att in (_z(B * K, i32, d), _z((B + 1, K), i32, d), _strided((B, K), i32, d)):
        with pytest.raises(ValueError, match="attention_indices"):
            hs.hisparse_swap_in(**swap_args(d, paged=paged(attention_indices=att), seq_lens=None))
    with pytest.raises(ValueError, match="attention_indices must be torch.int32"):
        hs.hisparse_swap_in(**swap_args(d, paged=paged(attention_indices=_z((B, K), i64, d)),
                                        seq_lens=None))
    with pytest.raises(ValueError, match="src_block_table must be torch.int32"):
        hs.hisparse_swap_in(**swap_args(d, paged=paged(src_block_table=_z((R, 6), i64, d)),
                                        seq_lens=None))
    # everything else well formed: only the hot buffer's placement is left to fail
    with pytest.raises(ValueError, match="hot must be a device tensor"):
        hs.hisparse_swap_in(**swap_args(d, paged=paged(attention_indices=_z((B, K + 1), i32, d)),
                                        seq_lens=None, hot=_z((R * S_r, rb), u8)))


@pytest.mark.gpu
def test_prepared_call_checks_each_step():
    d = "cuda"
    kw = {k: v for k, v in swap_args(d).items() if k not in ("topk", "req_rows", "seq_lens")}
    call = hs.SwapInCall(**kw)
    for topk in (_z((B, K, 1), i32, d), _z((B + 1, K), i32, d), _z((B, K - 1), i32, d),
                 _strided((B, K), i32, d)):
        with pytest.raises(ValueError, match="topk must be"):
            call(topk, _z(B, i64, d), _z(B, i64, d))
    with pytest.raises(ValueError, match="req_rows"):
        call(_z((B, K), i32, d), _z(B - 1, i64, d), _z(B, i64, d))
    with pytest.raises(ValueError, match="seq_lens is required"):
        call(_z((B, K), i32, d), _z(B, i64, d))
    with pytest.raises(ValueError, match="seq_lens"):
        call(_z((B, K), i32, d), _z(B, i64, d), _z(B - 1, i64, d))
    with pytest.raises(ValueError, match="no workspace"):
        hs.SwapInCall(entry="hisparse_swap_in_noalloc", **kw)
    # prepared, not launched: the allocation-free entry keeps no workspace, the others do
    assert hs.SwapInCall(entry="hisparse_swap_in_noalloc",
                         **{k: v for k, v in kw.items() if k != "workspace"})._ws is None
    assert call._ws is not None
    with pytest.raises(ValueError, match="no workspace"):
        hs.hisparse_swap_in_noalloc(**swap_args(d))
