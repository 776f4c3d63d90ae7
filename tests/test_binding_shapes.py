"""The Python binding checks every tensor's shape against the sizes of the
call before handing pointers to the library (no GPU needed: the checks run
before any device check, on CPU tensors)."""

import pytest
import torch

import sparse_attention_kv_hisparse_amd as hs

B, K, R, H, S_r, ctx = 3, 4, 5, 8, 9, 20


def _args(**over):
    a = dict(topk=torch.zeros((B, K), dtype=torch.int32),
             req_rows=torch.zeros(B, dtype=torch.int64),
             seq_lens=torch.zeros(B, dtype=torch.int64),
             slot_tokens=torch.zeros((R, S_r), dtype=torch.int32),
             lru=torch.zeros((R, H), dtype=torch.int16),
             pool=torch.zeros((R * ctx, 16), dtype=torch.uint8),
             hot=torch.zeros((R * S_r, 16), dtype=torch.uint8),
             out_rows=torch.zeros((B, K), dtype=torch.int32), ctx_stride=ctx,
             workspace=torch.zeros(1 << 16, dtype=torch.uint8))
    a.update(over)
    return a


@pytest.mark.parametrize("over,needle", [
    (dict(lru=torch.zeros((R - 1, H), dtype=torch.int16)), "lru has"),
    (dict(req_rows=torch.zeros(B - 1, dtype=torch.int64)), "req_rows"),
    (dict(seq_lens=torch.zeros(B - 1, dtype=torch.int64)), "seq_lens"),
    (dict(miss_counts=torch.zeros(B - 1, dtype=torch.int32)), "miss_counts"),
    (dict(miss_counts=torch.zeros((B, 2), dtype=torch.int32)[:, 0]), "miss_counts"),
    (dict(num_real=torch.zeros(0, dtype=torch.int32)), "num_real"),
    (dict(slot_rows=torch.zeros((R - 1, S_r), dtype=torch.int32)), "slot_rows"),
    (dict(slot_rows=torch.zeros((R, S_r - 1), dtype=torch.int32)), "slot_rows"),
    (dict(pool_rows=torch.zeros((R, ctx - 1), dtype=torch.int64)), "pool_rows"),
    (dict(pool_rows=torch.zeros((R - 1, ctx), dtype=torch.int64)), "pool_rows"),
    (dict(topk=torch.zeros((B, K - 1), dtype=torch.int32)), "topk"),
    (dict(paged={"hot_block_table": torch.zeros((R - 1, 4), dtype=torch.int32),
                 "hot_block_size": 2}), "hot_block_table"),
    (dict(paged={"hot_block_table": torch.zeros((R, 4), dtype=torch.int32), "hot_block_size": 2,
                 "src_block_table": torch.zeros((R - 2, 4), dtype=torch.int32),
                 "src_block_size": 4}), "src_block_table"),
])
def test_swap_in_rejects_mis_shaped_tensors(over, needle):
    with pytest.raises(ValueError, match=needle):
        hs.hisparse_swap_in(**_args(**over))


def test_well_shaped_cpu_tensors_fail_only_on_the_device_check():
    with pytest.raises(ValueError, match="device tensor"):
        hs.hisparse_swap_in(**_args(miss_counts=torch.zeros(B, dtype=torch.int32),
                                    pool_rows=torch.zeros((R, ctx), dtype=torch.int64)))


def test_scatter_rejects_more_locations_than_source_rows():
    with pytest.raises(ValueError, match="loc has"):
        hs.store_kv_scatter(src=torch.zeros((3, 8), dtype=torch.uint8),
                            dst=torch.zeros((9, 8), dtype=torch.uint8),
                            loc=torch.zeros(4, dtype=torch.int64))
    with pytest.raises(ValueError, match="row_bytes"):
        hs.store_kv_scatter(src=torch.zeros((3, 8), dtype=torch.uint8),
                            dst=torch.zeros((9, 4), dtype=torch.uint8),
                            loc=torch.zeros(3, dtype=torch.int64))


def test_state_reset_rejects_mismatched_rows():
    with pytest.raises(ValueError):
        hs.hisparse_state_reset(slot_tokens=torch.zeros((R, S_r), dtype=torch.int32),
                                lru=torch.zeros((R + 1, H), dtype=torch.int16),
                                rows=torch.zeros(2, dtype=torch.int64))


def test_prepared_call_rejects_step_arguments_and_unknown_entries():
    import sparse_attention_kv_hisparse_amd as hs
    with pytest.raises(ValueError, match="given per call"):
        hs.SwapInCall(topk=torch.zeros((1, 1), dtype=torch.int32))
    with pytest.raises(ValueError, match="unknown entry"):
        hs.SwapInCall(entry="hisparse_something")
    with pytest.raises(ValueError, match="no workspace"):
        hs.SwapInCall(entry="hisparse_swap_in_noalloc", workspace=torch.zeros(8, dtype=torch.uint8))
