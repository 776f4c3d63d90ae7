"""hisparse_swap_in_noalloc (the allocation-free entry point, for callers that
cannot allocate device memory) against hisparse_swap_in with a workspace, bit
for bit: two calls in a row, the second with a smaller batch and top_k, from a
pinned-host pool (the fused resolve + copy kernel) and from an HBM pool
(resolve, then the copy kernel reading the list back from the fixed array).
Both sides run on their own copies of the same state; outputs, counts, slot
tokens, LRU rows, counters and the whole hot buffer must match, and the oracle
checks the same calls. A batch whose miss list exceeds the fixed array is
rejected with HS_ERANGE and changes nothing."""

import numpy as np
import pytest
import torch

import oracle
from workloads import device as wdev
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import sparse_attention_kv_hisparse_amd as hs
    hs.load()
    assert torch.cuda.is_available()
    torch.cuda.set_device(0)


class _Side:
    def __init__(self, cfg, R):
        self.st = wdev.DeviceSwapState(cfg, R=R)
        self.stats = torch.zeros(2, dtype=torch.int64, device="cuda")


@pytest.mark.parametrize("kind", ["host", "device"])
def test_noalloc_matches_workspace_entry_point(kind):
    import sparse_attention_kv_hisparse_amd as hs
    # first call: 64 requests x 2048 ids (a 1.5 MiB miss list); second: 8 x 1000
    cfg = gen.SwapConfig("noalloc_" + kind, B=64, H=4096, K=2048, ctx=8192, row_bytes=656,
                         steps=2, rho=0.6, dist="uniform", pool_kind=kind, seed=4242)
    print(f"  noalloc {kind}: pool {cfg.pool_nrows} rows", flush=True)
    pool = wdev.make_pool(cfg)
    pool_np = pool.cpu().numpy() if pool.is_cuda else pool.numpy()
    R = cfg.B
    ws_side, na_side = _Side(cfg, R), _Side(cfg, R)
    o_tok, o_lru = gen.initial_state(R, cfg.H, cfg.S_r)
    o_hot = np.zeros((R * cfg.S_r, cfg.row_bytes), np.uint8)
    o_stats = np.zeros(2, np.uint64)
    trace = list(gen.topk_trace(cfg, 2))
    rng = np.random.default_rng(5)
    for call, (B, K) in enumerate([(64, 2048), (8, 1000)]):
        rows = rng.permutation(R)[:B].astype(np.int64)
        topk = np.ascontiguousarray(trace[call][rows, :K])
        seq = gen.seq_lens(cfg, call)[:B]
        print(f"  noalloc {kind} call {call}: B={B} K={K}", flush=True)
        common = dict(topk=torch.as_tensor(topk).cuda(), req_rows=torch.as_tensor(rows).cuda(),
                      seq_lens=torch.as_tensor(seq).cuda(), pool=pool, ctx_stride=cfg.ctx)
        outs = []
        for side, noalloc in ((ws_side, False), (na_side, True)):
            out = torch.full((B, K), -9, dtype=torch.int32, device="cuda")
            cnt = torch.full((B,), -9, dtype=torch.int32, device="cuda")
            kw = dict(common, slot_tokens=side.st.slot_tokens, lru=side.st.lru, hot=side.st.hot,
                      out_rows=out, miss_counts=cnt, stats=side.stats)
            if noalloc:
                hs.hisparse_swap_in_noalloc(**kw)
            else:
                hs.hisparse_swap_in(workspace=side.st.ws, **kw)
            outs.append((out, cnt))
        o_out, o_cnt = oracle.swap_in(topk=topk, req_rows=rows, seq_lens=seq, slot_tokens=o_tok,
                                      lru=o_lru, pool=pool_np, hot=o_hot, ctx_stride=cfg.ctx,
                                      stats=o_stats)
        torch.cuda.synchronize()
        (w_out, w_cnt), (n_out, n_cnt) = outs
        assert torch.equal(n_out, w_out), f"call {call}: out_rows"
        assert torch.equal(n_cnt, w_cnt), f"call {call}: miss_counts"
        assert torch.equal(na_side.st.slot_tokens, ws_side.st.slot_tokens), f"call {call}: slot_tokens"
        assert torch.equal(na_side.st.lru, ws_side.st.lru), f"call {call}: lru"
        assert torch.equal(na_side.stats, ws_side.stats), f"call {call}: stats"
        assert torch.equal(na_side.st.hot, ws_side.st.hot), f"call {call}: hot buffer"
        assert np.array_equal(n_out.cpu().numpy(), o_out), f"call {call}: out_rows vs oracle"
        assert np.array_equal(n_cnt.cpu().numpy(), o_cnt), f"call {call}: counts vs oracle"
        assert np.array_equal(na_side.st.hot.cpu().numpy(), o_hot), f"call {call}: hot vs oracle"
        assert int(o_cnt.sum()) > 0


def test_noalloc_rejects_lists_beyond_its_array():
    import sparse_attention_kv_hisparse_amd as hs
    from sparse_attention_kv_hisparse_amd._lib import HS_NOALLOC_SCRATCH_BYTES, HisparseError
    B, K, H = 256, 2048, 2048        # a 6 MiB miss list
    assert hs.swap_in_workspace_bytes(B, K) > HS_NOALLOC_SCRATCH_BYTES
    cfg = gen.SwapConfig("noalloc_big", B=B, H=H, K=K, ctx=4096, row_bytes=16, steps=1, rho=0.5,
                         dist="uniform", pool_kind="device", seed=1)
    st = wdev.DeviceSwapState(cfg)
    pool = torch.zeros((cfg.pool_nrows, 16), dtype=torch.uint8, device="cuda")
    st.out.fill_(7)
    before = (st.slot_tokens.clone(), st.lru.clone(), st.out.clone())
    topk = torch.arange(K, dtype=torch.int32, device="cuda").repeat(B, 1)
    with pytest.raises(HisparseError) as e:
        hs.hisparse_swap_in_noalloc(topk=topk, req_rows=torch.arange(B, device="cuda"),
                                    seq_lens=torch.full((B,), 4096, dtype=torch.int64, device="cuda"),
                                    slot_tokens=st.slot_tokens, lru=st.lru, pool=pool, hot=st.hot,
                                    out_rows=st.out, ctx_stride=cfg.ctx)
    assert e.value.status == -2
    torch.cuda.synchronize()
    for a, b in zip(before, (st.slot_tokens, st.lru, st.out)):
        assert torch.equal(a, b)
