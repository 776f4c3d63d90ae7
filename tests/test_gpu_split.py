"""hisparse_resolve + hisparse_gather_compact equal hisparse_swap_in, and the
miss list they hand over (read through hs_swap_in_workspace_layout) is the one
the oracle implies: misses in ascending top-k order, (pool row, hot row) each."""

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
    torch.cuda.set_device(0)


@pytest.mark.parametrize("cfg", [
    gen.SwapConfig("split", B=5, H=300, K=120, ctx=2000, row_bytes=656, steps=6, rho=0.6,
                   dist="uniform", pool_kind="host", seed=31),
    gen.DEVPOOL.with_(B=8, steps=4),
    # more requests than CUs: the host-pool copy's one-workgroup-per-CU grid
    gen.SwapConfig("split_many", B=400, H=64, K=30, ctx=300, row_bytes=656, steps=4, rho=0.5,
                   dist="uniform", pool_kind="host", seed=32),
], ids=["host", "device", "host_many_requests"])
def test_resolve_then_gather_matches_oracle(cfg):
    import sparse_attention_kv_hisparse_amd as hs
    pool = wdev.make_pool(cfg)
    pool_np = pool.cpu().numpy() if pool.is_cuda else pool.numpy()
    st = wdev.DeviceSwapState(cfg)
    lay = hs.swap_in_workspace_layout(cfg.B, cfg.K)
    assert lay["total"] == st.ws.numel()
    o_tok, o_lru = gen.initial_state(cfg)
    o_hot = np.zeros((cfg.R * cfg.S_r, cfg.row_bytes), np.uint8)
    rows = np.arange(cfg.B, dtype=np.int64)
    # uint64 counters: only the resolve adds to them, the gather leaves them alone
    stats = torch.zeros(2, dtype=torch.uint64).cuda()
    o_stats = np.zeros(2, np.uint64)
    for t, topk in enumerate(gen.topk_trace(cfg)):
        seq = gen.seq_lens(cfg, t)
        kw = dict(topk=torch.as_tensor(topk).cuda(), req_rows=torch.as_tensor(rows).cuda(),
                  seq_lens=torch.as_tensor(seq).cuda(), slot_tokens=st.slot_tokens, lru=st.lru,
                  pool=pool, hot=st.hot, out_rows=st.out, ctx_stride=cfg.ctx, workspace=st.ws,
                  miss_counts=st.counts, stats=stats)
        hs.hisparse_resolve(**kw)
        torch.cuda.synchronize()
        ws = st.ws.cpu().numpy()
        count = ws[lay["count"]:lay["count"] + 4 * cfg.B].view(np.int32)
        src = ws[lay["src"]:lay["src"] + 8 * cfg.B * cfg.K].view(np.int64).reshape(cfg.B, cfg.K)
        dst = ws[lay["dst"]:lay["dst"] + 4 * cfg.B * cfg.K].view(np.int32).reshape(cfg.B, cfg.K)
        tok_before = o_tok.copy()
        hs.hisparse_gather_compact(**kw)
        o_out, o_cnt = oracle.swap_in(topk=topk, req_rows=rows, seq_lens=seq, slot_tokens=o_tok,
                                      lru=o_lru, pool=pool_np, hot=o_hot, ctx_stride=cfg.ctx,
                                      stats=o_stats)
        torch.cuda.synchronize()
        assert np.array_equal(stats.view(torch.int64).cpu().numpy().astype(np.uint64), o_stats)
        assert np.array_equal(st.out.cpu().numpy(), o_out)
        assert np.array_equal(st.counts.cpu().numpy(), o_cnt)
        assert np.array_equal(st.slot_tokens.cpu().numpy(), o_tok)
        assert np.array_equal(st.lru.cpu().numpy(), o_lru)
        assert np.array_equal(st.hot.cpu().numpy(), o_hot)
        assert np.array_equal(count, o_cnt)
        for b in range(cfg.B):
            L = int(seq[b])
            resident = set(int(x) for x in tok_before[b, :cfg.H] if x >= 0)
            want = [(b * cfg.ctx + int(x), int(o_out[b, i])) for i, x in enumerate(topk[b])
                    if 0 <= x < L - 1 and int(x) not in resident]
            got = list(zip(src[b, :count[b]].tolist(), dst[b, :count[b]].tolist()))
            assert got == want
