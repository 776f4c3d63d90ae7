"""The swap-in under HIP graph capture.

One call is captured into a graph (torch.cuda.graph, which captures on its own
stream) over fixed input buffers; each decode step then copies its top-k ids
and sequence lengths into those buffers eagerly, replays the graph and
synchronizes. A second copy of the state runs the same steps eagerly through
hisparse_swap_in, and after every replay the graph's outputs, miss counts,
slot tokens, LRU rows and whole hot buffer must equal the eager ones byte for
byte. The library records no memset or copy nodes: a call is its kernel
launches only. Host pools (one fused launch) and an HBM pool (resolve and
copy), through hisparse_swap_in and through hisparse_swap_in_noalloc."""

import numpy as np
import pytest
import torch

from workloads import device as wdev
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import sparse_attention_kv_hisparse_amd as hs
    hs.load()
    torch.cuda.set_device(0)


@pytest.mark.parametrize("kind,entry", [("host", "hisparse_swap_in"), ("device", "hisparse_swap_in"),
                                        ("host", "hisparse_swap_in_noalloc")],
                         ids=["host", "device", "host_noalloc"])
def test_graph_replays_match_eager_calls(kind, entry):
    import sparse_attention_kv_hisparse_amd as hs
    cfg = gen.SwapConfig("graph", B=3, H=96, K=40, ctx=600, row_bytes=656, steps=6, rho=0.6,
                         dist="uniform", pool_kind=kind, seed=81)
    print(f"  graph capture: pool={kind} entry={entry}", flush=True)
    pool = wdev.make_pool(cfg)
    g_st = wdev.DeviceSwapState(cfg)     # state the graph updates
    e_st = wdev.DeviceSwapState(cfg)     # state the eager calls update
    rows = torch.arange(cfg.B, dtype=torch.int64, device="cuda")
    topk_in = torch.zeros((cfg.B, cfg.K), dtype=torch.int32, device="cuda")
    seq_in = torch.full((cfg.B,), cfg.ctx, dtype=torch.int64, device="cuda")
    g_counts = torch.zeros(cfg.B, dtype=torch.int32, device="cuda")
    fn = getattr(hs, entry)

    def graph_call(st):
        kw = {} if entry == "hisparse_swap_in_noalloc" else {"workspace": st.ws}
        fn(topk=topk_in, req_rows=rows, seq_lens=seq_in, slot_tokens=st.slot_tokens, lru=st.lru,
           pool=pool, hot=st.hot, out_rows=st.out, ctx_stride=cfg.ctx, miss_counts=g_counts, **kw)

    # Warm-up outside capture (the library's one-time device set-up): every
    # row is padding, so no state changes.
    pad = torch.zeros(1, dtype=torch.int32, device="cuda")
    kw = {} if entry == "hisparse_swap_in_noalloc" else {"workspace": g_st.ws}
    fn(topk=topk_in, req_rows=rows, seq_lens=seq_in, slot_tokens=g_st.slot_tokens, lru=g_st.lru,
       pool=pool, hot=g_st.hot, out_rows=g_st.out, ctx_stride=cfg.ctx, miss_counts=g_counts,
       num_real=pad, **kw)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graph_call(g_st)
    torch.cuda.synchronize()

    for t, topk in enumerate(gen.topk_trace(cfg)):
        seq = gen.seq_lens(cfg, t)
        topk_in.copy_(torch.as_tensor(topk))
        seq_in.copy_(torch.as_tensor(seq))
        torch.cuda.synchronize()
        g.replay()
        hs.hisparse_swap_in(topk=torch.as_tensor(topk).cuda(), req_rows=rows,
                            seq_lens=torch.as_tensor(seq).cuda(), slot_tokens=e_st.slot_tokens,
                            lru=e_st.lru, pool=pool, hot=e_st.hot, out_rows=e_st.out,
                            ctx_stride=cfg.ctx, workspace=e_st.ws, miss_counts=e_st.counts)
        torch.cuda.synchronize()
        for name, a, b in (("out_rows", g_st.out, e_st.out), ("miss_counts", g_counts, e_st.counts),
                           ("slot_tokens", g_st.slot_tokens, e_st.slot_tokens),
                           ("lru", g_st.lru, e_st.lru), ("hot buffer", g_st.hot, e_st.hot)):
            assert torch.equal(a, b), f"replay {t}: {name} differs from the eager call"
        assert int(e_st.counts.sum()) > 0 or t > 0
