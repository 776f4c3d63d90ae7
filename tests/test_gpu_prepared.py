"""SwapInCall (arguments checked once, per-step tensors per call) against
plain hisparse_swap_in calls: outputs, miss counts, state and the whole hot
buffer equal after every step; host and HBM pools, the split pair, and the
allocation-free entry; a step tensor of the wrong shape is refused before
anything is enqueued."""

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


@pytest.mark.parametrize("kind,entries", [
    ("host", ("hisparse_swap_in",)), ("device", ("hisparse_swap_in",)),
    ("host", ("hisparse_resolve", "hisparse_gather_compact")),
    ("device", ("hisparse_swap_in_noalloc",))], ids=["host", "device", "host_split", "device_noalloc"])
def test_prepared_call_matches_plain_calls(kind, entries):
    import sparse_attention_kv_hisparse_amd as hs
    cfg = gen.SwapConfig("prepared", B=4, H=300, K=120, ctx=2000, row_bytes=656, steps=5, rho=0.6,
                         dist="uniform", pool_kind=kind, seed=91)
    print(f"  prepared call: pool={kind} entries={entries}", flush=True)
    pool = wdev.make_pool(cfg)
    p_st = wdev.DeviceSwapState(cfg)
    e_st = wdev.DeviceSwapState(cfg)
    rows = torch.arange(cfg.B, dtype=torch.int64, device="cuda")
    calls = []
    for entry in entries:
        kw = dict(slot_tokens=p_st.slot_tokens, lru=p_st.lru, pool=pool, hot=p_st.hot,
                  out_rows=p_st.out, ctx_stride=cfg.ctx, miss_counts=p_st.counts)
        if entry != "hisparse_swap_in_noalloc":
            kw["workspace"] = p_st.ws
        calls.append(hs.SwapInCall(entry=entry, **kw))
    with pytest.raises(ValueError):
        calls[0](torch.zeros((cfg.B + 1, cfg.K), dtype=torch.int32, device="cuda"), rows,
                 torch.zeros(cfg.B, dtype=torch.int64, device="cuda"))
    for t, topk in enumerate(gen.topk_trace(cfg)):
        tk = torch.as_tensor(topk).cuda()
        seq = torch.as_tensor(gen.seq_lens(cfg, t)).cuda()
        for c in calls:
            c(tk, rows, seq)
        hs.hisparse_swap_in(topk=tk, req_rows=rows, seq_lens=seq, slot_tokens=e_st.slot_tokens,
                            lru=e_st.lru, pool=pool, hot=e_st.hot, out_rows=e_st.out,
                            ctx_stride=cfg.ctx, workspace=e_st.ws, miss_counts=e_st.counts)
        torch.cuda.synchronize()
        for name, a, b in (("out_rows", p_st.out, e_st.out), ("miss_counts", p_st.counts, e_st.counts),
                           ("slot_tokens", p_st.slot_tokens, e_st.slot_tokens),
                           ("lru", p_st.lru, e_st.lru), ("hot buffer", p_st.hot, e_st.hot)):
            assert torch.equal(a, b), f"step {t}: {name} differs from the plain call"
