"""Plan replay on index-sharing layers (hisparse_gather_compact_layers) and the
miss_mask output, against the oracle.

* A resolve on layer 0 followed by one replay launch over L layers must leave
  every layer's hot buffer as the oracle's swap-in (layer 0) plus its replay of
  the same plan (the other layers), with outputs, state, counts and miss_mask
  equal, on every step of a trace; host and device pools, 16- and 4-byte copy
  paths, and more layers than the kernel stages in LDS.
* A hand-built plan written into the workspace through its published layout
  exercises the entry rules: counts clamped to [0, K], negative pool rows and
  out-of-range hot rows skipped, pool rows past the end zero-filled.
"""

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


def _log(msg):
    print(msg, flush=True)


def _np(t):
    return t.cpu().numpy() if t.is_cuda else t.numpy()


CASES = {
    "host_3_layers": (gen.SwapConfig("plan_host", B=5, H=300, K=120, ctx=2000, row_bytes=656,
                                     steps=5, rho=0.6, dist="uniform", pool_kind="host", seed=41), 3),
    "device_132B_4_layers": (gen.SwapConfig("plan_dev", B=6, H=256, K=200, ctx=1500, row_bytes=132,
                                            steps=4, rho=0.5, dist="uniform", pool_kind="device",
                                            seed=42), 4),
    "host_300_layers": (gen.SwapConfig("plan_many", B=2, H=16, K=8, ctx=64, row_bytes=16, steps=4,
                                       rho=0.5, dist="uniform", pool_kind="host", seed=43), 300),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_replay_layers_matches_oracle(name):
    import sparse_attention_kv_hisparse_amd as hs
    cfg, L = CASES[name]
    _log(f"  plan replay {name}: B={cfg.B} K={cfg.K} H={cfg.H} rb={cfg.row_bytes} layers={L}")
    pools = [wdev.make_pool(cfg.with_(seed=cfg.seed + 1000 * l)) for l in range(L)]
    pools_np = [_np(p) for p in pools]
    st = wdev.DeviceSwapState(cfg)
    hot_nrows = st.hot.shape[0]
    hots = [st.hot] + [torch.zeros_like(st.hot) for _ in range(L - 1)]
    pool_ptrs = torch.tensor([p.data_ptr() for p in pools], dtype=torch.int64, device="cuda")
    hot_ptrs = torch.tensor([h.data_ptr() for h in hots], dtype=torch.int64, device="cuda")
    mask = torch.full((cfg.B, cfg.K), 7, dtype=torch.int32, device="cuda")
    o_tok, o_lru = gen.initial_state(cfg)
    o_hots = [np.zeros((hot_nrows, cfg.row_bytes), np.uint8) for _ in range(L)]
    rows = np.arange(cfg.B, dtype=np.int64)
    for t, topk in enumerate(gen.topk_trace(cfg)):
        seq = gen.seq_lens(cfg, t)
        hs.hisparse_resolve(topk=torch.as_tensor(topk).cuda(), req_rows=torch.as_tensor(rows).cuda(),
                            seq_lens=torch.as_tensor(seq).cuda(), slot_tokens=st.slot_tokens,
                            lru=st.lru, pool=pools[0], hot=hots[0], out_rows=st.out,
                            ctx_stride=cfg.ctx, workspace=st.ws, miss_counts=st.counts,
                            miss_mask=mask)
        hs.hisparse_gather_compact_layers(workspace=st.ws, B=cfg.B, K=cfg.K,
                                          pool_layer_ptrs=pool_ptrs, pool_nrows=cfg.pool_nrows,
                                          hot_layer_ptrs=hot_ptrs, hot_nrows=hot_nrows,
                                          row_bytes=cfg.row_bytes)
        o_out, o_cnt, plan = oracle.swap_in(topk=topk, req_rows=rows, seq_lens=seq, slot_tokens=o_tok,
                                            lru=o_lru, pool=pools_np[0], hot=o_hots[0],
                                            ctx_stride=cfg.ctx, plan=True)
        oracle.gather_compact_layers(plan["count"], plan["src"], plan["dst"], pools_np[1:], o_hots[1:])
        torch.cuda.synchronize()
        assert np.array_equal(_np(st.out), o_out), f"step {t}: out_rows"
        assert np.array_equal(_np(st.counts), o_cnt), f"step {t}: miss_counts"
        assert np.array_equal(_np(mask), plan["miss_mask"]), f"step {t}: miss_mask"
        assert np.array_equal(_np(st.slot_tokens), o_tok), f"step {t}: slot_tokens"
        assert np.array_equal(_np(st.lru), o_lru), f"step {t}: lru"
        for l in range(L):
            assert np.array_equal(_np(hots[l]), o_hots[l]), f"step {t}: hot buffer of layer {l}"


def _write_plan(ws, lay, count, src, dst):
    B, K = src.shape
    buf = ws.cpu().numpy()
    buf[lay["count"]:lay["count"] + 4 * B] = count.astype(np.int32).view(np.uint8)
    buf[lay["src"]:lay["src"] + 8 * B * K] = src.astype(np.int64).reshape(-1).view(np.uint8)
    buf[lay["dst"]:lay["dst"] + 4 * B * K] = dst.astype(np.int32).reshape(-1).view(np.uint8)
    ws.copy_(torch.as_tensor(buf))


@pytest.mark.parametrize("rb,seed", [(64, 0), (20, 1)])
def test_replay_entry_rules(rb, seed):
    """count clamping, skipped entries and zero-filled rows, on 2 layers."""
    import sparse_attention_kv_hisparse_amd as hs
    rng = np.random.default_rng(seed)
    B, K, L, P, Hn = 4, 16, 2, 50, 80
    count = np.array([K + 5, -3, 7, K], np.int32)
    src = rng.integers(-4, P + 6, size=(B, K)).astype(np.int64)
    dst = (rng.permutation(Hn + 8)[:B * K].reshape(B, K) - 4).astype(np.int32)
    lay = hs.swap_in_workspace_layout(B, K)
    ws = torch.zeros(lay["total"], dtype=torch.uint8, device="cuda")
    _write_plan(ws, lay, count, src, dst)
    pools = [torch.as_tensor(rng.integers(0, 256, size=(P, rb), dtype=np.uint8)).pin_memory()
             for _ in range(L)]
    hots0 = [rng.integers(0, 256, size=(Hn, rb), dtype=np.uint8) for _ in range(L)]
    hots = [torch.as_tensor(h).cuda() for h in hots0]
    hs.hisparse_gather_compact_layers(
        workspace=ws, B=B, K=K,
        pool_layer_ptrs=torch.tensor([p.data_ptr() for p in pools], dtype=torch.int64, device="cuda"),
        pool_nrows=P,
        hot_layer_ptrs=torch.tensor([h.data_ptr() for h in hots], dtype=torch.int64, device="cuda"),
        hot_nrows=Hn, row_bytes=rb)
    want = [h.copy() for h in hots0]
    zeroed = oracle.gather_compact_layers(count, src, dst, [p.numpy() for p in pools], want)
    assert zeroed > 0
    torch.cuda.synchronize()
    for l in range(L):
        assert np.array_equal(_np(hots[l]), want[l]), f"layer {l}"
