"""Non-MLA (K+V) variants on the GPU against the oracle, bit for bit.

* hisparse_swap_in with a V pool and V hot buffer: host pool (fused copy),
  device pool (wide copy kernel), 132-byte rows (4-byte path), and the split
  API (resolve, then gather_compact) -- outputs, state, counts, the K hot
  buffer and the V hot buffer after every step.
* transfer_kv_all_layer in both directions, including more layers than the
  kernel stages in LDS.
* store_kv_cache with a different row stride on each of its four arrays.
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


SWAP_CASES = {
    "host_fused": gen.SwapConfig("kv_host", B=6, H=320, K=160, ctx=2400, row_bytes=1024, steps=5,
                                 rho=0.6, dist="uniform", pool_kind="host", seed=51),
    "device": gen.SwapConfig("kv_dev", B=8, H=512, K=256, ctx=3000, row_bytes=512, steps=4, rho=0.5,
                             dist="uniform", pool_kind="device", seed=52),
    "host_132B": gen.SwapConfig("kv_132", B=4, H=300, K=200, ctx=1500, row_bytes=132, steps=4,
                                rho=0.5, dist="zipf", pool_kind="host", seed=53),
}


@pytest.mark.parametrize("split", [False, True], ids=["swap_in", "resolve_gather"])
@pytest.mark.parametrize("name", sorted(SWAP_CASES))
def test_kv_swap_in_matches_oracle(name, split):
    import sparse_attention_kv_hisparse_amd as hs
    cfg = SWAP_CASES[name]
    _log(f"  kv swap-in {name} split={split}: B={cfg.B} K={cfg.K} H={cfg.H} rb={cfg.row_bytes}")
    pool = wdev.make_pool(cfg)
    pool_v = wdev.make_pool(cfg.with_(seed=cfg.seed + 777))
    pool_np, pool_v_np = _np(pool), _np(pool_v)
    st = wdev.DeviceSwapState(cfg)
    hot_v = torch.zeros_like(st.hot)
    o_tok, o_lru = gen.initial_state(cfg)
    o_hot = np.zeros(tuple(st.hot.shape), np.uint8)
    o_hot_v = np.zeros_like(o_hot)
    rows = np.arange(cfg.B, dtype=np.int64)
    for t, topk in enumerate(gen.topk_trace(cfg)):
        seq = gen.seq_lens(cfg, t)
        kw = dict(topk=torch.as_tensor(topk).cuda(), req_rows=torch.as_tensor(rows).cuda(),
                  seq_lens=torch.as_tensor(seq).cuda(), slot_tokens=st.slot_tokens, lru=st.lru,
                  pool=pool, hot=st.hot, out_rows=st.out, ctx_stride=cfg.ctx, workspace=st.ws,
                  miss_counts=st.counts, pool_v=pool_v, hot_v=hot_v)
        if split:
            hs.hisparse_resolve(**kw)
            hs.hisparse_gather_compact(**kw)
        else:
            hs.hisparse_swap_in(**kw)
        o_out, o_cnt = oracle.swap_in(topk=topk, req_rows=rows, seq_lens=seq, slot_tokens=o_tok,
                                      lru=o_lru, pool=pool_np, hot=o_hot, ctx_stride=cfg.ctx,
                                      pool_v=pool_v_np, hot_v=o_hot_v)
        torch.cuda.synchronize()
        assert np.array_equal(_np(st.out), o_out), f"step {t}: out_rows"
        assert np.array_equal(_np(st.counts), o_cnt), f"step {t}: miss_counts"
        assert np.array_equal(_np(st.slot_tokens), o_tok), f"step {t}: slot_tokens"
        assert np.array_equal(_np(st.lru), o_lru), f"step {t}: lru"
        assert np.array_equal(_np(st.hot), o_hot), f"step {t}: K hot buffer"
        assert np.array_equal(_np(hot_v), o_hot_v), f"step {t}: V hot buffer"


def _layers(L, rows, rb, where, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    host = torch.randint(0, 256, (L * rows, rb), dtype=torch.uint8, generator=g)
    backing = host.pin_memory() if where == "host" else host.cuda()
    layers = [backing[l * rows:(l + 1) * rows] for l in range(L)]
    ptrs = torch.tensor([x.data_ptr() for x in layers], dtype=torch.int64, device="cuda")
    return layers, ptrs


@pytest.mark.parametrize("L,rows,rb,n,src_kind,dst_kind", [
    (3, 400, 656, 300, "host", "device"),
    (4, 300, 1024, 250, "device", "host"),
    (2, 200, 132, 150, "device", "device"),       # 4-byte path
    (150, 40, 64, 30, "host", "device"),          # 300 streams: more than are staged in LDS
])
@pytest.mark.parametrize("host_link", [False, True], ids=["hbm_launch", "host_link_launch"])
def test_transfer_kv_all_layer(L, rows, rb, n, src_kind, dst_kind, host_link):
    import sparse_attention_kv_hisparse_amd as hs
    _log(f"  transfer_kv L={L} rows={rows} rb={rb} n={n} {src_kind}->{dst_kind}")
    ks, ksp = _layers(L, rows, rb, src_kind, 1)
    vs, vsp = _layers(L, rows, rb, src_kind, 2)
    kd, kdp = _layers(L, rows, rb, dst_kind, 3)
    vd, vdp = _layers(L, rows, rb, dst_kind, 4)
    rng = np.random.default_rng(L + rows)
    si = rng.integers(-2, rows + 2, n).astype(np.int64)      # a few out of range: skipped
    di = (rng.permutation(rows + 4)[:n] - 2).astype(np.int64)
    want_k = [_np(x).copy() for x in kd]
    want_v = [_np(x).copy() for x in vd]
    oracle.transfer_kv_all_layer([_np(x) for x in ks], [_np(x) for x in vs], want_k, want_v, si, di)
    hs.transfer_kv_all_layer(k_src_layer_ptrs=ksp, v_src_layer_ptrs=vsp, k_dst_layer_ptrs=kdp,
                             v_dst_layer_ptrs=vdp, src_idx=torch.as_tensor(si).cuda(),
                             dst_idx=torch.as_tensor(di).cuda(), row_bytes=rb, src_nrows=rows,
                             dst_nrows=rows, host_link=host_link)
    torch.cuda.synchronize()
    for l in range(L):
        assert np.array_equal(_np(kd[l]), want_k[l]), f"K layer {l}"
        assert np.array_equal(_np(vd[l]), want_v[l]), f"V layer {l}"


@pytest.mark.parametrize("n,rb,strides,dst_rows", [
    (100, 656, (656, 1312, 672, 656), 300),
    (33, 132, (132, 136, 132, 140), 50),          # 4-byte path
    (500, 1024, (2048, 1024, 1024, 4096), 700),
])
def test_store_kv_cache(n, rb, strides, dst_rows):
    import sparse_attention_kv_hisparse_amd as hs
    rng = np.random.default_rng(n)
    ks_, vs_, kd_, vd_ = strides
    k_src = torch.as_tensor(rng.integers(0, 256, (n, ks_), dtype=np.uint8)).cuda()[:, :rb]
    v_src = torch.as_tensor(rng.integers(0, 256, (n, vs_), dtype=np.uint8)).cuda()[:, :rb]
    k_dst = torch.as_tensor(rng.integers(0, 256, (dst_rows, kd_), dtype=np.uint8)).cuda()[:, :rb]
    v_dst = torch.as_tensor(rng.integers(0, 256, (dst_rows, vd_), dtype=np.uint8)).cuda()[:, :rb]
    loc = (rng.permutation(dst_rows + 10)[:n] - 5).astype(np.int64)
    kdn, vdn = _np(k_dst).copy(), _np(v_dst).copy()
    oracle.store_kv_cache(_np(k_src), _np(v_src), kdn, vdn, loc)
    hs.store_kv_cache(k_src=k_src, v_src=v_src, k_dst=k_dst, v_dst=v_dst, loc=torch.as_tensor(loc).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(_np(k_dst), kdn)
    assert np.array_equal(_np(v_dst), vdn)


def test_kv_swap_in_full_size():
    """The non-MLA decode workload at full size (B=32, H=4096, K=2048, 32,768-token
    contexts, 1024-byte K and V rows in two 1 GiB pinned pools): the cold step and
    three steady steps, everything compared with the oracle."""
    import sparse_attention_kv_hisparse_amd as hs
    cfg = gen.KV_DECODE
    _log(f"  kv full size: B={cfg.B} K={cfg.K} H={cfg.H} rb={cfg.row_bytes}, building pools")
    pool = wdev.make_pool(cfg)
    pool_v = wdev.make_pool(cfg.with_(seed=cfg.seed + 777))
    st = wdev.DeviceSwapState(cfg)
    hot_v = torch.zeros_like(st.hot)
    o_tok, o_lru = gen.initial_state(cfg)
    o_hot = np.zeros(tuple(st.hot.shape), np.uint8)
    o_hot_v = np.zeros_like(o_hot)
    rows = np.arange(cfg.B, dtype=np.int64)
    for t, topk in enumerate(gen.topk_trace(cfg, 4)):
        seq = gen.seq_lens(cfg, t)
        hs.hisparse_swap_in(topk=torch.as_tensor(topk).cuda(), req_rows=torch.as_tensor(rows).cuda(),
                            seq_lens=torch.as_tensor(seq).cuda(), slot_tokens=st.slot_tokens,
                            lru=st.lru, pool=pool, hot=st.hot, out_rows=st.out, ctx_stride=cfg.ctx,
                            workspace=st.ws, miss_counts=st.counts, pool_v=pool_v, hot_v=hot_v)
        o_out, o_cnt = oracle.swap_in(topk=topk, req_rows=rows, seq_lens=seq, slot_tokens=o_tok,
                                      lru=o_lru, pool=pool.numpy(), hot=o_hot, ctx_stride=cfg.ctx,
                                      pool_v=pool_v.numpy(), hot_v=o_hot_v)
        torch.cuda.synchronize()
        _log(f"  kv full size step {t}: {int(o_cnt.sum())} misses")
        assert np.array_equal(_np(st.out), o_out), f"step {t}: out_rows"
        assert np.array_equal(_np(st.counts), o_cnt), f"step {t}: miss_counts"
        assert np.array_equal(_np(st.slot_tokens), o_tok), f"step {t}: slot_tokens"
        assert np.array_equal(_np(st.lru), o_lru), f"step {t}: lru"
        assert np.array_equal(_np(st.hot), o_hot), f"step {t}: K hot buffer"
        assert np.array_equal(_np(hot_v), o_hot_v), f"step {t}: V hot buffer"
