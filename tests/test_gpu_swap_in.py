"""GPU parity of hisparse_swap_in against the CPU oracle, bit for bit.

Full-size traces of the five workloads (tiny; DeepSeek-V3.2-like pinned-host
pool; device pool; cold/adversarial at 1152 B and 132 B rows), plus edge
cases: padding rows, permuted and sparse state rows, slot-row and pool-row
tables, invalid ids, K == H, ragged H and K, the 4-byte copy path, strided
top-k rows, hash clustering, empty calls and exact replays.
"""

import numpy as np
import pytest
import torch

from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import sparse_attention_kv_hisparse_amd as hs
    hs.load()
    assert torch.cuda.is_available()
    torch.cuda.set_device(0)


def _harness():
    import gpu_harness
    return gpu_harness


def test_tiny_trace_with_invariants():
    h = _harness()
    counts = h.run_trace(gen.TINY, check_invariants=True)
    assert (counts[0] == gen.TINY.K).all()


def test_dsv32_like_host_pool_full():
    h = _harness()
    cfg = gen.DSV32
    counts = h.run_trace(cfg)
    assert (counts[0] <= cfg.K).all() and (counts[0] >= cfg.K - 1).all()


def test_device_pool_full():
    h = _harness()
    cfg = gen.DEVPOOL
    counts = h.run_trace(cfg)
    # cold step: every id misses except the newest token when a row drew it
    assert (counts[0] <= cfg.K).all() and (counts[0] >= cfg.K - 1).all()


@pytest.mark.parametrize("cfg", [gen.ADVERSARIAL, gen.ADVERSARIAL_132, gen.ADVERSARIAL_KERNEL_HASH],
                         ids=["1152B", "132B", "kernel_hash_1152B"])
def test_adversarial_full(cfg):
    h = _harness()
    counts = h.run_trace(cfg)
    assert (counts[0] <= cfg.K).all() and (counts[0] >= cfg.K - 1).all()


def _small(**kw):
    base = dict(name="edge", B=3, H=40, K=12, ctx=300, row_bytes=48, steps=6, rho=0.5,
                dist="uniform", pool_kind="host", seed=99)
    base.update(kw)
    return gen.SwapConfig(**base)


@pytest.mark.parametrize("kw", [
    dict(),
    dict(H=64, K=64, ctx=500),                  # K == H, exact wave multiples
    dict(H=1000, K=999, ctx=3000, B=2),         # ragged, K just below H
    dict(H=5000, K=3000, ctx=9000, B=2),        # several LDS scan words, H > 4096
    dict(H=1, K=1, ctx=50, B=4),                # degenerate sizes
    dict(row_bytes=4), dict(row_bytes=132),     # 4-byte path
    dict(row_bytes=1152, pool_kind="device"),
    dict(B=1, H=2048, K=2048, ctx=4096),        # one request, all K = H
    dict(H=16384, K=2048, ctx=40000, B=2, steps=3),   # slot tokens too big to stage in LDS
    dict(H=16384, K=2048, ctx=40000, B=2, steps=3, pool_kind="device"),
    dict(B=600, H=96, K=40, ctx=400, steps=4),        # more requests than CUs (fused copy)
    dict(B=600, H=96, K=40, ctx=400, steps=4, pool_kind="device"),
    # largest sizes the per-request LDS scratch allows (160 KB per workgroup):
    dict(H=32768, K=584, ctx=70000, B=2, steps=3, row_bytes=16),   # H at its maximum
    dict(H=4096, K=4096, ctx=9000, B=2, steps=3, row_bytes=16),    # K at its maximum
    # positions past 65536 take the hashed plans: two classification passes,
    # and K at its maximum there too
    dict(H=5000, K=3000, ctx=70000, B=2),
    dict(H=4096, K=4096, ctx=70000, B=2, steps=3, row_bytes=16),
    # a direct table that fits only with the slot-token row left in HBM
    dict(H=16384, K=2048, ctx=32768, B=2, steps=3),
    # direct tables with the guard-free (exact) tiles past one pass: more LRU
    # positions and slot tokens than one pass of the workgroup stages, and
    # more top-k entries than a wave keeps in registers
    dict(H=8192, K=2048, ctx=16384, B=2, steps=3),
    dict(H=8192, K=4096, ctx=16384, B=2, steps=3, row_bytes=16, pool_kind="device"),
], ids=["base", "K_eq_H", "ragged", "bigH", "degenerate", "rb4", "rb132", "devpool", "single",
        "unstaged_host", "unstaged_dev", "many_host", "many_dev", "max_H", "max_K",
        "hashed_two_passes", "hashed_max_K", "direct_unstaged", "direct_exact_bigH",
        "direct_exact_K4096"])
def test_edge_traces(kw):
    h = _harness()
    cfg = _small(**kw)
    h.run_trace(cfg, check_invariants=cfg.K * cfg.B <= 4096)


def test_padding_permuted_rows_tables_invalid_ids():
    """R > B, permuted state rows, num_real < B, slot_rows/pool_rows tables,
    invalid ids (negative, >= seq_len, >= ctx_stride, pool row out of range)."""
    h = _harness()
    rng = np.random.default_rng(7)
    cfg = _small(B=4, H=30, K=10, ctx=100, row_bytes=32)
    R = 9
    S_r = cfg.S_r
    hot_nrows = R * S_r + 5
    slot_rows = rng.permutation(hot_nrows)[:R * S_r].astype(np.int32).reshape(R, S_r)
    pool_nrows = R * cfg.ctx - 17            # the last ids of the last row have no pool row
    pool_rows = rng.permutation(R * cfg.ctx)[:R * cfg.ctx].astype(np.int64).reshape(R, cfg.ctx)
    run = h.ParityRun(cfg, R=R, req_rows=np.asarray([7, 2, 5, 0], dtype=np.int64),
                      slot_rows=slot_rows, pool_rows=pool_rows, hot_nrows=hot_nrows,
                      pool_nrows=pool_nrows)
    for t in range(10):
        rows, seq, topk = gen.random_case(rng, B=4, R=R, H=cfg.H, K=cfg.K, ctx=cfg.ctx,
                                          n_invalid=int(rng.integers(0, 3)))
        run.req_rows = rows
        num_real = int(rng.integers(1, 5)) if t % 3 == 2 else -1
        run.step(topk, seq, num_real=num_real, check_invariants=True)


def test_state_row_out_of_range_is_padding():
    """State rows 5 and -1 with R = 3: padding. The pool and the hot buffer are
    sized for six state rows, so row 5's ids would have pool rows and hot rows
    in range: only the state-row bound makes them padding."""
    h = _harness()
    cfg = _small(B=3)
    run = h.ParityRun(cfg, R=3, req_rows=np.asarray([0, 5, -1], dtype=np.int64),
                      pool_nrows=6 * cfg.ctx, hot_nrows=6 * cfg.S_r)
    rng = np.random.default_rng(3)
    for _ in range(3):
        _, seq, topk = gen.random_case(rng, B=3, R=3, H=cfg.H, K=cfg.K, ctx=cfg.ctx)
        out, cnt = run.step(topk, seq)
        assert (out[1:] == -1).all() and (cnt[1:] == 0).all()


def test_negative_pool_row_entries_are_invalid():
    """A pool-row table with negative entries: those ids output -1, are not
    copied and are not counted (the pool has spare rows, so a kernel that let
    a negative row through would copy real bytes and differ)."""
    h = _harness()
    rng = np.random.default_rng(21)
    cfg = _small(B=3, H=40, K=12, ctx=120, row_bytes=48)
    R = 3
    pool_rows = rng.permutation(R * cfg.ctx).astype(np.int64).reshape(R, cfg.ctx)
    neg = rng.random(pool_rows.shape) < 0.2
    pool_rows[neg] = -rng.integers(1, 4, int(neg.sum()))
    run = h.ParityRun(cfg, R=R, pool_rows=pool_rows)
    seen_neg = 0
    for t in range(8):
        rows, seq, topk = gen.random_case(rng, B=3, R=R, H=cfg.H, K=cfg.K, ctx=cfg.ctx)
        run.req_rows = rows
        out, _ = run.step(topk, seq, check_invariants=True)
        for b in range(3):
            for i in range(cfg.K):
                t_id = int(topk[b, i])
                if 0 <= t_id < seq[b] and pool_rows[rows[b], t_id] < 0:
                    assert out[b, i] == -1
                    seen_neg += 1
    assert seen_neg > 0


def test_seq_len_past_the_row_stride():
    """seq_len beyond ctx_stride: ids at or past the stride (the newest token
    among them) have no pool row of their request and output -1, although the
    pool has rows there (the next request's); the rest swap in as usual."""
    h = _harness()
    rng = np.random.default_rng(13)
    cfg = _small(B=3, H=40, K=12, ctx=100, row_bytes=16)
    run = h.ParityRun(cfg, R=3, pool_nrows=4 * cfg.ctx)
    L = cfg.ctx + 7
    for _ in range(4):
        seq = np.full(3, L, np.int64)
        rest = np.delete(np.arange(L), cfg.ctx)
        topk = np.stack([np.concatenate([[cfg.ctx], rng.choice(rest, cfg.K - 1, replace=False)])
                         for _ in range(3)]).astype(np.int32)
        out, _ = run.step(topk, seq, check_invariants=True)
        assert (out[:, 0] == -1).all()


def test_strided_topk_rows():
    h = _harness()
    cfg = _small(B=5, H=70, K=33, ctx=400)
    run = h.ParityRun(cfg)
    for t, topk in enumerate(gen.topk_trace(cfg, 4)):
        run.step(topk, gen.seq_lens(cfg, t), topk_pad=11)


def test_misaligned_hot_uses_4byte_path():
    h = _harness()
    cfg = _small(row_bytes=64)
    run = h.ParityRun(cfg, hot_misalign=True)
    for t, topk in enumerate(gen.topk_trace(cfg, 4)):
        run.step(topk, gen.seq_lens(cfg, t))


@pytest.mark.parametrize("K,H,span", [(512, 1024, 200000), (3000, 4096, 600000)],
                         ids=["one_pass", "two_passes"])
def test_clusters_under_the_kernel_hash(K, H, span):
    """Ids that share the top bits of Knuth's multiplicative hash: inserts and
    lookups run past the kernel's trip limit, the workgroup rebuilds its table
    with the salted hash, and everything still resolves exactly. With K = 3000
    the ids take two classification passes, both in the first run and in the
    rebuild."""
    h = _harness()
    ids = np.arange(span, dtype=np.uint64)
    home = ((ids * np.uint64(2654435761)) & np.uint64(0xFFFFFFFF)) >> np.uint64(32 - 10)
    cand = ids[home < 8].astype(np.int64)           # ids in 8 of 1024 top-bit windows
    ctx = int(cand.max()) + 2
    cfg = _small(B=2, H=H, K=K, ctx=ctx, row_bytes=16)
    run = h.ParityRun(cfg)
    rng = np.random.default_rng(11)
    prev = None
    for t in range(4):
        rows = np.arange(2, dtype=np.int64)
        seq = np.full(2, ctx, dtype=np.int64)
        topk = np.stack([rng.choice(cand, size=K, replace=False) for _ in range(2)]).astype(np.int32)
        if prev is not None:
            topk[:, :K // 2] = prev[:, :K // 2]
            for b in range(2):
                fresh = np.setdiff1d(cand, prev[b])
                topk[b, K // 2:] = rng.choice(fresh, size=K - K // 2, replace=False)
        prev = topk.copy()
        run.step(topk, seq)


def test_empty_calls_are_noops():
    import sparse_attention_kv_hisparse_amd as hs
    cfg = _small()
    from workloads import device as wdev
    st = wdev.DeviceSwapState(cfg)
    pool = wdev.make_pool(cfg)
    before = st.lru.clone()
    out = torch.empty((0, cfg.K), dtype=torch.int32, device="cuda")
    hs.hisparse_swap_in(topk=torch.empty((0, cfg.K), dtype=torch.int32, device="cuda"),
                        req_rows=torch.empty(0, dtype=torch.int64, device="cuda"),
                        seq_lens=torch.empty(0, dtype=torch.int64, device="cuda"),
                        slot_tokens=st.slot_tokens, lru=st.lru, pool=pool, hot=st.hot,
                        out_rows=out, ctx_stride=cfg.ctx, workspace=st.ws)
    torch.cuda.synchronize()
    assert torch.equal(before, st.lru)


@pytest.mark.parametrize("H,K", [(32768, 585), (8192, 4097), (32768, 32768)])
def test_sizes_beyond_lds_are_rejected(H, K):
    """K and H whose per-request scratch does not fit one workgroup's LDS
    return HS_ERANGE before anything is enqueued: state and outputs untouched.
    The context (131,072 positions) is too long for a direct-address table,
    so the hash table's limits apply."""
    import sparse_attention_kv_hisparse_amd as hs
    from sparse_attention_kv_hisparse_amd._lib import HisparseError
    from workloads import device as wdev
    cfg = _small(H=H, K=K, ctx=1 << 17, B=1, row_bytes=16)
    st = wdev.DeviceSwapState(cfg)
    pool = wdev.make_pool(cfg)
    st.out.fill_(7)
    before = (st.slot_tokens.clone(), st.lru.clone(), st.out.clone())
    topk = torch.arange(K, dtype=torch.int32, device="cuda").reshape(1, K)
    with pytest.raises(HisparseError) as e:
        hs.hisparse_swap_in(topk=topk, req_rows=torch.zeros(1, dtype=torch.int64, device="cuda"),
                            seq_lens=torch.full((1,), cfg.ctx, dtype=torch.int64, device="cuda"),
                            slot_tokens=st.slot_tokens, lru=st.lru, pool=pool, hot=st.hot,
                            out_rows=st.out, ctx_stride=cfg.ctx, workspace=st.ws)
    assert e.value.status == -2 and "LDS" in str(e.value)
    torch.cuda.synchronize()
    for a, b in zip(before, (st.slot_tokens, st.lru, st.out)):
        assert torch.equal(a, b)


def test_replay_from_restored_state_is_identical():
    """Restoring the state and replaying a call reproduces every output bit:
    nothing depends on scheduling order."""
    import sparse_attention_kv_hisparse_amd as hs
    from workloads import device as wdev
    cfg = gen.DEVPOOL.with_(B=16)
    st = wdev.DeviceSwapState(cfg)
    pool = wdev.make_pool(cfg)
    rows = torch.arange(cfg.B, dtype=torch.int64, device="cuda")
    trace = list(gen.topk_trace(cfg, 3))
    for t, topk in enumerate(trace[:2]):
        hs.hisparse_swap_in(topk=torch.as_tensor(topk).cuda(), req_rows=rows,
                            seq_lens=torch.as_tensor(gen.seq_lens(cfg, t)).cuda(),
                            slot_tokens=st.slot_tokens, lru=st.lru, pool=pool, hot=st.hot,
                            out_rows=st.out, ctx_stride=cfg.ctx, workspace=st.ws,
                            miss_counts=st.counts)
    snap = (st.slot_tokens.clone(), st.lru.clone(), st.hot.clone())
    results = []
    for _ in range(3):
        st.slot_tokens.copy_(snap[0]); st.lru.copy_(snap[1]); st.hot.copy_(snap[2])
        hs.hisparse_swap_in(topk=torch.as_tensor(trace[2]).cuda(), req_rows=rows,
                            seq_lens=torch.as_tensor(gen.seq_lens(cfg, 2)).cuda(),
                            slot_tokens=st.slot_tokens, lru=st.lru, pool=pool, hot=st.hot,
                            out_rows=st.out, ctx_stride=cfg.ctx, workspace=st.ws,
                            miss_counts=st.counts)
        torch.cuda.synchronize()
        results.append([x.clone() for x in (st.out, st.counts, st.slot_tokens, st.lru, st.hot)])
    for r in results[1:]:
        for a, b in zip(results[0], r):
            assert torch.equal(a, b)
