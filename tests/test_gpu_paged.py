"""vLLM-style paged addressing and write invalidation on the GPU, against the
oracle, bit for bit: random hot, source and resident block tables (null
blocks, ids past the pool, padding rows), global-id slot keys, attention
indices, host and device pools, the fused and the split paths, K+V, a hot
block table too long to stage in LDS, hisparse_invalidate_written between
calls, and a dozen cases with sizes and options drawn from fixed seeds."""

import zlib

import numpy as np
import pytest
import torch

import oracle
from test_oracle_paged import _random_tables
from workloads import device as wdev
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import sparse_attention_kv_hisparse_amd as hs
    hs.load()
    torch.cuda.set_device(0)


def _np(t):
    return t.cpu().numpy() if t.is_cuda else t.numpy()


CASES = [
    # (name, R, B, H, K, ctx, row_bytes, pool kind, split, kv, hot block size or None = random)
    ("host_fused", 8, 6, 512, 256, 3000, 656, "host", False, False, None),
    ("host_split", 8, 6, 512, 256, 3000, 656, "host", True, False, None),
    ("device", 10, 8, 600, 300, 4000, 512, "device", False, False, None),
    ("host_132B_kv", 6, 4, 256, 200, 2000, 132, "host", False, True, None),
    # 3000 one-row hot blocks: the hot block table row is too long to stage in
    # LDS, so slot rows are read from HBM and the fused copy loads no chunk early
    ("host_fused_hbt_in_hbm", 4, 3, 3000, 500, 6000, 656, "host", False, False, 1),
]


def _random_cases(n):
    """Cases drawn from fixed seeds: sizes off the 64-slot and 1024-lane grids,
    random block sizes (the tables come from _random_tables), pool kind, the
    split path and K+V."""
    out = []
    for i in range(n):
        rng = np.random.default_rng(9_100 + i)
        H = int(rng.choice([1, 5, 63, 64, 100, 300, 1000, 2047]))
        K = int(rng.integers(1, H + 1))
        R = int(rng.integers(1, 9))
        B = int(rng.integers(1, R + 1))
        ctx = int(rng.integers(K + 2, 4 * K + 2_000))
        rb = int(rng.choice([4, 16, 132, 656]))
        out.append((f"rand{i}", R, B, H, K, ctx, rb, str(rng.choice(["host", "device"])),
                    bool(rng.random() < 0.3), bool(rng.random() < 0.3), None))
    return out


CASES += _random_cases(12)
# more slots than one pass of the workgroup inserts into the paged key hash
CASES.append(("host_key_hash_two_passes", 2, 2, 4500, 200, 12000, 16, "host", False, False, None))
# Hot sizes whose key hash does not fit LDS beside the LRU row: a hash of the
# pending global ids, probed with every slot's key. By the LDS arithmetic of
# the plans: a quarter-full hash with the slot keys staged (H 8192, K 2048);
# half full, staged, with K+V (H 12000); a quarter-full hash with the keys
# read from HBM, on the split path (H 16384).
CASES += [
    ("host_pending_hash", 2, 2, 8192, 2048, 12000, 16, "host", False, False, 8),
    ("host_pending_hash_half_full_kv", 2, 2, 12000, 2048, 16000, 16, "host", False, True, 4),
    ("device_pending_hash_unstaged_split", 2, 1, 16384, 1024, 24000, 16, "device", True, False, 16),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_swap_in_matches_oracle(case):
    name, R, B, H, K, ctx, rb, kind, split, kv, hb = case
    print(f"  paged {name}: R={R} B={B} H={H} K={K} rb={rb}", flush=True)
    rng = np.random.default_rng(zlib.crc32(name.encode()))   # the same tables in every process
    paged_np, hot_nrows, pool_nrows = _random_tables(rng, R, H, ctx, hb)
    run_paged_case(rng, name, R, B, H, K, ctx, rb, kind, split, kv, paged_np, hot_nrows, pool_nrows)


def run_paged_case(rng, name, R, B, H, K, ctx, rb, kind, split, kv, paged_np, hot_nrows, pool_nrows,
                   calls=8):
    """`calls` calls on fresh state (every fourth an invalidation of random
    written rows instead), each through the fused or the split path, with
    random top-k rows over positions -3 .. ctx+4, a padded batch on the third
    call, attention indices and the running counters; everything the call
    writes is compared with the oracle after each call."""
    import sparse_attention_kv_hisparse_amd as hs
    S_r = H + 1
    cfg = gen.SwapConfig(name, B=B, H=H, K=K, ctx=pool_nrows, row_bytes=rb, steps=1, rho=0.5,
                         dist="uniform", pool_kind=kind, seed=61)
    pool = wdev.make_pool(cfg.with_(B=1), kind=kind)[:pool_nrows]
    pool_v = wdev.make_pool(cfg.with_(B=1, seed=62), kind=kind)[:pool_nrows] if kv else None
    pool_np = _np(pool)
    pool_v_np = _np(pool_v) if kv else None
    keys = torch.full((R, S_r), -1, dtype=torch.int32, device="cuda")
    lru = torch.tensor(np.tile(np.arange(H, dtype=np.int16), (R, 1)), device="cuda")
    hot = torch.zeros((hot_nrows, rb), dtype=torch.uint8, device="cuda")
    hot_v = torch.zeros_like(hot) if kv else None
    out = torch.empty((B, K), dtype=torch.int32, device="cuda")
    counts = torch.empty(B, dtype=torch.int32, device="cuda")
    att = torch.full((B, K + 3), 7777, dtype=torch.int32, device="cuda")   # a tail past K
    ws = torch.zeros(hs.swap_in_workspace_bytes(B, K), dtype=torch.uint8, device="cuda")
    paged_dev = {k: (torch.as_tensor(v).cuda() if isinstance(v, np.ndarray) else v)
                 for k, v in paged_np.items()}
    paged_dev["attention_indices"] = att
    paged_dev["attention_block_stride"] = 40
    o_keys = np.full((R, S_r), -1, np.int32)
    o_lru = np.tile(np.arange(H, dtype=np.int16), (R, 1))
    o_hot = np.zeros((hot_nrows, rb), np.uint8)
    o_hot_v = np.zeros_like(o_hot) if kv else None
    stats = torch.zeros(2, dtype=torch.int64, device="cuda")
    o_stats = np.zeros(2, np.uint64)
    for call in range(calls):
        if call % 4 == 3:
            rows = rng.integers(-1, R + 1, 40).astype(np.int64)
            written = np.array([o_keys[r % R, rng.integers(0, H)] for r in rows], np.int64)
            hs.hisparse_invalidate_written(slot_keys=keys, rows=torch.as_tensor(rows).cuda(),
                                           written=torch.as_tensor(written).cuda())
            oracle.invalidate_written(o_keys, rows, written)
            torch.cuda.synchronize()
            assert np.array_equal(_np(keys), o_keys), f"call {call}: keys after invalidation"
            continue
        req = rng.permutation(R)[:B].astype(np.int64)
        topk = np.stack([rng.permutation(np.arange(-3, ctx + 5))[:K] for _ in range(B)]).astype(np.int32)
        nreal = int(rng.integers(1, B + 1)) if call == 2 else -1
        kw = dict(topk=torch.as_tensor(topk).cuda(), req_rows=torch.as_tensor(req).cuda(),
                  seq_lens=None, slot_tokens=keys, lru=lru, pool=pool, hot=hot, out_rows=out,
                  ctx_stride=0, workspace=ws, miss_counts=counts,
                  num_real=torch.tensor([nreal if nreal >= 0 else B], dtype=torch.int32, device="cuda"),
                  paged=paged_dev, stats=stats)
        if kv:
            kw.update(pool_v=pool_v, hot_v=hot_v)
        if split:
            hs.hisparse_resolve(**kw)
            hs.hisparse_gather_compact(**kw)
        else:
            hs.hisparse_swap_in(**kw)
        o_att = np.full((B, K + 3), 0, np.int32)
        pg = dict(paged_np, attention_indices=o_att, attention_block_stride=40)
        o_out, o_cnt = oracle.swap_in(topk=topk, req_rows=req, seq_lens=None, slot_tokens=o_keys,
                                      lru=o_lru, pool=pool_np, hot=o_hot, ctx_stride=0, num_real=nreal,
                                      paged=pg, pool_v=pool_v_np, hot_v=o_hot_v, stats=o_stats)
        torch.cuda.synchronize()
        assert np.array_equal(_np(stats).astype(np.uint64), o_stats), f"call {call}: stats"
        assert np.array_equal(_np(out), o_out), f"call {call}: out_rows"
        assert np.array_equal(_np(counts), o_cnt), f"call {call}: miss_counts"
        assert np.array_equal(_np(att)[:, :K], o_att[:, :K]), f"call {call}: attention_indices"
        assert (_np(att)[:, K:] == 7777).all(), f"call {call}: attention row tail written"
        assert np.array_equal(_np(keys), o_keys), f"call {call}: slot keys"
        assert np.array_equal(_np(lru), o_lru), f"call {call}: lru"
        assert np.array_equal(_np(hot), o_hot), f"call {call}: hot buffer"
        if kv:
            assert np.array_equal(_np(hot_v), o_hot_v), f"call {call}: V hot buffer"


@pytest.mark.parametrize("hb,block", [(1, 2**31 - 1), (2, 2**30)], ids=["row_int32_max", "row_past_int32"])
def test_paged_resident_rows_at_the_int32_limit(hb, block):
    """Every fourth resident block names a row of exactly INT32_MAX (one-row
    blocks: served as is) or rows past it (no int32 output can hold them: the
    positions are looked up and copied like any other)."""
    rng = np.random.default_rng(41 + hb)
    R, B, H, K, ctx, rb = 3, 2, 16, 8, 120, 16
    paged, hot_nrows, pool_nrows = _random_tables(rng, R, H, ctx, hb)
    tab = paged["resident_block_table"].copy()
    tab[:, ::4] = block
    paged["resident_block_table"] = tab
    run_paged_case(rng, f"resident_limit_{hb}", R, B, H, K, ctx, rb, "host", False, False, paged,
                   hot_nrows, pool_nrows)


def test_paged_full_size_dsv32():
    """The DeepSeek-V3.2-like shape (B=32, H=4096, K=2048, 32,768-token contexts,
    pinned-host pool) with vLLM-style addressing: 64-row source blocks (a seeded
    permutation, block 0 unused) and 64-slot hot blocks; the cold step and three
    steady steps against the oracle, with attention indices. A resident table
    of 64-row blocks (the hot block size) with null block 0 serves about 5% of
    each request's blocks from the device cache."""
    import sparse_attention_kv_hisparse_amd as hs
    cfg = gen.DSV32
    block = 64
    rng = np.random.default_rng(77)
    B, H, K, ctx, rb = cfg.B, cfg.H, cfg.K, cfg.ctx, cfg.row_bytes
    R = B
    nsb = ctx // block
    src = (rng.permutation(B * nsb) + 1).astype(np.int32).reshape(B, nsb)
    pool_nrows = (B * nsb + 1) * block
    nhb = H // block
    hot_tab = rng.permutation(R * nhb).astype(np.int32).reshape(R, nhb)
    res_tab = np.zeros((R, nsb), np.int32)                   # null block 0 everywhere ...
    live = rng.random((R, nsb)) < 0.05
    res_tab[live] = rng.integers(1, 1 << 14, int(live.sum()))  # ... but ~5% resident
    print(f"  paged full size: pool {pool_nrows} rows", flush=True)
    pool = wdev.make_pool(cfg.with_(B=1, ctx=pool_nrows))
    keys = torch.full((R, H + 1), -1, dtype=torch.int32, device="cuda")
    lru = torch.tensor(np.tile(np.arange(H, dtype=np.int16), (R, 1)), device="cuda")
    hot = torch.zeros((R * nhb * block, rb), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, K), dtype=torch.int32, device="cuda")
    counts = torch.empty(B, dtype=torch.int32, device="cuda")
    att = torch.empty((B, K), dtype=torch.int32, device="cuda")
    ws = torch.empty(hs.swap_in_workspace_bytes(B, K), dtype=torch.uint8, device="cuda")
    paged_dev = {"hot_block_table": torch.as_tensor(hot_tab).cuda(), "hot_block_size": block,
                 "src_block_table": torch.as_tensor(src).cuda(), "src_block_size": block,
                 "resident_block_table": torch.as_tensor(res_tab).cuda(),
                 "resident_block_size": block, "resident_null_block": 0,
                 "attention_indices": att, "attention_block_stride": 128}
    o_keys = np.full((R, H + 1), -1, np.int32)
    o_lru = np.tile(np.arange(H, dtype=np.int16), (R, 1))
    o_hot = np.zeros((R * nhb * block, rb), np.uint8)
    rows = np.arange(B, dtype=np.int64)
    for t, topk in enumerate(gen.topk_trace(cfg, 4)):
        hs.hisparse_swap_in(topk=torch.as_tensor(topk).cuda(), req_rows=torch.as_tensor(rows).cuda(),
                            seq_lens=None, slot_tokens=keys, lru=lru, pool=pool, hot=hot,
                            out_rows=out, ctx_stride=0, workspace=ws, miss_counts=counts,
                            paged=paged_dev)
        o_att = np.zeros((B, K), np.int32)
        o_out, o_cnt = oracle.swap_in(
            topk=topk, req_rows=rows, seq_lens=None, slot_tokens=o_keys, lru=o_lru,
            pool=pool.numpy(), hot=o_hot, ctx_stride=0,
            paged={"hot_block_table": hot_tab, "hot_block_size": block, "src_block_table": src,
                   "src_block_size": block, "resident_block_table": res_tab,
                   "resident_block_size": block, "resident_null_block": 0,
                   "attention_indices": o_att, "attention_block_stride": 128})
        torch.cuda.synchronize()
        print(f"  paged full size step {t}: {int(o_cnt.sum())} misses", flush=True)
        assert np.array_equal(_np(out), o_out), f"step {t}: out_rows"
        assert np.array_equal(_np(counts), o_cnt), f"step {t}: miss_counts"
        assert np.array_equal(_np(att), o_att), f"step {t}: attention_indices"
        assert np.array_equal(_np(keys), o_keys), f"step {t}: slot keys"
        assert np.array_equal(_np(lru), o_lru), f"step {t}: lru"
        assert np.array_equal(_np(hot), o_hot), f"step {t}: hot buffer"


@pytest.mark.parametrize("H,K,hb,bits,span,steps", [
    # the key hash of the slots' keys: pow2(4H) entries in buckets of four, H
    # buckets, picked by the top log2(H) = 10 bits of id * 2654435761 (mod 2^32)
    (1024, 512, 16, 10, 200_000, 4),
    # H 8192 leaves no room for the key hash: a quarter-full hash of the
    # pending ids, pow2(4K) entries, 2048 buckets (top 11 bits), probed with
    # every slot's key; eight steps, so that the last ones evict
    (8192, 2048, 64, 11, 1_200_000, 8),
], ids=["key_hash", "pending_id_hash"])
def test_paged_keys_clustered_in_the_kernel_hash(H, K, hb, bits, span, steps):
    """Paged addressing without a source table (a position is its global id),
    with ids that share the top bits of Knuth's multiplicative hash: the keys
    then crowd a few buckets of the table, inserts and lookups (or the probes)
    run past the kernel's trip limit, the workgroup rebuilds the table with the
    salted hash, and every call still matches the oracle."""
    import sparse_attention_kv_hisparse_amd as hs
    R = B = 2
    rb = 16
    ids = np.arange(span, dtype=np.uint64)
    home = ((ids * np.uint64(2654435761)) & np.uint64(0xFFFFFFFF)) >> np.uint64(32 - bits)
    cand = ids[home < 8].astype(np.int64)          # ids in 8 of the 2^bits buckets
    assert len(cand) >= 2 * K
    pool_nrows = int(cand.max()) + 1
    rng = np.random.default_rng(5)
    nhb = H // hb
    hot_tab = rng.permutation(R * nhb).astype(np.int32).reshape(R, nhb)
    cfg = gen.SwapConfig("paged_cluster", B=1, H=H, K=K, ctx=pool_nrows, row_bytes=rb, steps=1,
                         rho=0.5, dist="uniform", pool_kind="host", seed=63)
    pool = wdev.make_pool(cfg)
    keys = torch.full((R, H + 1), -1, dtype=torch.int32, device="cuda")
    lru = torch.tensor(np.tile(np.arange(H, dtype=np.int16), (R, 1)), device="cuda")
    hot = torch.zeros((R * nhb * hb, rb), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, K), dtype=torch.int32, device="cuda")
    counts = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = torch.zeros(hs.swap_in_workspace_bytes(B, K), dtype=torch.uint8, device="cuda")
    paged = {"hot_block_table": torch.as_tensor(hot_tab).cuda(), "hot_block_size": hb}
    o_keys = np.full((R, H + 1), -1, np.int32)
    o_lru = np.tile(np.arange(H, dtype=np.int16), (R, 1))
    o_hot = np.zeros((R * nhb * hb, rb), np.uint8)
    rows = np.arange(B, dtype=np.int64)
    prev = None
    for t in range(steps):
        topk = np.stack([rng.choice(cand, size=K, replace=False) for _ in range(B)]).astype(np.int32)
        if prev is not None:
            topk[:, :K // 2] = prev[:, :K // 2]
            for b in range(B):
                fresh = np.setdiff1d(cand, prev[b])
                topk[b, K // 2:] = rng.choice(fresh, size=K - K // 2, replace=False)
        prev = topk.copy()
        hs.hisparse_swap_in(topk=torch.as_tensor(topk).cuda(), req_rows=torch.as_tensor(rows).cuda(),
                            seq_lens=None, slot_tokens=keys, lru=lru, pool=pool, hot=hot,
                            out_rows=out, ctx_stride=0, workspace=ws, miss_counts=counts, paged=paged)
        o_out, o_cnt = oracle.swap_in(topk=topk, req_rows=rows, seq_lens=None, slot_tokens=o_keys,
                                      lru=o_lru, pool=pool.numpy(), hot=o_hot, ctx_stride=0,
                                      paged={"hot_block_table": hot_tab, "hot_block_size": hb})
        torch.cuda.synchronize()
        print(f"  paged cluster step {t}: {int(o_cnt.sum())} misses", flush=True)
        assert np.array_equal(_np(out), o_out), f"step {t}: out_rows"
        assert np.array_equal(_np(counts), o_cnt), f"step {t}: miss_counts"
        assert np.array_equal(_np(keys), o_keys), f"step {t}: slot keys"
        assert np.array_equal(_np(lru), o_lru), f"step {t}: lru"
        assert np.array_equal(_np(hot), o_hot), f"step {t}: hot buffer"
