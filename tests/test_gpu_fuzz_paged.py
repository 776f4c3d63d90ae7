"""Seeded random sweep of the swap-in under vLLM-style paged addressing,
against the oracle.

Each case draws its own sizes and tables from a fixed seed: hot sizes from 1
to 8192 (the slot-key hash while it fits LDS, the pending-id hash past it),
hot block sizes that are and are not powers of two (1 to 100, and hot block
table rows too long to stage in LDS), no source block table (a position is its
global id) or one with blocks of 1 to 128 rows (null and negative blocks, a
last block cut short, rows too long to stage), with or without a resident
table inside the vLLM page's domain (its block size the hot block size, a
non-negative null block), host and device pools, the fused and the split
paths, K+V, and rows of 4 to 656 bytes. Every call is compared with the oracle
on outputs, attention indices, counts, counters, slot keys, LRU and the whole
hot buffer (test_gpu_paged.run_paged_case), with an invalidation of written
rows between calls.
"""

import os

import numpy as np
import pytest

from test_gpu_paged import run_paged_case

pytestmark = pytest.mark.gpu

N_CASES = int(os.environ.get("HS_FUZZ_PAGED_CASES", 32))   # more seeds of the same draw on request
H_CHOICES = [1, 2, 7, 63, 64, 65, 255, 1000, 2047, 4096, 4500, 6000, 8192]
HB_CHOICES = [1, 2, 3, 5, 7, 16, 64, 100]
SB_CHOICES = [0, 1, 3, 4, 16, 64, 128]      # 0: no source block table
RB_CHOICES = [4, 16, 132, 656]
POOL_CAP = 64 << 20   # bytes of pool per case


def paged_tables(rng, R, H, ctx, hb, sb, resident):
    """Hot block table (a permutation of the buffer's blocks, a few spare),
    source table of sb-row blocks (about 10% null or negative, block 0 never
    used as a real block, the pool's last block cut short) or none, and a
    resident table with the hot block size whose entries are mostly the null
    block, some negative, some real blocks and a few blocks whose rows reach
    or pass INT32_MAX. Returns (paged, hot_nrows, pool_nrows)."""
    nhb = -(-H // hb)
    extra = int(rng.integers(0, 4))
    hot_blocks = rng.permutation(R * nhb + extra)[:R * nhb].reshape(R, nhb).astype(np.int32)
    paged = {"hot_block_table": hot_blocks, "hot_block_size": hb}
    hot_nrows = (R * nhb + extra) * hb
    if not sb:
        return paged, hot_nrows, ctx - int(rng.integers(0, 4))
    nsb = -(-ctx // sb) + 1
    phys = rng.permutation(np.arange(1, R * nsb + 4))[:R * nsb].reshape(R, nsb).astype(np.int32)
    nulls = rng.random((R, nsb)) < 0.1
    phys[nulls] = rng.choice([0, -1], size=int(nulls.sum()))
    paged.update(src_block_table=phys, src_block_size=sb)
    pool_nrows = (R * nsb + 4) * sb - sb // 2
    if resident:
        nrb = -(-ctx // hb)
        null = int(rng.choice([0, 3, 17]))
        res = np.full((R, nrb), null, np.int32)
        res[rng.random((R, nrb)) < 0.1] = -1
        hit = rng.random((R, nrb)) < 0.15
        res[hit] = rng.integers(0, 50, int(hit.sum()))
        # blocks whose rows reach INT32_MAX or pass it (no int32 output can
        # hold those: not resident)
        res[rng.random((R, nrb)) < 0.05] = int(rng.choice([2**30, 2**31 - 1]))
        paged.update(resident_block_table=res, resident_block_size=hb, resident_null_block=null)
    return paged, hot_nrows, pool_nrows


def draw_case(i: int) -> dict:
    rng = np.random.default_rng(8_000 + i)
    H = int(rng.choice(H_CHOICES))
    K = int(rng.integers(1, min(H, 4096 if H < 4096 else 2048) + 1))
    R = int(rng.integers(1, 7))
    sb = int(rng.choice(SB_CHOICES))
    return dict(i=i, H=H, K=K, R=R, B=int(rng.integers(1, R + 1)),
                ctx=int(rng.integers(K + 2, 4 * K + 3_000)), hb=int(rng.choice(HB_CHOICES)), sb=sb,
                resident=bool(sb and rng.random() < 0.5), rb=int(rng.choice(RB_CHOICES)),
                kind=str(rng.choice(["host", "device"])), split=bool(rng.random() < 0.3),
                kv=bool(rng.random() < 0.25), seed=int(rng.integers(1, 2**31)))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_paged_case_matches_oracle(i):
    c = draw_case(i)
    print(f"  paged fuzz case {c}", flush=True)
    rng = np.random.default_rng(c["seed"])
    paged, hot_nrows, pool_nrows = paged_tables(rng, c["R"], c["H"], c["ctx"], c["hb"], c["sb"],
                                                c["resident"])
    rb = c["rb"]
    while pool_nrows * rb * (2 if c["kv"] else 1) > POOL_CAP and rb > 4:
        rb = max(r for r in RB_CHOICES if r < rb)
    run_paged_case(rng, f"paged_fuzz{i}", c["R"], c["B"], c["H"], c["K"], c["ctx"], rb, c["kind"],
                   c["split"], c["kv"], paged, hot_nrows, pool_nrows, calls=6)


def test_the_paged_sweep_reaches_every_option():
    """The drawn cases cover what the sweep is for (checked on the CPU side of
    the draw, so a change of seeds cannot quietly narrow it)."""
    cases = [draw_case(i) for i in range(N_CASES)]
    assert any(c["H"] <= 4096 for c in cases) and any(c["H"] > 4500 for c in cases)
    assert any(c["hb"] & (c["hb"] - 1) for c in cases) and any(c["hb"] in (16, 64) for c in cases)
    assert any(-(-c["H"] // c["hb"]) > 2048 for c in cases)            # hot table not staged
    assert any(c["sb"] == 0 for c in cases) and any(c["sb"] in (3, 128) for c in cases)
    assert any(c["sb"] and -(-c["ctx"] // c["sb"]) + 1 > 2048 for c in cases)   # source table not staged
    assert any(c["resident"] for c in cases)
    assert {c["kind"] for c in cases} == {"host", "device"}
    assert any(c["split"] for c in cases) and any(c["kv"] for c in cases)
    assert any(c["rb"] % 16 for c in cases) and any(c["rb"] % 16 == 0 for c in cases)
