"""Broken state never makes the kernels write outside their buffers.

The swap-in's preconditions (an LRU row that is a permutation of 0..H-1, one
slot per resident token, block tables that name rows inside the hot buffer)
are the caller's; with them broken the results are unspecified, but every
index the kernels take from state or tables is range-checked before use.
These cases break the state on purpose -- LRU entries that are negative, past
H or repeated, slot tokens repeated across slots, paged hot block tables with
entries past the buffer or negative -- and check, after three calls, that the
guard zones around the hot buffer, the state rows, the outputs and the miss
counts still hold their fill pattern, that miss counts stay in [0, K], and
(flat layout) that every output is -1 or a row of its own request's region.
Two cases also repeat top-k ids within a row (the ids of a row are unique by
precondition). The oracle is not involved: it rejects such state."""

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


G = 64   # guard rows on each side


def _guarded(rows, cols, dtype, fill):
    back = torch.full((rows + 2 * G, cols), fill, dtype=dtype, device="cuda")
    return back, back[G:G + rows]


def _guards_hold(back, rows, fill, name):
    b = back.cpu()
    assert (b[:G] == fill).all() and (b[G + rows:] == fill).all(), f"{name}: a guard row was written"


@pytest.mark.parametrize("ctx,kind,paged,dup", [
    (2000, "host", False, False),      # direct table, fused copy
    (2000, "device", False, False),    # direct table, wide copy
    (70000, "host", False, False),     # hashed plan
    (3000, "host", True, False),       # paged: hot block table entries outside the buffer
    (3000, "device", True, False),
    (2000, "host", False, True),       # repeated top-k ids, direct table
    (70000, "device", False, True),    # repeated top-k ids, hashed plan
], ids=["direct_host", "direct_device", "hashed_host", "paged_host", "paged_device",
        "direct_dup_ids", "hashed_dup_ids"])
def test_broken_state_stays_in_bounds(ctx, kind, paged, dup):
    import sparse_attention_kv_hisparse_amd as hs
    R, B, H, K, rb = 6, 4, 256, 64, 32
    S_r = H + 1
    print(f"  broken state: ctx={ctx} pool={kind} paged={paged} dup={dup}", flush=True)
    rng = np.random.default_rng(ctx + 7 * paged + (kind == "device") + 13 * dup)
    hot_nrows = R * S_r
    hot_back, hot = _guarded(hot_nrows, rb, torch.uint8, 0xA5)
    tok_back, tokens = _guarded(R, S_r, torch.int32, 0x5A5A5A5A)
    lru_back, lru = _guarded(R, H, torch.int16, 0x5A5A)
    out_back, out = _guarded(B, K, torch.int32, 0x5A5A5A5A)
    cnt_back, counts = _guarded(B, 1, torch.int32, 0x5A5A5A5A)
    counts = counts.view(B)
    ws = torch.zeros(hs.swap_in_workspace_bytes(B, K), dtype=torch.uint8, device="cuda")
    cfg = gen.SwapConfig("broken", B=B, H=H, K=K, ctx=ctx, row_bytes=rb, steps=1, rho=0.5,
                         dist="uniform", pool_kind=kind, seed=71)
    pool_nrows = R * ctx
    pool = wdev.make_pool(cfg.with_(B=R), kind=kind)[:pool_nrows]
    # broken state: LRU entries out of range and repeated, slot tokens repeated
    tokens.copy_(torch.as_tensor(rng.integers(-5, ctx + 50, (R, S_r)), dtype=torch.int32))
    lru.copy_(torch.as_tensor(rng.integers(-300, H + 300, (R, H)), dtype=torch.int16))
    req_rows = torch.as_tensor(rng.permutation(R)[:B].astype(np.int64)).cuda()
    seq = torch.full((B,), ctx, dtype=torch.int64, device="cuda")
    kw = {}
    if paged:
        hbs = 16
        nb = (H + hbs - 1) // hbs
        # entries past the buffer, negative, and huge (a row past int32)
        hbt = rng.integers(-3, 3 * hot_nrows // hbs, (R, nb)).astype(np.int32)
        hbt[:, 0] = 2**30
        kw["paged"] = {"hot_block_table": torch.as_tensor(hbt).cuda(), "hot_block_size": hbs}
    for step in range(3):
        topk = np.stack([rng.choice(ctx, size=K, replace=False) for _ in range(B)]).astype(np.int32)
        # some ids are tokens the broken slots hold, several times over
        tok_np = tokens.cpu().numpy()
        for b in range(B):
            held = np.unique(tok_np[int(req_rows[b])][(tok_np[int(req_rows[b])] >= 0) &
                                                      (tok_np[int(req_rows[b])] < ctx)])
            take = held[:K // 4]
            rest = np.setdiff1d(topk[b], take)[:K - len(take)]
            row = np.concatenate([take, rest])
            if len(row) < K:
                row = np.concatenate([row, np.setdiff1d(np.arange(ctx), row)[:K - len(row)]])
            topk[b] = rng.permutation(row)
            if dup:   # an eighth of the row repeats other entries of it
                topk[b][K // 2:K // 2 + K // 8] = topk[b][:K // 8]
        hs.hisparse_swap_in(topk=torch.as_tensor(topk).cuda(), req_rows=req_rows,
                            seq_lens=None if paged else seq, slot_tokens=tokens, lru=lru,
                            pool=pool, hot=hot, out_rows=out, ctx_stride=0 if paged else ctx,
                            workspace=ws, miss_counts=counts, **kw)
        torch.cuda.synchronize()
        c = counts.cpu().numpy()
        assert ((c >= 0) & (c <= K)).all(), f"step {step}: miss counts {c}"
        if not paged:
            o = out.cpu().numpy()
            for b in range(B):
                r = int(req_rows[b])
                ok = (o[b] == -1) | ((o[b] >= r * S_r) & (o[b] <= r * S_r + H))
                assert ok.all(), f"step {step}: row {b} names a row outside its region"
    _guards_hold(hot_back, hot_nrows, 0xA5, "hot buffer")
    _guards_hold(tok_back, R, 0x5A5A5A5A, "slot tokens")
    _guards_hold(lru_back, R, 0x5A5A, "lru")
    _guards_hold(out_back, B, 0x5A5A5A5A, "out_rows")
    _guards_hold(cnt_back, B, 0x5A5A5A5A, "miss_counts")
