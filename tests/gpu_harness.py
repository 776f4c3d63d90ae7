"""Side-by-side runs of the HIP swap-in and the CPU oracle on identical inputs.

After every call the GPU's outputs and state are downloaded and compared with
the oracle's bit for bit: out_rows, miss_counts, slot_tokens, lru, the running
hit / miss counters and the whole hot buffer (every byte, every step, so a
stray write that a later copy would overwrite is still seen).
"""

from __future__ import annotations

import sys
from typing import Optional

import numpy as np
import torch

import oracle
import sparse_attention_kv_hisparse_amd as hs
from workloads import device as wdev
from workloads import gen


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def assert_equal(name: str, got: np.ndarray, want: np.ndarray) -> None:
    if got.shape != want.shape or not np.array_equal(got, want):
        bad = np.argwhere(got != want) if got.shape == want.shape else None
        first = bad[:5].tolist() if bad is not None else "shape"
        raise AssertionError(f"{name} differs from the oracle at {first} "
                             f"({0 if bad is None else len(bad)} entries)")


class ParityRun:
    def __init__(self, cfg: gen.SwapConfig, *, R: Optional[int] = None,
                 req_rows: Optional[np.ndarray] = None, pool_kind: Optional[str] = None,
                 slot_rows: Optional[np.ndarray] = None, pool_rows: Optional[np.ndarray] = None,
                 hot_nrows: Optional[int] = None, pool_nrows: Optional[int] = None,
                 hot_misalign: bool = False):
        self.cfg = cfg
        self.R = R or cfg.R
        self.req_rows = np.arange(cfg.B, dtype=np.int64) if req_rows is None else req_rows
        kind = pool_kind or cfg.pool_kind
        if pool_nrows is None:
            self.pool_t = wdev.make_pool(cfg, kind=kind)
        else:
            c2 = cfg.with_(B=max(1, -(-pool_nrows // cfg.ctx)))
            full = wdev.make_pool(c2, kind=kind)
            self.pool_t = full[:pool_nrows]
        self.pool_np = self.pool_t.cpu().numpy() if self.pool_t.is_cuda else self.pool_t.numpy()
        self.st = wdev.DeviceSwapState(cfg, R=self.R, hot_nrows=hot_nrows)
        if hot_misalign:
            # hot rows starting 4 bytes past a 16-byte boundary force the 4-byte copy path
            backing = torch.zeros((self.st.hot.shape[0] * cfg.row_bytes + 16,), dtype=torch.uint8,
                                  device="cuda")
            self.st.hot = backing[4:4 + self.st.hot.numel()].view(self.st.hot.shape)
        self.slot_rows = slot_rows
        self.pool_rows = pool_rows
        self.slot_rows_t = None if slot_rows is None else torch.as_tensor(slot_rows).cuda()
        self.pool_rows_t = None if pool_rows is None else torch.as_tensor(pool_rows).cuda()
        self.o_tokens, self.o_lru = gen.initial_state(self.R, cfg.H, cfg.S_r)
        self.o_hot = np.zeros(tuple(self.st.hot.shape), dtype=np.uint8)
        # running hit / miss counters, accumulated over the run on both sides
        self.stats = torch.zeros(2, dtype=torch.int64, device="cuda")
        self.o_stats = np.zeros(2, dtype=np.uint64)
        self.calls = 0

    def _newest_loc(self, seq: np.ndarray) -> np.ndarray:
        r = self.req_rows
        if self.slot_rows is not None:
            return self.slot_rows[r, self.cfg.H].astype(np.int64)
        return (r * self.cfg.S_r + self.cfg.H).astype(np.int64)

    def write_newest(self, seq: np.ndarray) -> None:
        """The caller's KV update: newest token's pool row into slot H (both sides)."""
        valid = (self.req_rows >= 0) & (self.req_rows < self.R)
        r = self.req_rows[valid]
        s = seq[valid]
        if self.pool_rows is not None:
            prow = self.pool_rows[r, s - 1]
        else:
            prow = r * self.cfg.ctx + s - 1
        loc = self._newest_loc(seq)[valid]
        keep = (prow >= 0) & (prow < self.pool_np.shape[0])
        prow, loc = prow[keep], loc[keep]
        if len(loc) == 0:
            return
        src_np = np.ascontiguousarray(self.pool_np[prow])
        oracle.store_kv_scatter(src_np, self.o_hot, np.ascontiguousarray(loc))
        hs.store_kv_scatter(src=torch.as_tensor(src_np).cuda(), dst=self.st.hot,
                            loc=torch.as_tensor(loc).cuda())

    def step(self, topk: np.ndarray, seq: np.ndarray, *, num_real: int = -1,
             topk_pad: int = 0, check_invariants: bool = False):
        cfg = self.cfg
        self.write_newest(seq)
        if topk_pad:
            padded = np.full((topk.shape[0], topk.shape[1] + topk_pad), -7, dtype=np.int32)
            padded[:, :topk.shape[1]] = topk
            topk_dev = torch.as_tensor(padded).cuda()[:, :topk.shape[1]]
        else:
            topk_dev = torch.as_tensor(topk).cuda()
        before = None
        if check_invariants:
            before = (self.o_tokens.copy(), self.o_lru.copy(), self.o_hot.copy())
        hs.hisparse_swap_in(
            topk=topk_dev, req_rows=torch.as_tensor(self.req_rows).cuda(),
            seq_lens=torch.as_tensor(seq).cuda(), slot_tokens=self.st.slot_tokens, lru=self.st.lru,
            pool=self.pool_t, hot=self.st.hot, out_rows=self.st.out, ctx_stride=cfg.ctx,
            workspace=self.st.ws, miss_counts=self.st.counts,
            num_real=None if num_real < 0 else torch.tensor([num_real], dtype=torch.int32).cuda(),
            slot_rows=self.slot_rows_t, pool_rows=self.pool_rows_t, stats=self.stats)
        o_out, o_cnt = oracle.swap_in(
            topk=topk, req_rows=self.req_rows, seq_lens=seq, slot_tokens=self.o_tokens,
            lru=self.o_lru, pool=self.pool_np, hot=self.o_hot, ctx_stride=cfg.ctx,
            num_real=num_real, slot_rows=self.slot_rows, pool_rows=self.pool_rows,
            stats=self.o_stats)
        torch.cuda.synchronize()
        tag = f"{cfg.name} call {self.calls}"
        assert_equal(f"{tag} out_rows", self.st.out.cpu().numpy(), o_out)
        assert_equal(f"{tag} miss_counts", self.st.counts.cpu().numpy(), o_cnt)
        assert_equal(f"{tag} slot_tokens", self.st.slot_tokens.cpu().numpy(), self.o_tokens)
        assert_equal(f"{tag} lru", self.st.lru.cpu().numpy(), self.o_lru)
        assert_equal(f"{tag} stats", self.stats.cpu().numpy().astype(np.uint64), self.o_stats)
        assert_equal(f"{tag} hot buffer", self.st.hot.cpu().numpy(), self.o_hot)
        if check_invariants:
            from invariants import check_swap_step
            check_swap_step(topk=topk, req_rows=self.req_rows, seq_lens=seq, num_real=num_real,
                            ctx_stride=cfg.ctx, pool=self.pool_np, tokens_before=before[0],
                            lru_before=before[1], hot_before=before[2], tokens_after=self.o_tokens,
                            lru_after=self.o_lru, hot_after=self.o_hot, out=o_out, counts=o_cnt,
                            slot_rows=self.slot_rows, pool_rows=self.pool_rows)
        self.calls += 1
        return o_out, o_cnt


def run_trace(cfg: gen.SwapConfig, steps: Optional[int] = None,
              check_invariants: bool = False, **kw) -> np.ndarray:
    """Every step of the workload's trace, with the whole hot buffer compared
    after each call."""
    steps = cfg.steps if steps is None else steps
    run = ParityRun(cfg, **kw)
    counts = []
    for t, topk in enumerate(gen.topk_trace(cfg, steps)):
        seq = gen.seq_lens(cfg, t)
        _, c = run.step(topk, seq, check_invariants=check_invariants)
        counts.append(c)
        log(f"  {cfg.name} step {t}: misses {int(c.sum())} ok")
    return np.asarray(counts)
