"""Device-side set-up of the synthetic workloads: allocation and filling of
pools, state, hot buffers and per-step inputs (plumbing only; every step of
the swap-in itself runs in libhisparse's kernels)."""

from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import gen


def pinned_uint8(rows: int, row_bytes: int) -> torch.Tensor:
    return torch.empty((rows, row_bytes), dtype=torch.uint8, pin_memory=True)


def make_pool(cfg: gen.SwapConfig, device: str = "cuda", kind: Optional[str] = None) -> torch.Tensor:
    """Pool of ``cfg.pool_nrows`` rows filled with the counter-based bytes, in pinned
    host memory (kind "host") or HBM (kind "device")."""
    kind = kind or cfg.pool_kind
    if kind == "host":
        pool = pinned_uint8(cfg.pool_nrows, cfg.row_bytes)
        gen.fill_pool(cfg.seed, pool.numpy())
        return pool
    pool = torch.empty((cfg.pool_nrows, cfg.row_bytes), dtype=torch.uint8, device=device)
    step = gen.POOL_CHUNK_ROWS * 64
    buf = pinned_uint8(step, cfg.row_bytes)
    for p in range(0, cfg.pool_nrows, step):
        n = min(step, cfg.pool_nrows - p)
        gen.pool_rows_bytes(cfg.seed, p, n, cfg.row_bytes, out=buf.numpy()[:n])
        pool[p:p + n].copy_(buf[:n], non_blocking=False)
    return pool


class DeviceSwapState:
    """Persistent per-request state, hot buffer, outputs and workspace on the GPU."""

    def __init__(self, cfg: gen.SwapConfig, device: str = "cuda", R: Optional[int] = None,
                 hot_nrows: Optional[int] = None):
        import sparse_attention_kv_hisparse_amd as hs
        self.cfg = cfg
        self.R = R or cfg.R
        self.slot_tokens = torch.empty((self.R, cfg.S_r), dtype=torch.int32, device=device)
        self.lru = torch.empty((self.R, cfg.H), dtype=torch.int16, device=device)
        hs.hisparse_state_reset(slot_tokens=self.slot_tokens, lru=self.lru,
                                rows=torch.arange(self.R, dtype=torch.int64, device=device))
        self.hot = torch.zeros((hot_nrows or self.R * cfg.S_r, cfg.row_bytes), dtype=torch.uint8,
                               device=device)
        self.out = torch.empty((cfg.B, cfg.K), dtype=torch.int32, device=device)
        self.counts = torch.empty(cfg.B, dtype=torch.int32, device=device)
        self.ws = torch.zeros(hs.swap_in_workspace_bytes(cfg.B, cfg.K), dtype=torch.uint8,
                              device=device)


def newest_rows_src(pool: torch.Tensor, cfg: gen.SwapConfig, req_rows: np.ndarray,
                    seq: np.ndarray, device: str = "cuda") -> torch.Tensor:
    """Pool rows of each request's newest token, as a device tensor the caller
    scatters into slot H with store_kv_scatter."""
    idx = torch.as_tensor(req_rows * cfg.ctx + seq - 1, dtype=torch.int64)
    if pool.is_cuda:
        return pool[idx.to(pool.device)].contiguous()
    return pool[idx].to(device)
