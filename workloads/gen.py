"""Seeded synthetic inputs for the HiSparse swap-in and the all-layer row transfer.

This module only draws inputs. It holds none of the swap-in arithmetic: no
hashing of keys into tables, no LRU order, no victim choice. Both the GPU path
and the CPU oracle are fed the same arrays from here, so neither side generates
anything the other must reproduce.

What is generated (the pages give shapes only, no traces, so every trace here
is a stand-in for an indexer's top-k output):

* Pool bytes. Rows are opaque (the vLLM page's header comment says the kernels
  move bytes and are dtype agnostic). Row ``p`` of a pool is a slice of the
  byte stream ``numpy.random.default_rng([seed, p // POOL_CHUNK_ROWS]).bytes``,
  so any row can be regenerated on its own without the whole pool.
* Per-step top-k ids. Step 0 draws ``K`` distinct ids from the workload's
  new-id distribution over ``[0, L_t)``. Each later step keeps
  ``round(rho*K)`` ids drawn without replacement from the previous step's set
  and fills up with fresh distinct ids from the distribution. Each row is then
  shuffled, because an indexer emits ids in score order, not position order.
* Sequence lengths. One decode step adds one token: ``L_t = ctx - S + 1 + t``
  for step ``t`` of ``S``, so the last step sees the full context.
"""

from __future__ import annotations

import dataclasses
from typing import Iterator, List, Optional, Sequence

import numpy as np

POOL_CHUNK_ROWS = 4096

# Odd 32-bit multiplier of the Knuth multiplicative hash that both pages use
# (SGLang hisparse.cuh and vLLM hisparse_kernels.cu, `hash_slot`). Only the
# adversarial id sets below use it, to pick ids that collide in the pages'
# low-bit form `(id * A mod 2^32) mod size`.
KNUTH_A = 2654435761


@dataclasses.dataclass(frozen=True)
class SwapConfig:
    """One swap-in workload. Sizes follow the names of the pages' kernels."""

    name: str
    B: int                 # batch rows (requests) per call
    H: int                 # hot_size: LRU-managed slots per request
    K: int                 # top_k ids per request per step
    ctx: int               # context tokens per request (pool rows per request)
    row_bytes: int         # opaque KV row size
    steps: int             # decode steps in the trace
    rho: float             # fraction of ids kept from the previous step
    dist: str              # "uniform" | "zipf" | "collide"
    pool_kind: str         # "host" (pinned) | "device"
    seed: int
    zipf_s: float = 1.1
    collide_window: int = 1024      # buckets per request window ("collide")
    collide_table: int = 0          # table size the ids collide in (2*H)
    # "collide" with collide_high_bits > 0: buckets are the TOP collide_high_bits
    # bits of the 32-bit product instead (collide_table = 2**collide_high_bits),
    # the form the GPU kernel hashes with (its home bucket of an id)
    collide_high_bits: int = 0
    newest_every_odd: bool = False  # request 0 picks L_t-1 at odd steps

    @property
    def S_r(self) -> int:
        # region_stride: H LRU slots plus the newest-token slot at index H.
        return self.H + 1

    @property
    def R(self) -> int:
        return self.B

    @property
    def pool_nrows(self) -> int:
        return self.B * self.ctx

    def seq_len(self, t: int) -> int:
        return self.ctx - self.steps + 1 + t

    def with_(self, **kw) -> "SwapConfig":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class TransferConfig:
    """Fused all-layer indexed row transfer workload."""

    name: str
    layers: int
    rows_per_layer: int
    row_bytes: int
    n_pairs: int
    seed: int


TINY = SwapConfig("tiny", B=2, H=64, K=16, ctx=2048, row_bytes=656, steps=8,
                  rho=0.7, dist="uniform", pool_kind="host", seed=20260001,
                  newest_every_odd=True)
DSV32 = SwapConfig("dsv32_decode", B=32, H=4096, K=2048, ctx=32768, row_bytes=656,
                   steps=64, rho=0.85, dist="zipf", pool_kind="host", seed=20260002)
DEVPOOL = SwapConfig("device_pool", B=128, H=4096, K=2048, ctx=16384, row_bytes=656,
                     steps=32, rho=0.6, dist="uniform", pool_kind="device",
                     seed=20260003)
ALL_LAYER = TransferConfig("all_layer", layers=61, rows_per_layer=262144,
                           row_bytes=656, n_pairs=8192, seed=20260004)
ADVERSARIAL = SwapConfig("adversarial", B=64, H=8192, K=2048, ctx=65536,
                         row_bytes=1152, steps=4, rho=0.5, dist="collide",
                         pool_kind="host", seed=20260005, collide_table=16384)
ADVERSARIAL_132 = ADVERSARIAL.with_(name="adversarial_132", row_bytes=132)
# The adversarial shape with ids that collide in the GPU kernel's own hash: at
# top_k 2048 the kernel's LDS table has 8192 entries in 2048 buckets of four,
# and an id's home bucket is the top 11 bits of id * 2654435761 (mod 2^32). A
# window of 128 of those buckets holds about 4096 ids of a 65,536-token
# context, the same 1/16 share as the low-bit window above.
ADVERSARIAL_KERNEL_HASH = ADVERSARIAL.with_(name="adversarial_kernel_hash", collide_high_bits=11,
                                            collide_table=2048, collide_window=128)
# Non-MLA caches (K and V rows per token): the DeepSeek-V3.2-like decode shape
# with 1024-byte rows, as for 4 KV heads x 128 dims x 2 bytes.
KV_DECODE = DSV32.with_(name="kv_decode", row_bytes=1024, seed=20260006)

SWAP_CONFIGS = {c.name: c for c in (TINY, DSV32, DEVPOOL, ADVERSARIAL, ADVERSARIAL_132,
                                    ADVERSARIAL_KERNEL_HASH)}


# --------------------------------------------------------------------------
# pool bytes
# --------------------------------------------------------------------------

def pool_rows_bytes(seed: int, first_row: int, nrows: int, row_bytes: int,
                    out: Optional[np.ndarray] = None) -> np.ndarray:
    """Bytes of pool rows ``[first_row, first_row + nrows)`` as ``uint8[nrows, row_bytes]``."""
    if out is None:
        out = np.empty((nrows, row_bytes), dtype=np.uint8)
    assert out.shape == (nrows, row_bytes) and out.dtype == np.uint8
    p = first_row
    end = first_row + nrows
    while p < end:
        chunk = p // POOL_CHUNK_ROWS
        c0 = chunk * POOL_CHUNK_ROWS
        stream = np.frombuffer(
            np.random.default_rng([seed, chunk]).bytes(POOL_CHUNK_ROWS * row_bytes),
            dtype=np.uint8).reshape(POOL_CHUNK_ROWS, row_bytes)
        take = min(end, c0 + POOL_CHUNK_ROWS) - p
        out[p - first_row:p - first_row + take] = stream[p - c0:p - c0 + take]
        p += take
    return out


def fill_pool(seed: int, out: np.ndarray) -> np.ndarray:
    """Fill a whole ``uint8[nrows, row_bytes]`` pool (any writable array, e.g. pinned)."""
    nrows, row_bytes = out.shape
    step = POOL_CHUNK_ROWS * 16
    for p in range(0, nrows, step):
        n = min(step, nrows - p)
        pool_rows_bytes(seed, p, n, row_bytes, out=out[p:p + n])
    return out


# --------------------------------------------------------------------------
# top-k traces
# --------------------------------------------------------------------------

def _zipf_cdf(L: int, s: float) -> np.ndarray:
    k = np.arange(1, L + 1, dtype=np.float64)
    return np.cumsum(k ** (-s))


def _collide_candidates(cfg: SwapConfig, L: int, window_start: int) -> np.ndarray:
    """Ids in [0, L) whose multiplicative bucket falls in
    ``[window_start, window_start + collide_window)`` (wrapping): the low-bit
    bucket ``(id*A mod 2^32) mod collide_table`` of the pages' hash, or with
    ``collide_high_bits`` the top bits ``(id*A mod 2^32) >> (32 - collide_high_bits)``."""
    ids = np.arange(L, dtype=np.uint64)
    prod = (ids * np.uint64(KNUTH_A)) & np.uint64(0xFFFFFFFF)
    if cfg.collide_high_bits:
        bucket = prod >> np.uint64(32 - cfg.collide_high_bits)
    else:
        bucket = prod % np.uint64(cfg.collide_table)
    rel = (bucket.astype(np.int64) - window_start) % cfg.collide_table
    return np.nonzero(rel < cfg.collide_window)[0].astype(np.int64)


class _RowStream:
    """Draws fresh ids for one request under the workload's distribution."""

    def __init__(self, cfg: SwapConfig, b: int):
        self.cfg = cfg
        self.rng = np.random.default_rng([cfg.seed, 1000 + b])
        self.window = int(self.rng.integers(0, max(1, cfg.collide_table))) if cfg.dist == "collide" else 0
        self._cdf_L = -1
        self._cdf = None
        self._cand_L = -1
        self._cand = None

    def draw(self, L: int, n: int) -> np.ndarray:
        cfg = self.cfg
        if cfg.dist == "uniform":
            return self.rng.integers(0, L, size=n, dtype=np.int64)
        if cfg.dist == "zipf":
            if self._cdf_L != L:
                self._cdf = _zipf_cdf(L, cfg.zipf_s)
                self._cdf_L = L
            u = self.rng.random(n) * self._cdf[-1]
            rank = np.searchsorted(self._cdf, u, side="right") + 1   # rank 1 = newest
            rank = np.minimum(rank, L)
            return (L - rank).astype(np.int64)
        if cfg.dist == "collide":
            if self._cand_L != L:
                self._cand = _collide_candidates(cfg, L, self.window)
                self._cand_L = L
            return self._cand[self.rng.integers(0, len(self._cand), size=n)]
        raise ValueError(cfg.dist)

    def fresh(self, L: int, n: int, exclude: set) -> List[int]:
        got: List[int] = []
        seen = set(exclude)
        while len(got) < n:
            for v in self.draw(L, max(64, 2 * (n - len(got)))).tolist():
                if v not in seen:
                    seen.add(v)
                    got.append(v)
                    if len(got) == n:
                        break
        return got


def topk_trace(cfg: SwapConfig, steps: Optional[int] = None) -> Iterator[np.ndarray]:
    """Yield ``int32[B, K]`` top-k ids for steps ``0 .. steps-1`` (default ``cfg.steps``).

    Steps beyond ``cfg.steps`` keep the last sequence length growing by one per step.
    """
    steps = cfg.steps if steps is None else steps
    streams = [_RowStream(cfg, b) for b in range(cfg.B)]
    prev: List[Optional[List[int]]] = [None] * cfg.B
    for t in range(steps):
        L = cfg.seq_len(t)
        out = np.empty((cfg.B, cfg.K), dtype=np.int32)
        for b in range(cfg.B):
            st = streams[b]
            if prev[b] is None:
                ids = st.fresh(L, cfg.K, set())
            else:
                keep_n = int(round(cfg.rho * cfg.K))
                keep = st.rng.choice(np.asarray(prev[b], dtype=np.int64), size=keep_n,
                                     replace=False).tolist()
                ids = keep + st.fresh(L, cfg.K - keep_n, set(keep))
            if cfg.newest_every_odd and b == 0 and t % 2 == 1 and (L - 1) not in ids:
                ids[-1] = L - 1
            prev[b] = list(ids)
            arr = np.asarray(ids, dtype=np.int64)
            st.rng.shuffle(arr)
            out[b] = arr.astype(np.int32)
        yield out


def seq_lens(cfg: SwapConfig, t: int) -> np.ndarray:
    return np.full(cfg.B, cfg.seq_len(t), dtype=np.int64)


def initial_state(cfg_or_R, H: Optional[int] = None, S_r: Optional[int] = None):
    """Empty tables (-1 everywhere, including the newest column) and identity LRU."""
    if isinstance(cfg_or_R, SwapConfig):
        R, H, S_r = cfg_or_R.R, cfg_or_R.H, cfg_or_R.S_r
    else:
        R = cfg_or_R
    slot_tokens = np.full((R, S_r), -1, dtype=np.int32)
    lru = np.tile(np.arange(H, dtype=np.int16), (R, 1))
    return slot_tokens, lru


# --------------------------------------------------------------------------
# all-layer transfer indices
# --------------------------------------------------------------------------

def transfer_indices(cfg: TransferConfig):
    rng = np.random.default_rng(cfg.seed)
    src = rng.permutation(cfg.rows_per_layer)[:cfg.n_pairs].astype(np.int64)
    dst = rng.permutation(cfg.rows_per_layer)[:cfg.n_pairs].astype(np.int64)
    return src, dst


def layer_seed(cfg: TransferConfig, layer: int) -> int:
    return cfg.seed * 1000 + layer


# --------------------------------------------------------------------------
# small random cases for unit tests
# --------------------------------------------------------------------------

def random_case(rng: np.random.Generator, *, B: int, R: int, H: int, K: int, ctx: int,
                n_invalid: int = 0, with_newest: bool = True,
                req_rows: Optional[Sequence[int]] = None):
    """One call's worth of ids for ``B`` rows: distinct valid ids, optional invalid
    ids (negative or >= L) and the newest token, with per-row lengths in [K+1, ctx]."""
    if req_rows is None:
        req_rows = rng.permutation(R)[:B]
    seq = rng.integers(K + 1, ctx + 1, size=B).astype(np.int64)
    topk = np.empty((B, K), dtype=np.int32)
    for b in range(B):
        L = int(seq[b])
        n_bad = min(n_invalid, K)
        want_new = with_newest and n_bad < K and rng.random() < 0.5
        n_valid = K - n_bad - (1 if want_new else 0)
        pool = np.arange(L - 1, dtype=np.int64)
        ids = list(rng.choice(pool, size=n_valid, replace=False))
        if want_new:
            ids.append(L - 1)
        for _ in range(n_bad):
            ids.append(int(rng.choice([-1 - int(rng.integers(0, 5)), L + int(rng.integers(0, 5))])))
        arr = np.asarray(ids, dtype=np.int64)
        rng.shuffle(arr)
        topk[b] = arr
    return np.asarray(req_rows, dtype=np.int64), seq, topk
