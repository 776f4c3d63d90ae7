"""MI355X HiSparse swap-in: Python binding of libhisparse.so.

Argument marshalling only. Each function takes torch tensors, checks the
dtype, device, contiguity and shape of every tensor against the sizes the call
derives (B, K, R, H, S_r, ctx_stride, n), raising ValueError before anything
is enqueued, and calls the C ABI of ``include/hisparse.h`` on torch's current
HIP stream. A tensor too small for the pointer the library is handed would
otherwise be read or written out of bounds on the device. All work runs in the
library's HIP kernels; nothing here computes, and nothing falls back.
"""

from __future__ import annotations

import ctypes
from typing import Optional

import torch

from ._lib import EXPORTS, HisparseError, PagedAddressing, SwapInArgs, check, load

__all__ = ["hisparse_swap_in", "hisparse_swap_in_noalloc", "SwapInCall", "hisparse_resolve", "hisparse_gather_compact",
           "hisparse_gather_compact_layers", "transfer_kv_all_layer", "store_kv_cache",
           "hisparse_invalidate_written",
           "swap_in_workspace_layout", "transfer_rows_all_layer", "transfer_host_link", "store_kv_scatter",
           "hisparse_state_reset", "swap_in_workspace_bytes", "HisparseError", "load", "EXPORTS"]


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _opt(t: Optional[torch.Tensor], dtype, name) -> Optional[int]:
    return None if t is None else _dev(t, dtype, name)


def _vec(t: Optional[torch.Tensor], n: int, name: str) -> None:
    """A contiguous 1-D tensor of at least n elements (or None)."""
    if t is not None and (t.dim() != 1 or not t.is_contiguous() or t.numel() < n):
        raise ValueError(f"{name} must be a contiguous 1-D tensor of at least {n} elements, "
                         f"got shape {tuple(t.shape)}")


def _mat(t: Optional[torch.Tensor], rows: int, cols: int, name: str) -> None:
    """A contiguous 2-D tensor of at least `rows` rows and exactly `cols` columns (or None)."""
    if t is not None and (t.dim() != 2 or not t.is_contiguous() or t.shape[0] < rows
                          or t.shape[1] != cols):
        raise ValueError(f"{name} must be a contiguous [>={rows}, {cols}] tensor, "
                         f"got shape {tuple(t.shape)}")


def swap_in_workspace_bytes(B: int, K: int) -> int:
    return int(load().hs_swap_in_workspace_bytes(B, K))


def swap_in_workspace_layout(B: int, K: int) -> dict:
    """Byte offsets of the miss list in the workspace: count int32[B], src int64[B,K],
    dst int32[B,K] (``hs_swap_in_workspace_layout``)."""
    c, s_, d = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    total = load().hs_swap_in_workspace_layout(B, K, ctypes.byref(c), ctypes.byref(s_), ctypes.byref(d))
    return {"count": c.value, "src": s_.value, "dst": d.value, "total": int(total)}


def hisparse_swap_in(*, topk: torch.Tensor, req_rows: torch.Tensor, seq_lens: torch.Tensor,
                     slot_tokens: torch.Tensor, lru: torch.Tensor, pool: torch.Tensor,
                     hot: torch.Tensor, out_rows: torch.Tensor, ctx_stride: int,
                     workspace: Optional[torch.Tensor], miss_counts: Optional[torch.Tensor] = None,
                     num_real: Optional[torch.Tensor] = None,
                     slot_rows: Optional[torch.Tensor] = None,
                     pool_rows: Optional[torch.Tensor] = None,
                     miss_mask: Optional[torch.Tensor] = None,
                     pool_v: Optional[torch.Tensor] = None, hot_v: Optional[torch.Tensor] = None,
                     paged: Optional[dict] = None, stats: Optional[torch.Tensor] = None,
                     stream=None, _entry: str = "hisparse_swap_in", _prepare_only: bool = False):
    """One decode-step swap-in (``hisparse_swap_in`` in include/hisparse.h).

    topk int32 [B, >=K] (rows may be strided), req_rows/seq_lens int64 [B],
    slot_tokens int32 [R, S_r], lru int16 [R, H], pool uint8 [rows, row_bytes]
    (pinned host or device), hot uint8 [rows, row_bytes] (device), out_rows int32 [B, K],
    workspace uint8 device tensor of at least ``swap_in_workspace_bytes(B, K)`` bytes,
    miss_mask int32 [B, K] (optional output: 1 where the entry missed and got a slot),
    pool_v / hot_v (non-MLA caches, both or neither): the V pool and V hot buffer, shaped
    and placed like pool / hot.
    paged (vLLM-style addressing): dict with ``hot_block_table`` int32 [R, n] and
    ``hot_block_size``; optionally ``src_block_table`` int32 [R, n] + ``src_block_size``,
    ``resident_block_table`` int32 [R, n] + ``resident_block_size`` + ``resident_null_block``,
    ``attention_indices`` int32 [B, >=K] output + ``attention_block_stride``. seq_lens may
    then be None and ctx_stride is unused.
    stats: int64 or uint64 device tensor of 2 elements (optional, in/out): the hits and
    misses of every real row are added to stats[0] and stats[1].
    """
    if (pool_v is None) != (hot_v is None):
        raise ValueError("pool_v and hot_v go together")
    if pool_v is not None:
        if pool_v.shape != pool.shape or hot_v.shape != hot.shape or pool_v.dtype != torch.uint8 \
                or hot_v.dtype != torch.uint8 or not pool_v.is_contiguous() or not hot_v.is_contiguous():
            raise ValueError("pool_v / hot_v must be contiguous uint8 shaped like pool / hot")
        if not hot_v.is_cuda:
            raise ValueError("hot_v must be a device tensor")
    if out_rows.dim() != 2:
        raise ValueError("out_rows must be [B, K]")
    B, K = out_rows.shape
    if topk.dim() != 2 or topk.shape[0] != B or topk.shape[1] < K or topk.stride(1) != 1:
        raise ValueError("topk must be [B, >=K] with contiguous columns")
    for t, n in ((slot_tokens, "slot_tokens"), (lru, "lru"), (out_rows, "out_rows")):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    if pool.dim() != 2 or hot.dim() != 2 or pool.shape[1] != hot.shape[1] or \
            not pool.is_contiguous() or not hot.is_contiguous():
        raise ValueError("pool and hot must be contiguous [rows, row_bytes] with equal row_bytes")
    if pool.dtype != torch.uint8 or hot.dtype != torch.uint8:
        raise ValueError("pool and hot are uint8 byte rows")
    if slot_tokens.dim() != 2 or lru.dim() != 2:
        raise ValueError("slot_tokens must be [R, S_r] and lru [R, H]")
    R, S_r = slot_tokens.shape
    H = lru.shape[1]
    if lru.shape[0] != R:
        raise ValueError(f"lru has {lru.shape[0]} rows, slot_tokens {R}")
    _vec(req_rows, B, "req_rows")
    _vec(seq_lens, B, "seq_lens")
    _vec(miss_counts, B, "miss_counts")
    _vec(num_real, 1, "num_real")
    _mat(slot_rows, R, S_r, "slot_rows")
    if pool_rows is not None:
        _mat(pool_rows, R, ctx_stride, "pool_rows")
    pg = None
    if paged is not None:
        def tab(name):
            t = paged.get(name)
            if t is None:
                return None, 0
            if t.dim() != 2 or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous 2-D int32 tensor")
            if t.shape[0] < R:   # tables are indexed by the state row
                raise ValueError(f"{name} must have a row for each of the {R} state rows")
            return t, t.shape[1]
        hbt, hst = tab("hot_block_table")
        sbt, sst = tab("src_block_table")
        rbt, rst = tab("resident_block_table")
        hbt = _opt(hbt, torch.int32, "hot_block_table")
        sbt = _opt(sbt, torch.int32, "src_block_table")
        rbt = _opt(rbt, torch.int32, "resident_block_table")
        att = paged.get("attention_indices")
        if att is not None and (att.dim() != 2 or att.shape[0] != B or not att.is_contiguous()):
            raise ValueError("attention_indices must be a contiguous [B, >=K] int32 tensor")
        pg = PagedAddressing(
            hot_block_table=hbt, hot_table_stride=hst, hot_block_size=paged["hot_block_size"],
            src_block_table=sbt, src_table_stride=sst, src_num_blocks=sst,
            src_block_size=paged.get("src_block_size", 1),
            resident_block_table=rbt, resident_table_stride=rst, resident_num_blocks=rst,
            resident_block_size=paged.get("resident_block_size", 1),
            resident_null_block=paged.get("resident_null_block", -1),
            attention_indices=_opt(att, torch.int32, "attention_indices"),
            attention_row_stride=0 if att is None else att.shape[1],
            attention_block_stride=paged.get("attention_block_stride", 0))
    if not hot.is_cuda:
        raise ValueError("hot must be a device tensor")
    a = SwapInArgs(
        B=B, K=K, H=H, S_r=S_r, R=R,
        topk_ids=_dev(topk, torch.int32, "topk"), topk_stride=topk.stride(0),
        req_rows=_dev(req_rows, torch.int64, "req_rows"),
        seq_lens=None if seq_lens is None else _dev(seq_lens, torch.int64, "seq_lens"),
        num_real=_opt(num_real, torch.int32, "num_real"),
        slot_tokens=_dev(slot_tokens, torch.int32, "slot_tokens"),
        lru=_dev(lru, torch.int16, "lru"),
        slot_rows=_opt(slot_rows, torch.int32, "slot_rows"),
        pool_rows=_opt(pool_rows, torch.int64, "pool_rows"),
        ctx_stride=ctx_stride, pool=pool.data_ptr(), pool_nrows=pool.shape[0],
        hot=hot.data_ptr(), hot_nrows=hot.shape[0], row_bytes=hot.shape[1],
        out_rows=_dev(out_rows, torch.int32, "out_rows"),
        miss_counts=_opt(miss_counts, torch.int32, "miss_counts"),
        miss_mask=_opt(miss_mask, torch.int32, "miss_mask"),
        pool_v=None if pool_v is None else pool_v.data_ptr(),
        hot_v=None if hot_v is None else hot_v.data_ptr(),
        paged=ctypes.pointer(pg) if pg is not None else None)
    if miss_mask is not None and (tuple(miss_mask.shape) != (B, K) or not miss_mask.is_contiguous()):
        raise ValueError("miss_mask must be a contiguous [B, K] int32 tensor")
    if stats is not None:
        if stats.dtype not in (torch.int64, torch.uint64) or stats.numel() != 2 or not stats.is_contiguous():
            raise ValueError("stats must be a contiguous 2-element int64 or uint64 tensor")
        a.stats = _dev(stats, stats.dtype, "stats")
    if _entry == "hisparse_swap_in_noalloc":
        ws = None
    else:
        ws = (_dev(workspace, torch.uint8, "workspace"), workspace.numel())
    if _prepare_only:
        return a, ws
    _launch(_entry, a, ws, stream)


def _launch(entry: str, a: SwapInArgs, ws, stream) -> None:
    if ws is None:
        check(entry, load().hisparse_swap_in_noalloc(ctypes.byref(a), _stream(stream)))
    else:
        check(entry, getattr(load(), entry)(ctypes.byref(a), ws[0], ws[1], _stream(stream)))


class SwapInCall:
    """A swap-in whose state, pool, hot buffer, outputs, workspace and options
    are fixed, for a loop of decode steps: every argument is checked once here,
    and each call checks and passes only the step's own tensors (top-k ids,
    request rows, sequence lengths), which keeps the host time per step small.

    Takes the keyword arguments of ``hisparse_swap_in`` except ``topk``,
    ``req_rows``, ``seq_lens`` and ``stream``; ``entry`` names the call
    (``hisparse_swap_in``, ``hisparse_resolve``, ``hisparse_gather_compact`` or
    ``hisparse_swap_in_noalloc``, which takes no workspace). The tensors given
    here must stay alive and keep their storage while the object is used.
    Call it as ``call(topk, req_rows, seq_lens=None, stream=None)``.
    """

    def __init__(self, *, entry: str = "hisparse_swap_in", **kw):
        if entry not in ("hisparse_swap_in", "hisparse_resolve", "hisparse_gather_compact",
                         "hisparse_swap_in_noalloc"):
            raise ValueError(f"unknown entry {entry}")
        for k in ("topk", "req_rows", "seq_lens", "stream", "_entry"):
            if k in kw:
                raise ValueError(f"{k} is given per call")
        if entry == "hisparse_swap_in_noalloc":
            if "workspace" in kw:
                raise ValueError("hisparse_swap_in_noalloc takes no workspace")
            kw["workspace"] = None
        out = kw["out_rows"]
        if out.dim() != 2:
            raise ValueError("out_rows must be [B, K]")
        B, K = out.shape
        dev = out.device
        self._B, self._K, self._entry = B, K, entry
        self._paged = kw.get("paged") is not None
        # placeholder step tensors: the full argument checks run once on them
        ph_topk = torch.zeros((B, K), dtype=torch.int32, device=dev)
        ph_rows = torch.zeros(B, dtype=torch.int64, device=dev)
        ph_seq = torch.zeros(B, dtype=torch.int64, device=dev)
        self._args, self._ws = hisparse_swap_in(topk=ph_topk, req_rows=ph_rows, seq_lens=ph_seq,
                                                _entry=entry, _prepare_only=True, **kw)
        self._keep = kw

    def __call__(self, topk: torch.Tensor, req_rows: torch.Tensor,
                 seq_lens: Optional[torch.Tensor] = None, stream=None) -> None:
        B, K = self._B, self._K
        if topk.dim() != 2 or topk.shape[0] != B or topk.shape[1] < K or topk.stride(1) != 1:
            raise ValueError("topk must be [B, >=K] with contiguous columns")
        _vec(req_rows, B, "req_rows")
        a = self._args
        a.topk_ids = _dev(topk, torch.int32, "topk")
        a.topk_stride = topk.stride(0)
        a.req_rows = _dev(req_rows, torch.int64, "req_rows")
        if seq_lens is None:
            if not self._paged:
                raise ValueError("seq_lens is required without paged addressing")
            a.seq_lens = None
        else:
            _vec(seq_lens, B, "seq_lens")
            a.seq_lens = _dev(seq_lens, torch.int64, "seq_lens")
        _launch(self._entry, a, self._ws, stream)


def hisparse_swap_in_noalloc(**kw) -> None:
    """``hisparse_swap_in_noalloc``: the swap-in without a workspace argument (for
    callers that cannot allocate); same arguments as ``hisparse_swap_in`` minus
    ``workspace``. The miss list lives in the library's fixed per-device array
    of ``HS_NOALLOC_SCRATCH_BYTES``; calls that overlap on one device race."""
    if "workspace" in kw:
        raise ValueError("hisparse_swap_in_noalloc takes no workspace")
    hisparse_swap_in(_entry="hisparse_swap_in_noalloc", workspace=None, **kw)


def hisparse_resolve(**kw) -> None:
    """Resolution half of the swap-in (``hisparse_resolve``): same arguments as
    ``hisparse_swap_in``; leaves the miss list in the workspace, copies nothing."""
    hisparse_swap_in(_entry="hisparse_resolve", **kw)


def hisparse_gather_compact(**kw) -> None:
    """Copy half (``hisparse_gather_compact``): copies the rows a preceding
    ``hisparse_resolve`` with the same workspace listed."""
    hisparse_swap_in(_entry="hisparse_gather_compact", **kw)


def hisparse_gather_compact_layers(*, workspace: torch.Tensor, B: int, K: int,
                                   pool_layer_ptrs: torch.Tensor, pool_nrows: int,
                                   hot_layer_ptrs: torch.Tensor, hot_nrows: int, row_bytes: int,
                                   stream=None) -> None:
    """Replay the plan a preceding ``hisparse_resolve`` left in ``workspace`` on every
    layer pair; layer pointer arrays are device uint64 (torch int64) [L]."""
    L = pool_layer_ptrs.numel()
    if hot_layer_ptrs.numel() != L:
        raise ValueError("pool and hot layer pointer arrays must have equal lengths")
    check("hisparse_gather_compact_layers", load().hisparse_gather_compact_layers(
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), B, K,
        _dev(pool_layer_ptrs, torch.int64, "pool_layer_ptrs"), pool_nrows,
        _dev(hot_layer_ptrs, torch.int64, "hot_layer_ptrs"), hot_nrows, L, row_bytes,
        _stream(stream)))


HOST_LINK = 1   # HS_TRANSFER_HOST_LINK


def transfer_rows_all_layer(*, src_layer_ptrs: torch.Tensor, dst_layer_ptrs: torch.Tensor,
                            src_idx: torch.Tensor, dst_idx: torch.Tensor, row_bytes: int,
                            src_nrows: int, dst_nrows: int, host_link: bool = False,
                            stream=None) -> None:
    """All-layer indexed row copy; layer pointer arrays are device uint64 (torch int64) [L].
    ``host_link``: one side is pinned host memory (launch shaped for the host link)."""
    L = src_layer_ptrs.numel()
    if dst_layer_ptrs.numel() != L or src_idx.numel() != dst_idx.numel():
        raise ValueError("pointer arrays / index arrays must have equal lengths")
    for t, n in ((src_layer_ptrs, "src_layer_ptrs"), (dst_layer_ptrs, "dst_layer_ptrs"),
                 (src_idx, "src_idx"), (dst_idx, "dst_idx")):
        _vec(t, 0, n)
    check("transfer_rows_all_layer", load().transfer_rows_all_layer(
        _dev(src_layer_ptrs, torch.int64, "src_layer_ptrs"),
        _dev(dst_layer_ptrs, torch.int64, "dst_layer_ptrs"),
        _dev(src_idx, torch.int64, "src_idx"), _dev(dst_idx, torch.int64, "dst_idx"),
        src_idx.numel(), L, row_bytes, src_nrows, dst_nrows, HOST_LINK if host_link else 0,
        _stream(stream)))


def transfer_host_link(src_layer: torch.Tensor, dst_layer: torch.Tensor) -> bool:
    """Whether transfers between layers that live where ``src_layer`` and
    ``dst_layer`` do should take ``host_link=True`` (either side is pinned host
    memory). Reads the memory kind of the two tensors' storage; meant for
    once, where the caches are set up."""
    flags = ctypes.c_uint32(0)
    check("hs_transfer_flags_for", load().hs_transfer_flags_for(
        ctypes.c_void_p(src_layer.data_ptr()), ctypes.c_void_p(dst_layer.data_ptr()),
        ctypes.byref(flags)))
    return bool(flags.value & HOST_LINK)


def transfer_kv_all_layer(*, k_src_layer_ptrs: torch.Tensor, v_src_layer_ptrs: torch.Tensor,
                          k_dst_layer_ptrs: torch.Tensor, v_dst_layer_ptrs: torch.Tensor,
                          src_idx: torch.Tensor, dst_idx: torch.Tensor, row_bytes: int,
                          src_nrows: int, dst_nrows: int, host_link: bool = False,
                          stream=None) -> None:
    """K+V all-layer indexed row copy; the four layer pointer arrays are device
    uint64 (torch int64) [L]. ``host_link`` as for transfer_rows_all_layer."""
    L = k_src_layer_ptrs.numel()
    if not (v_src_layer_ptrs.numel() == k_dst_layer_ptrs.numel() == v_dst_layer_ptrs.numel() == L):
        raise ValueError("layer pointer arrays must have equal lengths")
    if src_idx.numel() != dst_idx.numel():
        raise ValueError("index arrays must have equal lengths")
    for t, n in ((k_src_layer_ptrs, "k_src_layer_ptrs"), (v_src_layer_ptrs, "v_src_layer_ptrs"),
                 (k_dst_layer_ptrs, "k_dst_layer_ptrs"), (v_dst_layer_ptrs, "v_dst_layer_ptrs"),
                 (src_idx, "src_idx"), (dst_idx, "dst_idx")):
        _vec(t, 0, n)
    check("transfer_kv_all_layer", load().transfer_kv_all_layer(
        _dev(k_src_layer_ptrs, torch.int64, "k_src_layer_ptrs"),
        _dev(v_src_layer_ptrs, torch.int64, "v_src_layer_ptrs"),
        _dev(k_dst_layer_ptrs, torch.int64, "k_dst_layer_ptrs"),
        _dev(v_dst_layer_ptrs, torch.int64, "v_dst_layer_ptrs"),
        _dev(src_idx, torch.int64, "src_idx"), _dev(dst_idx, torch.int64, "dst_idx"),
        src_idx.numel(), L, row_bytes, src_nrows, dst_nrows, HOST_LINK if host_link else 0,
        _stream(stream)))


def store_kv_cache(*, k_src: torch.Tensor, v_src: torch.Tensor, k_dst: torch.Tensor,
                   v_dst: torch.Tensor, loc: torch.Tensor, row_bytes: int = 0, stream=None) -> None:
    """``k_dst[loc[j]] = k_src[j]; v_dst[loc[j]] = v_src[j]`` for 2-D uint8 row tensors whose
    leading axes may be strided."""
    for t, n in ((k_src, "k_src"), (v_src, "v_src"), (k_dst, "k_dst"), (v_dst, "v_dst")):
        if t.dtype != torch.uint8 or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{n} must be a 2-D uint8 tensor with contiguous rows")
    if k_dst.shape[0] != v_dst.shape[0] or k_src.shape != v_src.shape:
        raise ValueError("K and V sides must have matching row counts")
    _vec(loc, 0, "loc")
    if loc.numel() > k_src.shape[0]:
        raise ValueError(f"loc has {loc.numel()} entries, the sources {k_src.shape[0]} rows")
    rb = row_bytes or k_src.shape[1]
    if rb > min(k_src.shape[1], k_dst.shape[1], v_dst.shape[1]):
        raise ValueError("row_bytes exceeds a row of the sources or destinations")
    check("store_kv_cache", load().store_kv_cache(
        _dev(k_src, torch.uint8, "k_src"), k_src.stride(0), _dev(v_src, torch.uint8, "v_src"),
        v_src.stride(0), _dev(k_dst, torch.uint8, "k_dst"), k_dst.stride(0),
        _dev(v_dst, torch.uint8, "v_dst"), v_dst.stride(0), k_dst.shape[0],
        _dev(loc, torch.int64, "loc"), loc.numel(), rb, _stream(stream)))


def store_kv_scatter(*, src: torch.Tensor, dst: torch.Tensor, loc: torch.Tensor, row_bytes: int = 0,
                     stream=None) -> None:
    """``dst[loc[j]] = src[j]`` for uint8 row tensors whose leading axis may be strided."""
    if src.dtype != torch.uint8 or dst.dtype != torch.uint8 or src.dim() != 2 or dst.dim() != 2:
        raise ValueError("src and dst are 2-D uint8 row tensors")
    if src.stride(1) != 1 or dst.stride(1) != 1:
        raise ValueError("rows must be contiguous")
    _vec(loc, 0, "loc")
    if loc.numel() > src.shape[0]:
        raise ValueError(f"loc has {loc.numel()} entries, src {src.shape[0]} rows")
    rb = row_bytes or src.shape[1]
    if rb > min(src.shape[1], dst.shape[1]):
        raise ValueError("row_bytes exceeds a row of src or dst")
    check("store_kv_scatter", load().store_kv_scatter(
        _dev(src, torch.uint8, "src"), src.stride(0), _dev(dst, torch.uint8, "dst"), dst.stride(0),
        dst.shape[0], _dev(loc, torch.int64, "loc"), loc.numel(), rb, _stream(stream)))


def hisparse_invalidate_written(*, slot_keys: torch.Tensor, rows: torch.Tensor,
                                written: torch.Tensor, stream=None) -> None:
    """Empty every slot of state row ``rows[j]`` whose global-id key is ``written[j]``."""
    if slot_keys.dim() != 2 or not slot_keys.is_contiguous():
        raise ValueError("slot_keys must be a contiguous [R, S_r] int32 tensor")
    if rows.numel() != written.numel():
        raise ValueError("rows and written must have equal lengths")
    _vec(rows, 0, "rows")
    _vec(written, 0, "written")
    R, S_r = slot_keys.shape
    check("hisparse_invalidate_written", load().hisparse_invalidate_written(
        _dev(slot_keys, torch.int32, "slot_keys"), R, S_r, _dev(rows, torch.int64, "rows"),
        _dev(written, torch.int64, "written"), rows.numel(), _stream(stream)))


def hisparse_state_reset(*, slot_tokens: torch.Tensor, lru: torch.Tensor, rows: torch.Tensor,
                         stream=None) -> None:
    """Initial state for state rows ``rows``: every slot token -1, LRU 0..H-1."""
    if slot_tokens.dim() != 2 or lru.dim() != 2 or not slot_tokens.is_contiguous() \
            or not lru.is_contiguous() or lru.shape[0] != slot_tokens.shape[0]:
        raise ValueError("slot_tokens [R, S_r] and lru [R, H] must be contiguous with R rows each")
    _vec(rows, 0, "rows")
    R, S_r = slot_tokens.shape
    check("hisparse_state_reset", load().hisparse_state_reset(
        _dev(slot_tokens, torch.int32, "slot_tokens"), _dev(lru, torch.int16, "lru"),
        _dev(rows, torch.int64, "rows"), rows.numel(), lru.shape[1], S_r, R, _stream(stream)))
