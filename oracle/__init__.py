"""HiSparse CPU oracle -- TEST INFRASTRUCTURE ONLY.

Python access to the plain C oracle in ``hisparse_oracle.c``. Only the tests,
``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may import
this package. The GPU library and its binding never do.

Every function takes and returns host numpy arrays. The swap-in updates the
caller's state arrays (``slot_tokens``, ``lru``, ``hot``) in place, as the GPU
call updates device state.

Parity pins (the tests under ``tests/test_oracle_*.py``):
  * an ``OrderedDict`` LRU model and, at top_k = 1, the textbook LRU cache;
  * closed forms for a cold start, a repeated step and a disjoint step;
  * invariants after every step of every workload trace;
  * hand-derived worked examples under ``tests/golden/``;
  * numpy fancy indexing for both row copies;
  * the plan: replaying a call's compact miss list on the hot buffer as it was
    before the call reproduces the call's hot buffer, the list agrees with the
    dense form (out_rows, miss_mask, each entry's pool row), and miss_mask
    marks exactly the ids the LRU model did not hold.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hisparse_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_hisparse.so")

ORACLE_OK = 0
ERRORS = {
    -1: "ORACLE_EARG", -2: "ORACLE_EDUP_ID", -3: "ORACLE_ELRU", -4: "ORACLE_EROWS",
    -5: "ORACLE_EHOT", -6: "ORACLE_ESTATE", -7: "ORACLE_EINDEX",
}


class OracleError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"oracle precondition failed: {ERRORS.get(code, code)}")
        self.code = code


_LIB_SANITIZED = os.path.join(_HERE, "liboracle_hisparse_sanitized.so")


def build(force: bool = False, sanitize: bool = False, out: Optional[str] = None) -> str:
    """Compile the oracle with gcc (plain C11, -O2). With ``sanitize`` the build
    is instrumented with AddressSanitizer and UndefinedBehaviorSanitizer (any
    report aborts) into a separate library (``out``, or one beside the plain
    build); a process loading it needs gcc's libasan and libubsan preloaded
    (``tests/test_sanitizers.py`` does this)."""
    lib = out or (_LIB_SANITIZED if sanitize else _LIB)
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < max(
            os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "hisparse_oracle.h"))):
        tmp = lib + ".tmp"
        extra = (["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                  "-fno-omit-frame-pointer", "-g"] if sanitize else [])
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-fPIC", "-shared",
                               *extra, "-o", tmp, _SRC])
        os.replace(tmp, lib)
    return lib


class _Paged(ctypes.Structure):
    _fields_ = [
        ("hot_block_table", ctypes.c_void_p), ("hot_table_stride", ctypes.c_int64),
        ("hot_block_size", ctypes.c_int32),
        ("src_block_table", ctypes.c_void_p), ("src_table_stride", ctypes.c_int64),
        ("src_num_blocks", ctypes.c_int32), ("src_block_size", ctypes.c_int32),
        ("resident_block_table", ctypes.c_void_p), ("resident_table_stride", ctypes.c_int64),
        ("resident_num_blocks", ctypes.c_int32), ("resident_block_size", ctypes.c_int32),
        ("resident_null_block", ctypes.c_int32),
        ("attention_indices", ctypes.c_void_p), ("attention_row_stride", ctypes.c_int64),
        ("attention_block_stride", ctypes.c_int64),
    ]


class _SwapArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("K", ctypes.c_int32), ("H", ctypes.c_int32),
        ("S_r", ctypes.c_int64), ("R", ctypes.c_int64),
        ("topk", ctypes.c_void_p), ("topk_stride", ctypes.c_int64),
        ("req_rows", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("num_real", ctypes.c_int32),
        ("slot_tokens", ctypes.c_void_p), ("lru", ctypes.c_void_p),
        ("slot_rows", ctypes.c_void_p), ("pool_rows", ctypes.c_void_p),
        ("ctx_stride", ctypes.c_int64),
        ("pool", ctypes.c_void_p), ("pool_nrows", ctypes.c_int64),
        ("hot", ctypes.c_void_p), ("hot_nrows", ctypes.c_int64),
        ("row_bytes", ctypes.c_int64),
        ("out_rows", ctypes.c_void_p), ("miss_counts", ctypes.c_void_p),
        ("miss_mask", ctypes.c_void_p), ("list_count", ctypes.c_void_p),
        ("list_src", ctypes.c_void_p), ("list_dst", ctypes.c_void_p),
        ("pool_v", ctypes.c_void_p), ("hot_v", ctypes.c_void_p),
        ("paged", ctypes.POINTER(_Paged)),
        ("stats", ctypes.c_void_p),
    ]


_lib = None


def _load(path: Optional[str] = None):
    global _lib
    if _lib is None or path is not None:
        lib = ctypes.CDLL(path or build())
        lib.oracle_swap_in.argtypes = [ctypes.POINTER(_SwapArgs)]
        lib.oracle_swap_in.restype = ctypes.c_int
        lib.oracle_transfer_rows_all_layer.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int64]
        lib.oracle_transfer_rows_all_layer.restype = ctypes.c_int64
        lib.oracle_store_kv_scatter.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64]
        lib.oracle_store_kv_scatter.restype = ctypes.c_int64
        lib.oracle_state_reset.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
            ctypes.c_int64, ctypes.c_int64]
        lib.oracle_state_reset.restype = ctypes.c_int
        lib.oracle_gather_compact_layers.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
            ctypes.c_int64]
        lib.oracle_gather_compact_layers.restype = ctypes.c_int64
        lib.oracle_transfer_kv_all_layer.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
            ctypes.c_int64]
        lib.oracle_transfer_kv_all_layer.restype = ctypes.c_int64
        lib.oracle_store_kv_cache.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64]
        lib.oracle_store_kv_cache.restype = ctypes.c_int64
        lib.oracle_invalidate_written.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64]
        lib.oracle_invalidate_written.restype = ctypes.c_int64
        _lib = lib
    return _lib


def use_library(path: Optional[str]) -> None:
    """Point this module at another build of the oracle source (the mutation
    tests load copies with planted mistakes); ``None`` returns to the real one."""
    global _lib
    _lib = None
    if path is not None:
        _load(path)


def _ptr(a: Optional[np.ndarray], dtype, writable: bool = False) -> Optional[int]:
    if a is None:
        return None
    assert a.dtype == dtype, (a.dtype, dtype)
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    if writable:
        assert a.flags["WRITEABLE"]
    return a.ctypes.data


def _rows_ptr(a: np.ndarray, dtype) -> int:
    """Pointer to a 2-D array whose rows may be strided but whose columns are contiguous."""
    assert a.dtype == dtype and a.ndim == 2 and (a.strides[1] == a.itemsize or a.shape[1] <= 1)
    if a.shape[0] > 1:
        assert a.strides[0] % a.itemsize == 0 and a.strides[0] >= a.shape[1] * a.itemsize
    return a.ctypes.data


def _row_stride(a: np.ndarray) -> int:
    return a.strides[0] // a.itemsize if a.shape[0] > 1 else a.shape[1]


def swap_in(*, topk: np.ndarray, req_rows: np.ndarray, seq_lens: np.ndarray,
            slot_tokens: np.ndarray, lru: np.ndarray, pool: np.ndarray, hot: np.ndarray,
            ctx_stride: int, num_real: int = -1, slot_rows: Optional[np.ndarray] = None,
            pool_rows: Optional[np.ndarray] = None, out_rows: Optional[np.ndarray] = None,
            miss_counts: Optional[np.ndarray] = None, plan: bool = False,
            pool_v: Optional[np.ndarray] = None, hot_v: Optional[np.ndarray] = None,
            paged: Optional[dict] = None, stats: Optional[np.ndarray] = None):
    """One swap-in call on host state; returns ``(out_rows int32[B,K], miss_counts int32[B])``,
    and with ``plan=True`` a third item: the plan index-sharing layers replay,
    ``{"miss_mask": int32[B,K], "count": int32[B], "src": int64[B,K], "dst": int32[B,K]}``
    (the compact miss list in miss order; entries past ``count[b]`` are unspecified).

    ``pool`` and ``hot`` are ``uint8[nrows, row_bytes]``. State arrays are updated in place.
    ``pool_v``/``hot_v`` (non-MLA caches, both or neither) have the same shapes as
    ``pool``/``hot``; every miss copies its V row too.
    ``paged`` selects vLLM-style addressing (global-id keys, block tables), a dict with
    ``hot_block_table`` int32 [R, n] and ``hot_block_size``, and optionally
    ``src_block_table`` int32 [R, n] + ``src_block_size``, ``resident_block_table`` int32
    [R, n] + ``resident_block_size`` + ``resident_null_block``, ``attention_indices`` int32
    [B, K] (output) + ``attention_block_stride``; ``seq_lens`` and ``ctx_stride`` are unused.
    ``stats`` (uint64[2], in/out): every real row adds its hits and its misses.
    """
    assert (pool_v is None) == (hot_v is None)
    if pool_v is not None:
        assert pool_v.shape == pool.shape and hot_v.shape == hot.shape
    B, K = topk.shape
    R, S_r = slot_tokens.shape
    H = lru.shape[1]
    assert lru.shape[0] == R and pool.shape[1] == hot.shape[1]
    if out_rows is None:
        out_rows = np.empty((B, K), dtype=np.int32)
    if miss_counts is None:
        miss_counts = np.empty(B, dtype=np.int32)
    p = None
    if plan:
        p = {"miss_mask": np.empty((B, K), np.int32), "count": np.empty(B, np.int32),
             "src": np.zeros((B, K), np.int64), "dst": np.zeros((B, K), np.int32)}
    pg = None
    if paged is not None:
        hbt = paged["hot_block_table"]
        sbt = paged.get("src_block_table")
        rbt = paged.get("resident_block_table")
        att = paged.get("attention_indices")
        pg = _Paged(hot_block_table=_ptr(hbt, np.int32), hot_table_stride=hbt.shape[1],
                    hot_block_size=paged["hot_block_size"],
                    src_block_table=_ptr(sbt, np.int32),
                    src_table_stride=0 if sbt is None else sbt.shape[1],
                    src_num_blocks=0 if sbt is None else sbt.shape[1],
                    src_block_size=paged.get("src_block_size", 1),
                    resident_block_table=_ptr(rbt, np.int32),
                    resident_table_stride=0 if rbt is None else rbt.shape[1],
                    resident_num_blocks=0 if rbt is None else rbt.shape[1],
                    resident_block_size=paged.get("resident_block_size", 1),
                    resident_null_block=paged.get("resident_null_block", -1),
                    attention_indices=_ptr(att, np.int32, True),
                    attention_row_stride=0 if att is None else att.shape[1],
                    attention_block_stride=paged.get("attention_block_stride", 0))
    a = _SwapArgs(
        B=B, K=K, H=H, S_r=S_r, R=R,
        topk=_rows_ptr(topk, np.int32), topk_stride=_row_stride(topk),
        req_rows=_ptr(req_rows, np.int64),
        seq_lens=None if seq_lens is None else _ptr(seq_lens, np.int64),
        num_real=num_real,
        slot_tokens=_ptr(slot_tokens, np.int32, True), lru=_ptr(lru, np.int16, True),
        slot_rows=_ptr(slot_rows, np.int32), pool_rows=_ptr(pool_rows, np.int64),
        ctx_stride=ctx_stride,
        pool=_ptr(pool, np.uint8), pool_nrows=pool.shape[0],
        hot=_ptr(hot, np.uint8, True), hot_nrows=hot.shape[0],
        row_bytes=pool.shape[1],
        out_rows=_ptr(out_rows, np.int32, True), miss_counts=_ptr(miss_counts, np.int32, True),
        miss_mask=p and _ptr(p["miss_mask"], np.int32, True),
        list_count=p and _ptr(p["count"], np.int32, True),
        list_src=p and _ptr(p["src"], np.int64, True), list_dst=p and _ptr(p["dst"], np.int32, True),
        pool_v=_ptr(pool_v, np.uint8), hot_v=_ptr(hot_v, np.uint8, True),
        paged=ctypes.pointer(pg) if pg is not None else None,
        stats=None if stats is None else _ptr(stats, np.uint64, True))
    rc = _load().oracle_swap_in(ctypes.byref(a))
    if rc != ORACLE_OK:
        raise OracleError(rc)
    return (out_rows, miss_counts, p) if plan else (out_rows, miss_counts)


def gather_compact_layers(count: np.ndarray, src: np.ndarray, dst: np.ndarray,
                          pool_layers: Sequence[np.ndarray], hot_layers: Sequence[np.ndarray]) -> int:
    """Replay a compact miss plan (``count[B]``, ``src[B,K]``, ``dst[B,K]``) on every
    (pool, hot) layer pair; returns the number of hot rows zeroed for want of a
    source row."""
    B, K = src.shape
    L = len(pool_layers)
    assert len(hot_layers) == L and count.shape == (B,) and dst.shape == (B, K)
    rb = hot_layers[0].shape[1] if L else 1
    for pl, hl in zip(pool_layers, hot_layers):
        assert pl.shape[1] == rb and hl.shape[1] == rb
        assert pl.shape[0] == pool_layers[0].shape[0] and hl.shape[0] == hot_layers[0].shape[0]
    pp = (ctypes.c_void_p * max(L, 1))(*[_ptr(x, np.uint8) for x in pool_layers])
    hp = (ctypes.c_void_p * max(L, 1))(*[_ptr(x, np.uint8, True) for x in hot_layers])
    r = _load().oracle_gather_compact_layers(
        _ptr(count, np.int32), _ptr(src, np.int64), _ptr(dst, np.int32), B, K, pp,
        pool_layers[0].shape[0] if L else 0, hp, hot_layers[0].shape[0] if L else 0, L, rb)
    if r < 0:
        raise OracleError(int(r))
    return int(r)


def transfer_rows_all_layer(src_layers: Sequence[np.ndarray], dst_layers: Sequence[np.ndarray],
                            src_idx: np.ndarray, dst_idx: np.ndarray) -> int:
    """``dst_layers[l][dst_idx[i]] = src_layers[l][src_idx[i]]``; returns the pairs skipped."""
    L = len(src_layers)
    assert len(dst_layers) == L and L > 0
    rb = src_layers[0].shape[1]
    for s, d in zip(src_layers, dst_layers):
        assert s.shape[1] == rb and d.shape[1] == rb
        assert s.shape[0] == src_layers[0].shape[0] and d.shape[0] == dst_layers[0].shape[0]
    sp = (ctypes.c_void_p * L)(*[_ptr(s, np.uint8) for s in src_layers])
    dp = (ctypes.c_void_p * L)(*[_ptr(d, np.uint8, True) for d in dst_layers])
    r = _load().oracle_transfer_rows_all_layer(
        sp, dp, src_layers[0].shape[0], dst_layers[0].shape[0], _ptr(src_idx, np.int64),
        _ptr(dst_idx, np.int64), src_idx.shape[0], L, rb)
    if r < 0:
        raise OracleError(int(r))
    return int(r)


def transfer_kv_all_layer(k_src: Sequence[np.ndarray], v_src: Sequence[np.ndarray],
                          k_dst: Sequence[np.ndarray], v_dst: Sequence[np.ndarray],
                          src_idx: np.ndarray, dst_idx: np.ndarray) -> int:
    """K and V rows of every layer: ``k_dst[l][dst_idx[i]] = k_src[l][src_idx[i]]`` and the
    same for V; returns the pairs skipped."""
    L = len(k_src)
    assert len(v_src) == len(k_dst) == len(v_dst) == L and L > 0
    rb = k_src[0].shape[1]
    for x in list(k_src) + list(v_src):
        assert x.shape == k_src[0].shape
    for x in list(k_dst) + list(v_dst):
        assert x.shape == k_dst[0].shape and x.shape[1] == rb
    arr = lambda xs, w: (ctypes.c_void_p * L)(*[_ptr(x, np.uint8, w) for x in xs])
    r = _load().oracle_transfer_kv_all_layer(
        arr(k_src, False), arr(v_src, False), arr(k_dst, True), arr(v_dst, True),
        k_src[0].shape[0], k_dst[0].shape[0], _ptr(src_idx, np.int64), _ptr(dst_idx, np.int64),
        src_idx.shape[0], L, rb)
    if r < 0:
        raise OracleError(int(r))
    return int(r)


def store_kv_cache(k_src: np.ndarray, v_src: np.ndarray, k_dst: np.ndarray, v_dst: np.ndarray,
                   loc: np.ndarray) -> int:
    """``k_dst[loc[j]] = k_src[j]`` and ``v_dst[loc[j]] = v_src[j]`` over rows of
    ``k_src.shape[1]`` bytes (row strides may differ per array); returns rows skipped."""
    n, rb = k_src.shape
    assert v_src.shape == (n, rb) and k_dst.shape[0] == v_dst.shape[0]
    assert k_dst.shape[1] >= rb and v_dst.shape[1] >= rb
    for x in (k_src, v_src, k_dst, v_dst):
        assert x.strides[1] == 1
    r = _load().oracle_store_kv_cache(
        k_src.ctypes.data, k_src.strides[0], v_src.ctypes.data, v_src.strides[0],
        k_dst.ctypes.data, k_dst.strides[0], v_dst.ctypes.data, v_dst.strides[0], k_dst.shape[0],
        _ptr(loc, np.int64), n, rb)
    if r < 0:
        raise OracleError(int(r))
    return int(r)


def store_kv_scatter(src: np.ndarray, dst: np.ndarray, loc: np.ndarray) -> int:
    """``dst[loc[j]] = src[j]`` over rows of ``src.shape[1]`` bytes; returns rows skipped."""
    n, rb = src.shape
    assert dst.shape[1] >= rb and src.strides[1] == 1 and dst.strides[1] == 1
    r = _load().oracle_store_kv_scatter(
        src.ctypes.data, src.strides[0], dst.ctypes.data, dst.strides[0], dst.shape[0],
        _ptr(loc, np.int64), n, rb)
    if r < 0:
        raise OracleError(int(r))
    return int(r)


def invalidate_written(slot_keys: np.ndarray, rows: np.ndarray, written: np.ndarray) -> int:
    """Clear every slot of state row ``rows[j]`` that holds global row ``written[j]``;
    returns the number of slots cleared."""
    R, S_r = slot_keys.shape
    r = _load().oracle_invalidate_written(_ptr(slot_keys, np.int32, True), R, S_r,
                                          _ptr(rows, np.int64), _ptr(written, np.int64),
                                          rows.shape[0])
    if r < 0:
        raise OracleError(int(r))
    return int(r)


def state_reset(slot_tokens: np.ndarray, lru: np.ndarray, rows: Sequence[int]) -> None:
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    R, S_r = slot_tokens.shape
    rc = _load().oracle_state_reset(_ptr(slot_tokens, np.int32, True), _ptr(lru, np.int16, True),
                                    rows.ctypes.data, rows.shape[0], lru.shape[1], S_r, R)
    if rc != ORACLE_OK:
        raise OracleError(rc)
