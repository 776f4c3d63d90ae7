"""ctypes declarations of libhisparse.so's C ABI (include/hisparse.h).

Loading never falls back to anything: if the library is missing or does not
load, every call raises.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libhisparse.so")

HS_OK = 0
HS_NOALLOC_SCRATCH_BYTES = 4 << 20   # include/hisparse.h
STATUS = {0: "HS_OK", -1: "HS_EINVAL", -2: "HS_ERANGE", -3: "HS_EMEMKIND", -4: "HS_ELAUNCH",
          -5: "HS_EWORKSPACE"}

# Every function include/hisparse.h declares.
EXPORTS = ("hs_swap_in_workspace_bytes", "hisparse_swap_in", "hisparse_swap_in_noalloc",
           "hisparse_resolve",
           "hisparse_gather_compact", "hisparse_gather_compact_layers",
           "hs_swap_in_workspace_layout", "transfer_rows_all_layer", "transfer_kv_all_layer",
           "hs_transfer_flags_for", "store_kv_scatter", "store_kv_cache",
           "hisparse_invalidate_written", "hisparse_state_reset", "hisparse_last_error")


class PagedAddressing(ctypes.Structure):
    """Mirror of ``hs_paged_addressing``."""

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


class SwapInArgs(ctypes.Structure):
    """Mirror of ``hs_swap_in_args``."""

    _fields_ = [
        ("B", ctypes.c_int32), ("K", ctypes.c_int32), ("H", ctypes.c_int32),
        ("S_r", ctypes.c_int64), ("R", ctypes.c_int64),
        ("topk_ids", ctypes.c_void_p), ("topk_stride", ctypes.c_int64),
        ("req_rows", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("num_real", ctypes.c_void_p),
        ("slot_tokens", ctypes.c_void_p), ("lru", ctypes.c_void_p),
        ("slot_rows", ctypes.c_void_p), ("pool_rows", ctypes.c_void_p),
        ("ctx_stride", ctypes.c_int64),
        ("pool", ctypes.c_void_p), ("pool_nrows", ctypes.c_int64),
        ("hot", ctypes.c_void_p), ("hot_nrows", ctypes.c_int64),
        ("row_bytes", ctypes.c_int64),
        ("out_rows", ctypes.c_void_p), ("miss_counts", ctypes.c_void_p),
        ("miss_mask", ctypes.c_void_p),
        ("pool_v", ctypes.c_void_p), ("hot_v", ctypes.c_void_p),
        ("paged", ctypes.POINTER(PagedAddressing)),
        ("stats", ctypes.c_void_p),
    ]


class HisparseError(RuntimeError):
    def __init__(self, call: str, status: int, message: str):
        super().__init__(f"{call} failed: {STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() or "
                           f"python sparse_attention_kv_hisparse_amd/build.py")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.hs_swap_in_workspace_bytes.argtypes = [i32, i32]
    lib.hs_swap_in_workspace_bytes.restype = sz
    for name in ("hisparse_swap_in", "hisparse_resolve", "hisparse_gather_compact"):
        getattr(lib, name).argtypes = [ctypes.POINTER(SwapInArgs), vp, sz, vp]
        getattr(lib, name).restype = ctypes.c_int
    lib.hisparse_swap_in_noalloc.argtypes = [ctypes.POINTER(SwapInArgs), vp]
    lib.hisparse_swap_in_noalloc.restype = ctypes.c_int
    lib.hisparse_gather_compact_layers.argtypes = [vp, sz, i32, i32, vp, i64, vp, i64, i32, i64, vp]
    lib.hisparse_gather_compact_layers.restype = ctypes.c_int
    szp = ctypes.POINTER(ctypes.c_size_t)
    lib.hs_swap_in_workspace_layout.argtypes = [i32, i32, szp, szp, szp]
    lib.hs_swap_in_workspace_layout.restype = sz
    u32 = ctypes.c_uint32
    lib.transfer_rows_all_layer.argtypes = [vp, vp, vp, vp, i64, i32, i64, i64, i64, u32, vp]
    lib.transfer_rows_all_layer.restype = ctypes.c_int
    lib.store_kv_scatter.argtypes = [vp, i64, vp, i64, i64, vp, i64, i64, vp]
    lib.store_kv_scatter.restype = ctypes.c_int
    lib.transfer_kv_all_layer.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i64, i64, i64, u32, vp]
    lib.transfer_kv_all_layer.restype = ctypes.c_int
    lib.hs_transfer_flags_for.argtypes = [vp, vp, ctypes.POINTER(u32)]
    lib.hs_transfer_flags_for.restype = ctypes.c_int
    lib.store_kv_cache.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, i64, vp, i64, i64, vp]
    lib.store_kv_cache.restype = ctypes.c_int
    lib.hisparse_invalidate_written.argtypes = [vp, i64, i64, vp, vp, i64, vp]
    lib.hisparse_invalidate_written.restype = ctypes.c_int
    lib.hisparse_state_reset.argtypes = [vp, vp, vp, i64, i32, i64, i64, vp]
    lib.hisparse_state_reset.restype = ctypes.c_int
    lib.hisparse_last_error.argtypes = []
    lib.hisparse_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(call: str, status: int) -> None:
    if status != HS_OK:
        msg = load().hisparse_last_error()
        raise HisparseError(call, status, msg.decode() if msg else "")
