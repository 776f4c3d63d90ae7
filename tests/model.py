"""Independent small models of the swap-in, used only to pin the C oracle.

``lru_model_swap_in`` restates the swap-in as operations on a
``collections.OrderedDict`` used as a textbook LRU cache:

* resident tokens are found through a plain ``dict`` (token -> slot);
* slots holding a requested token are hits and are set aside;
* the remaining slots form an LRU cache in their old order; each miss, in
  ascending top-k order, evicts the least recently used of them
  (``popitem(last=False)``) and re-inserts it as most recently used;
* the hits then go after all of them, keeping their old relative order.

Both pages place the freshly filled slots just before the hits and leave the
hits in their old relative order (SGLang ``load_cache_to_device_buffer_kernel``
and vLLM ``hisparse_resolve_residency_kernel``, LRU write-back), which is what
this sequence of cache operations produces. It shares no code with the oracle
and uses no sorting or index algebra.
"""

from __future__ import annotations

from collections import OrderedDict
from typing import Dict, List, Optional


def _paged_lookup(table, block_size, r, t):
    """Physical block of position t in row r of a block table, or None past its end."""
    if t < 0:
        return None
    blk = t // block_size
    if blk >= table.shape[1]:
        return None
    return int(table[r, blk])


def lru_model_swap_in(*, topk, req_rows, seq_lens, slot_tokens, lru, pool, hot, ctx_stride,
                      num_real=-1, slot_rows=None, pool_rows=None, plan=False, pool_v=None,
                      hot_v=None, paged=None):
    """Same contract as ``oracle.swap_in`` (numpy arrays updated in place). With
    ``plan=True`` also returns the plan: ``miss_mask`` [B,K] (1 for each entry
    whose token no slot held) and, per row, the list of (pool row, hot row)
    copies in the order they were made."""
    import numpy as np

    B, K = topk.shape
    R, S_r = slot_tokens.shape
    H = lru.shape[1]
    out = np.full((B, K), -1, dtype=np.int32)
    counts = np.zeros(B, dtype=np.int32)
    mask = np.zeros((B, K), dtype=np.int32)
    copies = [[] for _ in range(B)]

    def row_of(r, s):
        if paged is not None:
            bs = paged["hot_block_size"]
            return int(paged["hot_block_table"][r, s // bs]) * bs + s % bs
        return int(slot_rows[r, s]) if slot_rows is not None else r * S_r + s

    def global_id(r, t):
        """vLLM addressing: (global id or None, resident row or None)."""
        g = t
        if paged.get("src_block_table") is not None:
            bs = paged["src_block_size"]
            p = _paged_lookup(paged["src_block_table"], bs, r, t)
            g = p * bs + t % bs if (p is not None and p > 0) else None
        if g is not None and g >= pool.shape[0]:
            g = None
        res = None
        if paged.get("resident_block_table") is not None:
            bs = paged["resident_block_size"]
            p = _paged_lookup(paged["resident_block_table"], bs, r, t)
            if p is not None and p >= 0 and p != paged["resident_null_block"]:
                res = p * bs + t % bs
            if res is not None and res >= 2**31:      # no int32 output can hold it
                res = None
        return g, res

    def pool_of(r, t):
        return int(pool_rows[r, t]) if pool_rows is not None else r * ctx_stride + t

    nreal = B if num_real < 0 else min(num_real, B)
    for b in range(B):
        r = int(req_rows[b])
        if b >= nreal or not (0 <= r < R):
            continue
        wanted: Dict[int, int] = {}
        if paged is not None:
            # keys are global ids; resident entries are served in place
            for i in range(K):
                g, res = global_id(r, int(topk[b, i]))
                if res is not None:
                    out[b, i] = res
                elif g is not None:
                    assert g not in wanted, "duplicate id"
                    wanted[g] = i
            L = None
        else:
            L = int(seq_lens[b])
        for i in range(K if paged is None else 0):
            t = int(topk[b, i])
            if not (0 <= t < L and t < ctx_stride):
                continue
            if not (0 <= pool_of(r, t) < pool.shape[0]):
                continue
            if t == L - 1:
                out[b, i] = row_of(r, H)
                continue
            assert t not in wanted, "duplicate id"
            wanted[t] = i
        where = {int(slot_tokens[r, s]): s for s in range(H) if slot_tokens[r, s] >= 0}
        hit_slots = set()
        for t, i in wanted.items():
            if t in where:
                out[b, i] = row_of(r, where[t])
                hit_slots.add(where[t])
        order = [int(s) for s in lru[r]]
        cache: "OrderedDict[int, None]" = OrderedDict((s, None) for s in order if s not in hit_slots)
        misses = sorted(i for t, i in wanted.items() if t not in where)
        key_of = {i: t for t, i in wanted.items()}
        for i in misses:
            t = key_of[i]
            v, _ = cache.popitem(last=False)
            cache[v] = None
            slot_tokens[r, v] = t
            src = t if paged is not None else pool_of(r, t)
            hot[row_of(r, v)] = pool[src]
            if pool_v is not None:
                hot_v[row_of(r, v)] = pool_v[src]
            out[b, i] = row_of(r, v)
            mask[b, i] = 1
            copies[b].append((src, row_of(r, v)))
        lru[r] = np.asarray(list(cache) + [s for s in order if s in hit_slots], dtype=np.int16)
        counts[b] = len(misses)
    if plan:
        return out, counts, {"miss_mask": mask, "copies": copies}
    return out, counts


class TextbookLRU:
    """Classic LRU cache of ``capacity`` tokens over an OrderedDict (token -> None).

    A hit moves the token to the most-recently-used end; a miss inserts it there
    and, when full, evicts the least recently used token.
    """

    def __init__(self, capacity: int):
        self.capacity = capacity
        self.d: "OrderedDict[int, None]" = OrderedDict()

    def access(self, token: int) -> bool:
        if token in self.d:
            self.d.move_to_end(token)
            return True
        if len(self.d) == self.capacity:
            self.d.popitem(last=False)
        self.d[token] = None
        return False

    def resident(self) -> List[int]:
        return list(self.d)


def invert_rows(slot_rows, r: int, S_r: int) -> Optional[dict]:
    if slot_rows is None:
        return None
    return {int(slot_rows[r, s]): s for s in range(S_r)}
