"""Invariants of one swap-in call, checked on host copies of the state.

They restate what both pages' swap-in kernels promise, not how they compute it:

I1  every valid, non-newest top-k id is resident after the call: the slot its
    output names holds that token, and the slot's hot row holds the token's pool row;
I2  the newest token (seq_len-1) is served from slot H and nothing else is;
I3  each real LRU row is a permutation of [0, H);
I4  valid tokens in slots [0, H) of a region are distinct;
I5  hit slots do not move: their token and bytes are unchanged;
I6  miss_count == slots whose token changed == K - hits - newest - invalid;
I7  slots that were not victims keep their token and bytes;
I8  new LRU = stale evictables (old order) ++ filled slots (miss order) ++ hits (old order);
I10 the pool is unchanged (checked by the caller, which owns the pool);
I11 outputs within a row are distinct apart from -1;
plus: padding rows output -1 and count 0, their state and slot H never change.
"""

from __future__ import annotations

import numpy as np


def check_swap_step(*, topk, req_rows, seq_lens, num_real, ctx_stride, pool,
                    tokens_before, lru_before, hot_before,
                    tokens_after, lru_after, hot_after, out, counts,
                    slot_rows=None, pool_rows=None):
    B, K = topk.shape
    R, S_r = tokens_before.shape
    H = lru_before.shape[1]
    nreal = B if num_real < 0 else min(num_real, B)

    def row_of(r, s):
        return int(slot_rows[r, s]) if slot_rows is not None else r * S_r + s

    def pool_of(r, t):
        return int(pool_rows[r, t]) if pool_rows is not None else r * ctx_stride + t

    touched_rows = set()
    changed_hot_rows = set()
    for b in range(B):
        r = int(req_rows[b])
        if b >= nreal or not (0 <= r < R):
            assert (out[b] == -1).all(), f"padding row {b} must output -1"
            assert counts[b] == 0
            continue
        touched_rows.add(r)
        slot_of_row = {row_of(r, s): s for s in range(S_r)}
        L = int(seq_lens[b])
        # I3
        assert sorted(lru_after[r].tolist()) == list(range(H)), "I3: LRU not a permutation"
        # I4
        valid = tokens_after[r, :H][tokens_after[r, :H] >= 0]
        assert len(np.unique(valid)) == len(valid), "I4: duplicate resident token"
        # slot H is never written by the swap-in
        assert tokens_after[r, H:].tolist() == tokens_before[r, H:].tolist()
        before_where = {int(tokens_before[r, s]): s for s in range(H) if tokens_before[r, s] >= 0}
        n_hit = n_new = n_bad = 0
        hit_slots, fill = set(), {}
        for i in range(K):
            t = int(topk[b, i])
            ok = 0 <= t < L and t < ctx_stride and 0 <= pool_of(r, t) < pool.shape[0]
            if not ok:
                assert out[b, i] == -1, "invalid id must output -1"
                n_bad += 1
                continue
            if t == L - 1:
                assert out[b, i] == row_of(r, H), "I2: newest must map to slot H"
                n_new += 1
                continue
            s = slot_of_row.get(int(out[b, i]))
            assert s is not None and s < H, "output must name an LRU slot"
            # I1
            assert tokens_after[r, s] == t, "I1: token not resident where output says"
            assert np.array_equal(hot_after[out[b, i]], pool[pool_of(r, t)]), "I1: bytes"
            if t in before_where:
                # I5
                assert before_where[t] == s, "I5: hit moved"
                hit_slots.add(s)
                n_hit += 1
            else:
                fill[i] = s
        # I11
        o = out[b][out[b] >= 0]
        assert len(np.unique(o)) == len(o), "I11: duplicate outputs"
        # I6
        changed = [s for s in range(H) if tokens_after[r, s] != tokens_before[r, s]]
        assert counts[b] == len(fill) == K - n_hit - n_new - n_bad, "I6: miss count"
        victims = set(fill.values())
        assert len(victims) == len(fill), "one victim slot per miss"
        # a victim never held a requested token, so every victim's token changes
        assert sorted(changed) == sorted(victims), "I6: changed slots != victims"
        # I7
        for s in range(S_r):
            if s not in victims:
                assert tokens_after[r, s] == tokens_before[r, s], "I7: non-victim token changed"
                assert np.array_equal(hot_after[row_of(r, s)], hot_before[row_of(r, s)]), \
                    "I7: non-victim bytes changed"
            else:
                changed_hot_rows.add(row_of(r, s))
        # I8
        old = lru_before[r].tolist()
        fills_in_miss_order = [fill[i] for i in sorted(fill)]
        stale = [s for s in old if s not in hit_slots and s not in victims]
        hits_old = [s for s in old if s in hit_slots]
        assert lru_after[r].tolist() == stale + fills_in_miss_order + hits_old, "I8: LRU order"
        # victims are the oldest non-hit slots
        evictable_old = [s for s in old if s not in hit_slots]
        assert fills_in_miss_order == evictable_old[:len(fills_in_miss_order)], "victim order"
    # untouched state rows and hot rows keep everything
    for r in range(R):
        if r not in touched_rows:
            assert np.array_equal(tokens_after[r], tokens_before[r])
            assert np.array_equal(lru_after[r], lru_before[r])
    mask = np.ones(hot_before.shape[0], dtype=bool)
    if changed_hot_rows:
        mask[list(changed_hot_rows)] = False
    assert np.array_equal(hot_after[mask], hot_before[mask]), "rows outside the victims changed"
