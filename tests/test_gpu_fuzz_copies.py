"""Seeded random sweep of the row copies and the key invalidation against the
oracle, byte for byte: transfer_rows_all_layer and transfer_kv_all_layer
(1 to 300 layers, past the 256 staged in LDS; source and destination row
counts that differ; rows of 4 to 1152 bytes, many not a multiple of 16, so
that layer bases fall off 16-byte alignment; pinned-host and HBM sides in
both directions; either launch shape; pairs out of range on either side),
store_kv_scatter and store_kv_cache (row strides above the row size,
destinations misaligned to 4 bytes, skipped locations), and
hisparse_invalidate_written (rows outside [0, R), negative ids)."""

import os

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

N_CASES = int(os.environ.get("HS_FUZZ_COPY_CASES", 24))
RB_CHOICES = [4, 8, 12, 20, 64, 132, 656, 1024, 1152]
L_CHOICES = [1, 2, 3, 5, 8, 61, 130, 300]
CAP = 24 << 20      # bytes per side


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import sparse_attention_kv_hisparse_amd as hs
    hs.load()
    torch.cuda.set_device(0)


def _np(t):
    return t.cpu().numpy() if t.is_cuda else t.numpy()


def _rows_np(t):
    return np.ascontiguousarray(_np(t))


def _layers(rng, L, rows, rb, where):
    data = rng.integers(0, 256, (L * rows, rb), dtype=np.uint8)
    if where == "host":
        backing = torch.empty((L * rows, rb), dtype=torch.uint8, pin_memory=True)
        backing.copy_(torch.as_tensor(data))
    else:
        backing = torch.as_tensor(data).cuda()
    layers = [backing[l * rows:(l + 1) * rows] for l in range(L)]
    ptrs = torch.tensor([t.data_ptr() for t in layers], dtype=torch.int64, device="cuda")
    return layers, ptrs


def draw_transfer(i):
    rng = np.random.default_rng(12_000 + i)
    rb = int(rng.choice(RB_CHOICES))
    L = int(rng.choice(L_CHOICES))
    rows_cap = max(1, CAP // (L * rb * 2))
    src_rows = int(rng.integers(1, min(4000, rows_cap) + 1))
    dst_rows = int(rng.integers(1, min(4000, rows_cap) + 1))
    n = int(rng.integers(0, min(src_rows, dst_rows) + 5))
    return dict(i=i, rb=rb, L=L, src_rows=src_rows, dst_rows=dst_rows, n=n,
                src_kind=str(rng.choice(["host", "device"])), dst_kind=str(rng.choice(["host", "device"])),
                host_link=bool(rng.random() < 0.5), kv=bool(rng.random() < 0.4),
                seed=int(rng.integers(1, 2**31)))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_transfer_matches_oracle(i):
    import sparse_attention_kv_hisparse_amd as hs
    c = draw_transfer(i)
    print(f"  transfer case {c}", flush=True)
    rng = np.random.default_rng(c["seed"])
    L, rb, sr, dr, n = c["L"], c["rb"], c["src_rows"], c["dst_rows"], c["n"]
    si = rng.integers(-3, sr + 3, n).astype(np.int64)                # some out of range
    di = (rng.permutation(dr + 4)[:n] - 2).astype(np.int64)          # unique, some out of range
    ks, ksp = _layers(rng, L, sr, rb, c["src_kind"])
    kd, kdp = _layers(rng, L, dr, rb, c["dst_kind"])
    want_k = [_np(x).copy() for x in kd]
    idx = dict(src_idx=torch.as_tensor(si).cuda(), dst_idx=torch.as_tensor(di).cuda(), row_bytes=rb,
               src_nrows=sr, dst_nrows=dr, host_link=c["host_link"])
    if c["kv"]:
        vs, vsp = _layers(rng, L, sr, rb, c["src_kind"])
        vd, vdp = _layers(rng, L, dr, rb, c["dst_kind"])
        want_v = [_np(x).copy() for x in vd]
        skipped = oracle.transfer_kv_all_layer([_np(x) for x in ks], [_np(x) for x in vs], want_k, want_v,
                                               si, di)
        hs.transfer_kv_all_layer(k_src_layer_ptrs=ksp, v_src_layer_ptrs=vsp, k_dst_layer_ptrs=kdp,
                                 v_dst_layer_ptrs=vdp, **idx)
    else:
        skipped = oracle.transfer_rows_all_layer([_np(x) for x in ks], want_k, si, di)
        hs.transfer_rows_all_layer(src_layer_ptrs=ksp, dst_layer_ptrs=kdp, **idx)
    torch.cuda.synchronize()
    assert skipped == int(((si < 0) | (si >= sr) | (di < 0) | (di >= dr)).sum())
    for l in range(L):
        assert np.array_equal(_np(kd[l]), want_k[l]), f"layer {l}"
        if c["kv"]:
            assert np.array_equal(_np(vd[l]), want_v[l]), f"V layer {l}"


def draw_store(i):
    rng = np.random.default_rng(13_000 + i)
    rb = int(rng.choice(RB_CHOICES))
    n = int(rng.integers(0, 3000))
    return dict(i=i, rb=rb, n=n, dst_rows=int(rng.integers(1, 6000)),
                src_pad=4 * int(rng.integers(0, 9)), dst_pad=4 * int(rng.integers(0, 9)),
                misaligned=bool(rng.random() < 0.3), kv=bool(rng.random() < 0.5),
                seed=int(rng.integers(1, 2**31)))


def _rows(rng, n, rb, pad, misaligned):
    """n rows of rb bytes at a row stride of rb + pad, the first 4 bytes past a
    16-byte boundary when misaligned."""
    off = 4 if misaligned else 0
    stride = rb + pad
    back = torch.as_tensor(rng.integers(0, 256, n * stride + off + 16, dtype=np.uint8)).cuda()
    return back[off:off + n * stride].view(n, stride)[:, :rb]


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_store_matches_oracle(i):
    import sparse_attention_kv_hisparse_amd as hs
    c = draw_store(i)
    print(f"  store case {c}", flush=True)
    rng = np.random.default_rng(c["seed"])
    n, rb, dr = c["n"], c["rb"], c["dst_rows"]
    loc = np.full(n, -1, np.int64)               # distinct rows in range, then some skipped
    m = min(n, dr)
    loc[:m] = rng.permutation(dr)[:m]
    bad = rng.random(n) < 0.1
    loc[bad] = rng.choice([-2, -1, dr, dr + 1], int(bad.sum()))
    rng.shuffle(loc)
    k_src = _rows(rng, n, rb, c["src_pad"], False)
    k_dst = _rows(rng, dr, rb, c["dst_pad"], c["misaligned"])
    want_k = _np(k_dst).copy()
    if c["kv"]:
        v_src = _rows(rng, n, rb, c["dst_pad"], c["misaligned"])
        v_dst = _rows(rng, dr, rb, c["src_pad"], False)
        want_v = _np(v_dst).copy()
        skipped = 0 if n == 0 else oracle.store_kv_cache(_rows_np(k_src), _rows_np(v_src), want_k,
                                                         want_v, loc)
        hs.store_kv_cache(k_src=k_src, v_src=v_src, k_dst=k_dst, v_dst=v_dst, loc=torch.as_tensor(loc).cuda())
    else:
        skipped = 0 if n == 0 else oracle.store_kv_scatter(_rows_np(k_src), want_k, loc)
        hs.store_kv_scatter(src=k_src, dst=k_dst, loc=torch.as_tensor(loc).cuda())
    torch.cuda.synchronize()
    assert skipped == int(((loc < 0) | (loc >= dr)).sum())
    assert np.array_equal(_np(k_dst), want_k)
    if c["kv"]:
        assert np.array_equal(_np(v_dst), want_v)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_invalidation_matches_oracle(i):
    import sparse_attention_kv_hisparse_amd as hs
    rng = np.random.default_rng(14_000 + i)
    R, S_r, n = int(rng.integers(1, 40)), int(rng.integers(1, 9000)), int(rng.integers(0, 500))
    keys = rng.integers(-1, 3 * S_r, (R, S_r)).astype(np.int32)
    rows = rng.integers(-2, R + 2, n).astype(np.int64)
    written = np.where(rng.random(n) < 0.7, keys[rows % R, rng.integers(0, S_r, n)],
                       rng.integers(-3, 3 * S_r, n)).astype(np.int64)
    dev = torch.as_tensor(keys).cuda()
    want = keys.copy()
    oracle.invalidate_written(want, rows, written)
    hs.hisparse_invalidate_written(slot_keys=dev, rows=torch.as_tensor(rows).cuda(),
                                   written=torch.as_tensor(written).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(_np(dev), want)
