"""GPU parity of transfer_rows_all_layer, store_kv_scatter and
hisparse_state_reset against the CPU oracle, byte for byte."""

import numpy as np
import pytest
import torch

import oracle
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import sparse_attention_kv_hisparse_amd as hs
    hs.load()
    torch.cuda.set_device(0)


def _log(msg):
    print(msg, flush=True)


def _rand_dev(rows, rb, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randint(0, 256, (rows, rb), dtype=torch.uint8, device="cuda", generator=g)


def _layers(L, rows, rb, where, seed):
    """L layers as one backing tensor (device or pinned host) and their base pointers."""
    backing = _rand_dev(L * rows, rb, seed)
    if where == "host":
        host = torch.empty((L * rows, rb), dtype=torch.uint8, pin_memory=True)
        host.copy_(backing)
        backing = host
    layers = [backing[l * rows:(l + 1) * rows] for l in range(L)]
    ptrs = torch.tensor([t.data_ptr() for t in layers], dtype=torch.int64, device="cuda")
    return backing, layers, ptrs


def _np(t):
    return t.cpu().numpy() if t.is_cuda else t.numpy()


@pytest.mark.parametrize("host_link", [False, True], ids=["hbm_launch", "host_link_launch"])
@pytest.mark.parametrize("L,rows,rb,n,src_kind,dst_kind", [
    (1, 64, 656, 17, "device", "device"),
    (3, 500, 656, 300, "host", "device"),
    (5, 300, 656, 250, "device", "host"),
    (2, 200, 132, 150, "host", "device"),       # 4-byte path
    (7, 100, 4, 100, "device", "device"),
    (61, 300, 1152, 257, "device", "host"),
    (4, 40000, 656, 30000, "host", "device"),   # more items than one host-link launch round
])
def test_transfer_parity(L, rows, rb, n, src_kind, dst_kind, host_link):
    import sparse_attention_kv_hisparse_amd as hs
    rng = np.random.default_rng(L * 1000 + n)
    _, src_l, src_p = _layers(L, rows, rb, src_kind, 1 + L)
    _, dst_l, dst_p = _layers(L, rows, rb, dst_kind, 2 + L)
    si = rng.permutation(rows)[:n].astype(np.int64)
    di = rng.permutation(rows)[:n].astype(np.int64)
    si[::37] = rows + 3          # out-of-range pairs are skipped on both sides
    want_src = [_np(t).copy() for t in src_l]
    want_dst = [_np(t).copy() for t in dst_l]
    skipped = oracle.transfer_rows_all_layer(want_src, want_dst, si, di)
    hs.transfer_rows_all_layer(src_layer_ptrs=src_p, dst_layer_ptrs=dst_p,
                               src_idx=torch.as_tensor(si).cuda(), dst_idx=torch.as_tensor(di).cuda(),
                               row_bytes=rb, src_nrows=rows, dst_nrows=rows, host_link=host_link)
    torch.cuda.synchronize()
    assert skipped == len(si[::37])
    for l in range(L):
        assert np.array_equal(_np(dst_l[l]), want_dst[l]), f"layer {l}"
        assert np.array_equal(_np(src_l[l]), want_src[l]), f"source layer {l} changed"


@pytest.mark.parametrize("src_kind,dst_kind,want", [
    ("device", "device", False), ("host", "device", True), ("device", "host", True),
    ("host", "host", True)])
def test_transfer_host_link_from_memory_kind(src_kind, dst_kind, want):
    import sparse_attention_kv_hisparse_amd as hs
    _, src_l, _ = _layers(2, 8, 656, src_kind, 5)
    _, dst_l, _ = _layers(2, 8, 656, dst_kind, 6)
    assert hs.transfer_host_link(src_l[1], dst_l[0]) is want


def test_transfer_host_link_rejects_unknown_memory():
    import sparse_attention_kv_hisparse_amd as hs
    pageable = torch.zeros((8, 656), dtype=torch.uint8)      # plain host memory, not pinned
    dev = torch.zeros((8, 656), dtype=torch.uint8, device="cuda")
    with pytest.raises(hs.HisparseError, match="HS_EMEMKIND"):
        hs.transfer_host_link(pageable, dev)


@pytest.mark.parametrize("direction", ["offload", "load"])
def test_transfer_all_layer_full_size(direction):
    """61 layers x 262,144 rows x 656 B, 8192 pairs, one direction per case:
    offload = HBM -> pinned host, load = pinned host -> HBM. Every destination
    row named by a pair is checked on every layer; three whole layers are
    checked against the oracle."""
    import sparse_attention_kv_hisparse_amd as hs
    cfg = gen.ALL_LAYER
    L, rows, rb = cfg.layers, cfg.rows_per_layer, cfg.row_bytes
    src_kind, dst_kind = ("device", "host") if direction == "offload" else ("host", "device")
    _log(f"  all-layer {direction}: allocating 2 x {L * rows * rb / 1e9:.1f} GB")
    _, src_l, src_p = _layers(L, rows, rb, src_kind, 11)
    _, dst_l, dst_p = _layers(L, rows, rb, dst_kind, 12)
    si, di = gen.transfer_indices(cfg)
    sample = (0, L // 2, L - 1)
    before = {l: _np(dst_l[l]).copy() for l in sample}
    hs.transfer_rows_all_layer(src_layer_ptrs=src_p, dst_layer_ptrs=dst_p,
                               src_idx=torch.as_tensor(si).cuda(), dst_idx=torch.as_tensor(di).cuda(),
                               row_bytes=rb, src_nrows=rows, dst_nrows=rows, host_link=True)
    torch.cuda.synchronize()
    _log(f"  all-layer {direction}: copied, checking")
    sit, dit = torch.as_tensor(si), torch.as_tensor(di)
    for l in range(L):
        s = src_l[l][sit.to(src_l[l].device)]
        d = dst_l[l][dit.to(dst_l[l].device)]
        assert torch.equal(s.cpu(), d.cpu()), f"layer {l}: destination rows differ"
    for l in sample:
        want = before[l]
        oracle.transfer_rows_all_layer([_np(src_l[l])], [want], si, di)
        assert np.array_equal(_np(dst_l[l]), want), f"layer {l} differs from the oracle"


@pytest.mark.parametrize("n,rb,src_stride,dst_rows,aligned", [
    (1, 656, 656, 4, True), (100, 656, 1312, 300, True), (33, 132, 132, 50, True),
    (64, 64, 96, 70, False), (2000, 1152, 1152, 4100, True)])
def test_scatter_parity(n, rb, src_stride, dst_rows, aligned):
    import sparse_attention_kv_hisparse_amd as hs
    rng = np.random.default_rng(n)
    src_back = _rand_dev(n, src_stride, n)
    src = src_back[:, :rb]
    dst_back = torch.zeros((dst_rows * rb + 16,), dtype=torch.uint8, device="cuda")
    off = 0 if aligned else 4
    dst = dst_back[off:off + dst_rows * rb].view(dst_rows, rb)
    loc = rng.permutation(dst_rows)[:n].astype(np.int64)
    loc[::9] = -1
    loc[5::13] = dst_rows + 1
    want = _np(dst).copy()
    skipped = oracle.store_kv_scatter(np.ascontiguousarray(_np(src)), want, loc)
    hs.store_kv_scatter(src=src, dst=dst, loc=torch.as_tensor(loc).cuda())
    torch.cuda.synchronize()
    assert skipped == int(((loc < 0) | (loc >= dst_rows)).sum())
    assert np.array_equal(_np(dst), want)


def test_state_reset_parity():
    import sparse_attention_kv_hisparse_amd as hs
    R, H, S_r = 7, 300, 302
    st = torch.randint(-5, 100, (R, S_r), dtype=torch.int32, device="cuda")
    lru = torch.randint(-5, 100, (R, H), dtype=torch.int16, device="cuda")
    st_np, lru_np = _np(st).copy(), _np(lru).copy()
    rows = np.asarray([5, 0, 3, 9, -1], dtype=np.int64)
    oracle.state_reset(st_np, lru_np, rows[(rows >= 0) & (rows < R)])
    hs.hisparse_state_reset(slot_tokens=st, lru=lru, rows=torch.as_tensor(rows).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(_np(st), st_np) and np.array_equal(_np(lru), lru_np)
