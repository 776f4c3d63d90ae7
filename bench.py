"""Benchmark of the HiSparse decode-step swap-in on one MI355X.

One "step" is one hisparse_swap_in call (resolve + row copy) over one batch of
synthetic top-k ids. Headline workload: DeepSeek-V3.2-like decode, B=32
requests, 32,768-token contexts in a pinned-host pool of 1,048,576 x 656-byte
rows, hot_size 4096, top_k 2048, Zipf(1.1) recency ids with 85% retention.
W warm-up steps (the first is the cold step) run untimed, then K steps are
timed; inputs for every step are resident in HBM before timing starts.

Also reported in the same JSON line:
  * device_pool: the same call on the device-pool workload (B=128, 16,384-token
    contexts, pool of 2,097,152 rows in HBM, 60% retention) against 8 TB/s;
  * host_link: the measured host-link ceiling the host-pool roofline uses;
  * cpu_baseline: the CPU oracle (single thread) on the headline steps.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PCIE5_X16_GBS = 64.0   # PCIe 5.0 x16, one direction, published link rate


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=63)
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--device-pool-steps", type=int, default=31)
    p.add_argument("--no-device-pool", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-host-link", action="store_true")
    p.add_argument("--calibrate", action="store_true",
                   help="only run a plain device-to-device stream copy of known size "
                        "(256 MiB read + 256 MiB written per launch, 3 launches) so HBM byte "
                        "counters can be scaled, then exit")
    return p.parse_args()


class Trace:
    """Pre-generated inputs of one workload, uploaded to HBM."""

    def __init__(self, cfg, steps, torch):
        from workloads import gen
        self.cfg = cfg
        self.steps = steps
        self.topk_np = np.stack(list(gen.topk_trace(cfg, steps)))
        self.seq_np = np.stack([gen.seq_lens(cfg, t) for t in range(steps)])
        self.topk = torch.as_tensor(self.topk_np).cuda()
        self.seq = torch.as_tensor(self.seq_np).cuda()
        self.rows = torch.arange(cfg.B, dtype=torch.int64, device="cuda")


def run_gpu(cfg, warmup, steps, torch, hs, wdev):
    """Time K swap-in calls after W warm-up calls.

    Pass 1 (the timed region of the contract): W untimed calls, then K plain
    hisparse_swap_in calls bracketed by two events and the wall clock.
    Pass 2: the state is reset and the same trace replayed with resolve-only
    calls (hisparse_resolve); the state after each call is identical because
    row copies never touch it, so the K timed resolves give the resolve kernel's
    time and the difference gives the copy kernel's.
    Returns dict(us_total, us_resolve, counts, wall).
    """
    log(f"[bench] {cfg.name}: building pool ({cfg.pool_nrows} x {cfg.row_bytes} B, {cfg.pool_kind})")
    pool = wdev.make_pool(cfg)
    st = wdev.DeviceSwapState(cfg)
    tr = Trace(cfg, warmup + steps, torch)
    counts = torch.empty((warmup + steps, cfg.B), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def call(t, fn):
        fn(topk=tr.topk[t], req_rows=tr.rows, seq_lens=tr.seq[t], slot_tokens=st.slot_tokens,
           lru=st.lru, pool=pool, hot=st.hot, out_rows=st.out, ctx_stride=cfg.ctx, workspace=st.ws,
           miss_counts=counts[t], stream=stream)

    def timed(fn):
        for t in range(warmup):
            call(t, fn)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record(stream)
        for k in range(steps):
            call(warmup + k, fn)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000.0, time.perf_counter() - w0

    us_total, wall = timed(hs.hisparse_swap_in)
    log(f"[bench] {cfg.name}: {steps} timed calls after {warmup} warm-up, {us_total / steps:.1f} us/call")
    c = counts.cpu().numpy()[warmup:].copy()
    hs.hisparse_state_reset(slot_tokens=st.slot_tokens, lru=st.lru,
                            rows=torch.arange(st.R, dtype=torch.int64, device="cuda"))
    us_resolve, _ = timed(hs.hisparse_resolve)
    c2 = counts.cpu().numpy()[warmup:]
    assert (c == c2).all(), "resolve-only replay diverged from the timed pass"
    del pool, st, tr
    torch.cuda.empty_cache()
    return dict(us_total=us_total, us_resolve=us_resolve, counts=c, wall=wall)


def kernel_sources_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ("swap_in.hip", "hs_common.hpp"):
        h.update(open(os.path.join(ROOT, "sparse_attention_kv_hisparse_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM/fabric bytes per copy-kernel launch from the committed rocprofv3
    counter summary, if it was taken on the kernel sources as they are now."""
    path = os.path.join(ROOT, "profiles", "swap_copy_traffic.json")
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    if d.get("kernel_sources_sha256_16") != kernel_sources_hash():
        return None
    w = d.get("workloads", {}).get(workload)
    return None if w is None else w.get("bytes_per_launch")


def host_link_ceiling(torch, hs):
    """Best-of-N host->device rate of (a) hipMemcpyAsync of 1 GiB pinned and
    (b) a zero-copy streaming kernel (the library's row transfer over 1 MiB
    sequential rows of pinned memory). Also device->host for reference."""
    n = 1 << 30
    host = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    host.numpy()[:] = 7
    dev = torch.empty(n, dtype=torch.uint8, device="cuda")
    res = {}
    s = torch.cuda.current_stream()

    def best(fn, reps=5):
        b = 0.0
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            fn()
            e1.record(s)
            torch.cuda.synchronize()
            b = max(b, n / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        return b

    res["memcpy_h2d_gbs"] = best(lambda: dev.copy_(host, non_blocking=True))
    res["memcpy_d2h_gbs"] = best(lambda: host.copy_(dev, non_blocking=True))
    rb = 1 << 20
    rows = n // rb
    idx = torch.arange(rows, dtype=torch.int64, device="cuda")
    hp = torch.tensor([host.data_ptr()], dtype=torch.int64, device="cuda")
    dp = torch.tensor([dev.data_ptr()], dtype=torch.int64, device="cuda")
    res["zero_copy_h2d_gbs"] = best(lambda: hs.transfer_rows_all_layer(
        src_layer_ptrs=hp, dst_layer_ptrs=dp, src_idx=idx, dst_idx=idx, row_bytes=rb,
        src_nrows=rows, dst_nrows=rows))
    res["zero_copy_d2h_gbs"] = best(lambda: hs.transfer_rows_all_layer(
        src_layer_ptrs=dp, dst_layer_ptrs=hp, src_idx=idx, dst_idx=idx, row_bytes=rb,
        src_nrows=rows, dst_nrows=rows))
    res["h2d_ceiling_gbs"] = max(res["memcpy_h2d_gbs"], res["zero_copy_h2d_gbs"])
    res["d2h_ceiling_gbs"] = max(res["memcpy_d2h_gbs"], res["zero_copy_d2h_gbs"])
    del host, dev
    torch.cuda.empty_cache()
    return res


def calibrate(torch, hs):
    """Three launches of the library's row transfer over contiguous 1 MiB rows:
    exactly 256 MiB read and 256 MiB written per launch, device to device."""
    n = 256 << 20
    rb = 1 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.zeros(n, dtype=torch.uint8, device="cuda")
    idx = torch.arange(n // rb, dtype=torch.int64, device="cuda")
    sp = torch.tensor([src.data_ptr()], dtype=torch.int64, device="cuda")
    dp = torch.tensor([dst.data_ptr()], dtype=torch.int64, device="cuda")
    for _ in range(3):
        hs.transfer_rows_all_layer(src_layer_ptrs=sp, dst_layer_ptrs=dp, src_idx=idx, dst_idx=idx,
                                   row_bytes=rb, src_nrows=n // rb, dst_nrows=n // rb)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "transfer_kernel<16>", "bytes_read_per_launch": n,
                      "bytes_written_per_launch": n, "launches": 3}), flush=True)


def cpu_baseline(cfg, warmup, steps):
    """The oracle, single-threaded, on the headline trace: steps before the timed
    window are replayed untimed to reach the same state, then the timed steps."""
    import oracle
    from workloads import gen
    pool = gen.fill_pool(cfg.seed, np.empty((cfg.pool_nrows, cfg.row_bytes), np.uint8))
    tok, lru = gen.initial_state(cfg)
    hot = np.zeros((cfg.R * cfg.S_r, cfg.row_bytes), np.uint8)
    rows = np.arange(cfg.B, dtype=np.int64)
    secs, rows_copied = 0.0, 0
    for t, topk in enumerate(gen.topk_trace(cfg, warmup + steps)):
        seq = gen.seq_lens(cfg, t)
        t0 = time.perf_counter()
        _, cnt = oracle.swap_in(topk=topk, req_rows=rows, seq_lens=seq, slot_tokens=tok, lru=lru,
                                pool=pool, hot=hot, ctx_stride=cfg.ctx)
        dt = time.perf_counter() - t0
        if t >= warmup:
            secs += dt
            rows_copied += int(cnt.sum())
    return rows_copied, secs


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); every GPU box here has "
              f"one GPU and this path has no multi-GPU leg.", file=sys.stderr)
        sys.exit(2)
    import torch
    import sparse_attention_kv_hisparse_amd as hs
    from workloads import device as wdev
    from workloads import gen
    hs.load()
    torch.cuda.set_device(0)
    if args.calibrate:
        calibrate(torch, hs)
        return
    cfg = gen.DSV32

    link = None if args.no_host_link else host_link_ceiling(torch, hs)
    if link:
        log(f"[bench] host link: {json.dumps({k: round(v, 2) for k, v in link.items()})}")

    r = run_gpu(cfg, args.warmup, args.steps, torch, hs, wdev)
    K = args.steps
    rows = int(r["counts"].sum())
    bytes_link = rows * cfg.row_bytes
    us_copy = max(r["us_total"] - r["us_resolve"], 1e-9)
    value = rows / r["wall"]
    achieved = bytes_link / (us_copy * 1e-6) / 1e9          # copy kernel alone
    call_gbs = bytes_link / (r["us_total"] * 1e-6) / 1e9     # whole call
    peak = link["h2d_ceiling_gbs"] if link else None
    out = {
        "metric": "swapped-in rows/s + effective GB/s (% of HBM/host-link peak); µs per decode-step call",
        "value": round(value, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(r["wall"] / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": "dsv32_decode_swap_in_pinned_host_pool", "batch": cfg.B,
                   "context": cfg.ctx, "hot_size": cfg.H, "top_k": cfg.K,
                   "row_bytes": cfg.row_bytes, "pool": "pinned_host", "retention": cfg.rho,
                   "new_ids": "zipf1.1_recency"},
        "us_per_call": round(r["us_total"] / K, 2),
        "us_resolve_kernel": round(r["us_resolve"] / K, 2),
        "us_copy_kernel": round(us_copy / K, 2),
        "rows_per_call": round(rows / K, 1),
        "effective_GBps_call": round(call_gbs, 2),
        "frac_host_link_call": round(call_gbs / peak, 4) if peak else None,
        "roofline": {"bound": "host_link", "kernel": "swap_copy_kernel<16>",
                     "achieved": round(achieved, 2), "peak": round(peak, 2) if peak else None,
                     "unit": "GB/s", "frac": round(achieved / peak, 4) if peak else None,
                     "peak_published": PCIE5_X16_GBS,
                     "traffic": measured_traffic("dsv32_decode")},
        "host_link": {k: round(v, 2) for k, v in link.items()} if link else None,
    }

    if not args.no_device_pool:
        dcfg = gen.DEVPOOL
        n = args.device_pool_steps
        d = run_gpu(dcfg, 1, n, torch, hs, wdev)
        drows = int(d["counts"].sum())
        d_copy = max(d["us_total"] - d["us_resolve"], 1e-9)
        # algorithmic HBM bytes of the copy kernel: each missed row read once and
        # written once, plus its (pool row, hot row) list entry (12 B)
        dbytes = drows * (2 * dcfg.row_bytes + 12)
        dach = dbytes / (d_copy * 1e-6) / 1e9
        # whole call: rows plus the resolve's own traffic (ids, LRU read and
        # write, slot tokens read, outputs, list) per request
        meta = dcfg.B * (4 * dcfg.K + 2 * dcfg.H * 2 + 4 * dcfg.H + 4 * dcfg.K) * n
        dcall = (drows * 2 * dcfg.row_bytes + meta) / (d["us_total"] * 1e-6) / 1e9
        out["device_pool"] = {
            "workload": "device_pool_swap_in_hbm", "batch": dcfg.B, "context": dcfg.ctx,
            "hot_size": dcfg.H, "top_k": dcfg.K, "row_bytes": dcfg.row_bytes, "steps": n,
            "rows_per_s": round(drows / d["wall"], 1), "rows_per_call": round(drows / n, 1),
            "us_per_call": round(d["us_total"] / n, 2),
            "us_resolve_kernel": round(d["us_resolve"] / n, 2),
            "us_copy_kernel": round(d_copy / n, 2),
            "effective_GBps_call": round(dcall, 1), "frac_hbm_call": round(dcall / HBM_PEAK_GBS, 4),
            "roofline": {"bound": "hbm", "kernel": "swap_copy_kernel<16>", "achieved": round(dach, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dach / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("device_pool")},
        }

    if not args.no_cpu_baseline:
        log("[bench] cpu baseline: oracle on the headline steps")
        crow, csec = cpu_baseline(cfg, args.warmup, args.steps)
        out["cpu_baseline"] = {"value": round(crow / csec, 1), "unit": "rows/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"the headline trace's {args.steps} timed steps "
                                         f"(B={cfg.B}, K={cfg.K}, H={cfg.H}), single thread, "
                                         f"host pool image in RAM; {csec:.2f} s"}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
