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
    """Returns event-timed µs over the K timed calls, miss counts per timed step, wall seconds."""
    from workloads import gen  # noqa: F401
    log(f"[bench] {cfg.name}: building pool ({cfg.pool_nrows} x {cfg.row_bytes} B, {cfg.pool_kind})")
    pool = wdev.make_pool(cfg)
    st = wdev.DeviceSwapState(cfg)
    tr = Trace(cfg, warmup + steps, torch)
    counts = torch.empty((warmup + steps, cfg.B), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def call(t):
        hs.hisparse_swap_in(topk=tr.topk[t], req_rows=tr.rows, seq_lens=tr.seq[t],
                            slot_tokens=st.slot_tokens, lru=st.lru, pool=pool, hot=st.hot,
                            out_rows=st.out, ctx_stride=cfg.ctx, workspace=st.ws,
                            miss_counts=counts[t], stream=stream)

    for t in range(warmup):
        call(t)
    torch.cuda.synchronize()
    log(f"[bench] {cfg.name}: {warmup} warm-up steps done, timing {steps}")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record(stream)
    for k in range(steps):
        call(warmup + k)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    us_total = e0.elapsed_time(e1) * 1000.0
    c = counts.cpu().numpy()[warmup:]
    del pool, st, tr
    torch.cuda.empty_cache()
    return us_total, c, wall


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
    cfg = gen.DSV32

    link = None if args.no_host_link else host_link_ceiling(torch, hs)
    if link:
        log(f"[bench] host link: {json.dumps({k: round(v, 2) for k, v in link.items()})}")

    us_total, counts, wall = run_gpu(cfg, args.warmup, args.steps, torch, hs, wdev)
    rows = int(counts.sum())
    bytes_link = rows * cfg.row_bytes
    total_s = us_total * 1e-6
    value = rows / wall
    achieved = bytes_link / total_s / 1e9
    peak = link["h2d_ceiling_gbs"] if link else None
    out = {
        "metric": "swapped-in rows/s + effective GB/s (% of HBM/host-link peak); µs per decode-step call",
        "value": round(value, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": "dsv32_decode_swap_in_pinned_host_pool", "batch": cfg.B,
                   "context": cfg.ctx, "hot_size": cfg.H, "top_k": cfg.K,
                   "row_bytes": cfg.row_bytes, "pool": "pinned_host", "retention": cfg.rho,
                   "new_ids": "zipf1.1_recency"},
        "us_per_call": round(us_total / args.steps, 2),
        "rows_per_call": round(rows / args.steps, 1),
        "effective_GBps": round(achieved, 2),
        "roofline": {"bound": "host_link", "kernel": "hisparse_swap_in call (resolve_kernel + swap_copy_kernel)",
                     "achieved": round(achieved, 2), "peak": round(peak, 2) if peak else None,
                     "unit": "GB/s", "frac": round(achieved / peak, 4) if peak else None,
                     "peak_published": PCIE5_X16_GBS, "traffic": None},
        "host_link": {k: round(v, 2) for k, v in link.items()} if link else None,
    }

    if not args.no_device_pool:
        dcfg = gen.DEVPOOL
        dus_total, dcounts, dwall = run_gpu(dcfg, 1, args.device_pool_steps, torch, hs, wdev)
        drows = int(dcounts.sum())
        # algorithmic HBM bytes: each row read once and written once, plus the
        # per-request metadata (top-k ids, LRU read+write, slot tokens gathered,
        # outputs written, new owners written)
        meta = dcfg.B * (4 * dcfg.K * 2 + 2 * dcfg.H * 2 + 4 * dcfg.H) + 4 * drows / args.device_pool_steps
        dbytes = 2 * drows * dcfg.row_bytes + meta * args.device_pool_steps
        dach = dbytes / (dus_total * 1e-6) / 1e9
        out["device_pool"] = {
            "workload": "device_pool_swap_in_hbm", "batch": dcfg.B, "context": dcfg.ctx,
            "hot_size": dcfg.H, "top_k": dcfg.K, "row_bytes": dcfg.row_bytes, "steps": args.device_pool_steps,
            "rows_per_s": round(drows / dwall, 1), "rows_per_call": round(drows / args.device_pool_steps, 1),
            "us_per_call": round(dus_total / args.device_pool_steps, 2),
            "roofline": {"bound": "hbm", "achieved": round(dach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(dach / HBM_PEAK_GBS, 4), "traffic": None},
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
